"""The measurement hook fa_time_next_call through the C ABI: the next call records the
caller's events around each of its kernels, in launch order, and the request is then
forgotten. The bench's per-kernel figures (and the roofline) rest on it."""
import sys

import numpy as np
import pytest
import torch

from exact_tiled_attention_32_amd import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:  # recorded once, so that the HIP events exist
        e.record()
    torch.cuda.synchronize()
    return evs


def _spans(evs):
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(len(evs) - 1)]


def _bwd_inputs(fa, case, mask):
    q, k, v, do = (case[n].to(DEV) for n in ("q", "k", "v", "do"))
    if mask is None:
        o, lse = fa.fa_fwd(q, k, v, case["scale"], case["causal"])
    else:
        o, lse = fa.fa_fwd_blocksparse(q, k, v, case["scale"], mask, mask_block=128)
    return q, k, v, o, do, lse


@pytest.mark.parametrize("sparse", [False, True])
def test_backward_kernels_bracketed_in_order(gpu_lib, sparse):
    fa = gpu_lib
    print(f"[hook] backward sparse={sparse}", flush=True)
    sys.stdout.flush()
    case = workloads.make_case(1, 2, 1024, 64, seed=91, causal=not sparse)
    mask = None
    if sparse:
        m = np.ones((8, 8), dtype=np.uint8)
        m[0, 5] = 0
        mask = torch.from_numpy(m).to(DEV)
    q, k, v, o, do, lse = _bwd_inputs(fa, case, mask)
    nk = 3 if sparse else 2  # [order,] dQ, dK/dV
    # a first call loads the kernels, so that the timed call brackets their runs alone
    fa.fa_bwd(q, k, v, o, do, lse, case["scale"], not sparse, block_mask=mask, mask_block=128)
    evs = _events(nk + 1)
    fa.fa_time_next_call(evs)
    fa.fa_bwd(q, k, v, o, do, lse, case["scale"], not sparse, block_mask=mask, mask_block=128)
    torch.cuda.synchronize()
    spans = _spans(evs)
    assert all(s > 0 for s in spans), spans
    # each kernel of this small call takes well under a millisecond once loaded
    assert all(s < 5.0 for s in spans), spans
    # the request is forgotten: a second call leaves the events where they were
    first = _spans(evs)
    fa.fa_bwd(q, k, v, o, do, lse, case["scale"], not sparse, block_mask=mask, mask_block=128)
    torch.cuda.synchronize()
    assert _spans(evs) == first


def test_cache_forward_split_and_merge(gpu_lib):
    fa = gpu_lib
    print("[hook] cache forward", flush=True)
    case = workloads.make_decode_case(4, 8, 2, 8000, 128, seed=92, causal=True, kv_len=[8000, 100, 0, 4000])
    q, k, v = (case[n].to(DEV) for n in ("q", "k", "v"))
    kv = case["kv_len"].to(DEV)
    fa.fa_fwd_kvcache(q, k, v, case["scale"], True, kv)
    evs = _events(3)
    fa.fa_time_next_call(evs)
    fa.fa_fwd_kvcache(q, k, v, case["scale"], True, kv)
    torch.cuda.synchronize()
    split, merge = _spans(evs)
    assert split > 0 and merge > 0


def test_cleared_request_records_nothing(gpu_lib):
    fa = gpu_lib
    case = workloads.make_case(1, 1, 256, 64, seed=93)
    q, k, v = (case[n].to(DEV) for n in ("q", "k", "v"))
    evs = _events(2)
    before = _spans(evs)
    fa.fa_time_next_call(evs)
    fa.fa_time_next_call(None)
    fa.fa_fwd(q, k, v, case["scale"], False)
    torch.cuda.synchronize()
    assert _spans(evs) == before
