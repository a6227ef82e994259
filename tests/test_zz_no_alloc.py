"""The cache forward's no-allocation entry point (fa_fwd_kvcache_noalloc) against the
workspace entry point (fa_fwd_kvcache) through the C ABI.

Both run the same kernels with the same key split, so their outputs must be identical bit
for bit; each is also held to the oracle's bars (tests/parity.py). Two calls in a row, the
second on a smaller input, show that the static scratch needs no clearing between calls
(every slot a call reads is written by that call first).
"""
import sys

import pytest
import torch

import oracle
from exact_tiled_attention_32_amd import workloads
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [  # (B, H, Nq, Nk, d, causal, kv_len): the second is smaller than the first
    (4, 8, 16, 4096, 128, True, [4096, 3000, 17, 0]),
    (2, 3, 1, 700, 64, False, [700, 5]),
]


def test_noalloc_matches_workspace_call(gpu_lib):
    fa = gpu_lib
    for i, (B, H, Nq, Nk, d, causal, kv) in enumerate(CASES):
        print(f"[no-alloc] call {i}: B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal}", flush=True)
        sys.stdout.flush()
        assert fa.fa_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d) <= fa.NOALLOC_SCRATCH_BYTES
        case = workloads.make_decode_case(B, H, Nq, Nk, d, seed=300 + i, causal=causal, kv_len=kv)
        q, k, v = (case[n].to(DEV) for n in ("q", "k", "v"))
        kl = case["kv_len"].to(DEV)
        o_ws, lse_ws = fa.fa_fwd_kvcache(q, k, v, case["scale"], causal, kl)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
        fa.fa_fwd_kvcache_noalloc(q, k, v, case["scale"], o, lse, causal, kl)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ws), f"call {i}: O differs from the workspace call"
        assert torch.equal(lse, lse_ws), f"call {i}: lse differs from the workspace call"
        ref_o, ref_lse = oracle.kvcache_forward(case["q"], case["k"], case["v"], case["scale"], causal=causal,
                                                kv_len=kv)
        parity.check_o(o.cpu(), ref_o, "bf16", f"no-alloc call {i} O")
        parity.check_lse(lse.cpu(), ref_lse, f"no-alloc call {i} lse")


def test_noalloc_rejects_beyond_scratch(gpu_lib):
    """A request whose partial results exceed the static scratch fails before any launch."""
    fa = gpu_lib
    B, H, Nq, Nk, d = 64, 64, 32, 32, 128
    assert fa.fa_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d) > fa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
    with pytest.raises(fa.FAError) as ei:
        fa.fa_fwd_kvcache_noalloc(q, k, k, 0.1, o, lse)
    assert ei.value.status == fa.FA_ERR_UNSUPPORTED
