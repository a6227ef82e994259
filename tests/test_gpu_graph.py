"""HIP-graph capture of a forward + backward call pair, and of the cache forward (with a
workspace and through the entry point that allocates nothing).

The library keeps no per-call state, allocates nothing and issues no memset, so a caller
can capture its calls into a graph (torch.cuda.CUDAGraph records them on its capture
stream) and replay them. Each replay is checked bitwise against the eager result (the
kernels are deterministic: no atomics), with eager work between replays: the outputs are
overwritten with NaN before every replay, and an eager call runs after it.
"""
import sys

import pytest
import torch

from exact_tiled_attention_32_amd import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("o", "lse", "dq", "dk", "dv")


def _setup(fa, name):
    w = workloads.WORKLOADS[name]
    x = workloads.generate(w)
    q, k, v, do = (x[n].to(DEV) for n in ("q", "k", "v", "do"))
    kv = None if x["kv_len"] is None else x["kv_len"].to(DEV)
    out = {
        "o": torch.empty_like(q),
        "lse": torch.empty(q.shape[:3], dtype=torch.float32, device=DEV),
        "dq": torch.empty_like(q), "dk": torch.empty_like(q), "dv": torch.empty_like(q),
    }
    ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=DEV)

    def step():
        fa.fa_fwd(q, k, v, x["scale"], w.causal, kv, o=out["o"], lse=out["lse"])
        fa.fa_bwd(q, k, v, out["o"], do, out["lse"], x["scale"], w.causal, kv,
                  dq=out["dq"], dk=out["dk"], dv=out["dv"], workspace=ws)
    return step, out


@pytest.mark.parametrize("name", ["bert_padded", "gpt2_causal"])
def test_graph_replay_matches_eager(gpu_lib, name):
    print(f"[graph] {name}", flush=True)
    sys.stdout.flush()
    step, out = _setup(gpu_lib, name)
    step()
    torch.cuda.synchronize()
    ref = {n: out[n].clone() for n in NAMES}
    # warm-up on a side stream before capture, as torch's graph API asks
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for n in NAMES:
            out[n].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in NAMES:
            assert torch.equal(out[n], ref[n]), f"{name}: replay {rep} {n} differs from the eager result"
        step()  # eager work between replays
        torch.cuda.synchronize()
        for n in NAMES:
            assert torch.equal(out[n], ref[n]), f"{name}: eager call after replay {rep}: {n} differs"


@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_replay_cache_forward(gpu_lib, noalloc):
    # the cache forward captured as a graph: with a caller workspace, and through the entry
    # point that allocates nothing (its partial results in the library's static array)
    fa = gpu_lib
    print(f"[graph] cache forward noalloc={noalloc}", flush=True)
    sys.stdout.flush()
    case = workloads.make_decode_case(4, 8, 5, 3000, 128, seed=61, causal=True, kv_len=[3000, 17, 0, 2048])
    q, k, v = (case[n].to(DEV) for n in ("q", "k", "v"))
    kv = case["kv_len"].to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    ws = torch.empty(fa.fa_fwd_kvcache_workspace_bytes(4, 8, 5, 3000, 128), dtype=torch.uint8, device=DEV)

    def call():
        if noalloc:
            fa.fa_fwd_kvcache_noalloc(q, k, v, case["scale"], o, lse, True, kv)
        else:
            fa.fa_fwd_kvcache(q, k, v, case["scale"], True, kv, o=o, lse=lse, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref_o, ref_l = o.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"replay {rep} differs from the eager result"
        call()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"eager call after replay {rep} differs"
