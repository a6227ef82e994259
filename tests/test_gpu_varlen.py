"""Parity of the packed variable-length path (with sliding windows) against the fp64 oracle.

Bars (tests/parity.py): bf16 O within 1e-2 after discounting its own rounding, lse within
1e-3, dQ/dK/dV relative L2 within 2e-2 (absolute 1e-4 where the exact value is zero).
The sweep packs sequences of ragged lengths (0, 1, one tile, several tiles with a ragged
tail) and runs full, causal and windowed masks, comparing every element; the long
windowed workload is compared on sampled heads, rows and keys.
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from exact_tiled_attention_32_amd import workloads
from tests import parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_varlen(fa, case, backward=True):
    q, k, v = (case[n].to(DEV) for n in ("q", "k", "v"))
    cu = case["cu_seqlens"].to(DEV)
    kw = dict(causal=case["causal"], window_left=case["window_left"], window_right=case["window_right"])
    o, lse = fa.fa_fwd_varlen(q, k, v, cu, case["max_seqlen"], case["scale"], **kw)
    out = {"o": o, "lse": lse}
    if backward:
        do = case["do"].to(DEV)
        out["dq"], out["dk"], out["dv"] = fa.fa_bwd_varlen(q, k, v, o, do, lse, cu, case["max_seqlen"],
                                                           case["scale"], **kw)
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in out.items()}


def oracle_kw(case):
    return dict(causal=case["causal"], window_left=case["window_left"], window_right=case["window_right"])


def check_grads(got, ref_grads, label):
    for name, ref in zip(("dq", "dk", "dv"), ref_grads):
        if np.linalg.norm(ref) == 0:
            m = float(got[name].abs().max())
            assert m <= parity.ZERO_REF_ABS, f"{label} {name}: {m:.2e} where the exact value is 0"
        else:
            parity.check_grad(got[name], ref, f"{label} {name}")


def full_check(fa, case, label):
    note(f"[varlen] {label}")
    got = gpu_varlen(fa, case)
    cu = case["cu_seqlens"].tolist()
    ref_o, ref_lse = oracle.varlen_forward(case["q"], case["k"], case["v"], cu, case["scale"], **oracle_kw(case))
    parity.check_o(got["o"], ref_o, "bf16", f"{label} O")
    parity.check_lse(got["lse"], ref_lse, f"{label} lse")
    grads = oracle.varlen_backward(case["q"], case["k"], case["v"], case["do"], cu, case["scale"],
                                   **oracle_kw(case))
    check_grads(got, grads, label)


MODES = [  # (name, causal, window_left, window_right)
    ("full", False, -1, -1),
    ("causal", True, -1, -1),
    ("causal_w37", True, 37, -1),
    ("win_100_50", False, 100, 50),
    ("win_0_0", False, 0, 0),
    ("causal_w500", True, 500, -1),
    ("right_only_20", False, -1, 20),
]
LENGTHS = [[1, 0, 130, 257, 64], [300], [129, 128, 127]]
SWEEP = [(f"d{d}_{m[0]}_L{i}", d, m, L) for d in (16, 32, 64, 128) for m in MODES for i, L in enumerate(LENGTHS)]


@pytest.mark.parametrize("name,d,mode,lengths", SWEEP, ids=[c[0] for c in SWEEP])
def test_sweep(gpu_lib, name, d, mode, lengths):
    _, causal, wl, wr = mode
    case = workloads.make_varlen_case(lengths, 2, d, seed=zlib.crc32(name.encode()) % 10007, causal=causal,
                                      window_left=wl, window_right=wr)
    full_check(gpu_lib, case, name)


def test_max_seqlen_above_longest(gpu_lib):
    # a larger max_seqlen than needed only adds workgroups that find no rows
    case = workloads.make_varlen_case([200, 70], 3, 64, seed=5, causal=True, window_left=90)
    case["max_seqlen"] = 700
    full_check(gpu_lib, case, "max_seqlen_700")


INT_MAX = 2**31 - 1


@pytest.mark.parametrize("causal", [False, True])
def test_window_extent_int_max(gpu_lib, causal):
    """Window extents of 2^31 - 1 (far beyond any sequence) are the same as unbounded: the
    result must match the oracle without a window, with no overflow in the tile ranges."""
    lengths = [1, 130, 257]
    case = workloads.make_varlen_case(lengths, 2, 64, seed=31 + causal, causal=causal,
                                      window_left=INT_MAX, window_right=INT_MAX)
    note(f"[varlen] window INT_MAX causal={causal}")
    got = gpu_varlen(gpu_lib, case)
    cu = case["cu_seqlens"].tolist()
    ref_o, ref_lse = oracle.varlen_forward(case["q"], case["k"], case["v"], cu, case["scale"], causal=causal)
    parity.check_o(got["o"], ref_o, "bf16", "INT_MAX window O")
    parity.check_lse(got["lse"], ref_lse, "INT_MAX window lse")
    grads = oracle.varlen_backward(case["q"], case["k"], case["v"], case["do"], cu, case["scale"], causal=causal)
    check_grads(got, grads, "INT_MAX window")
    # and bitwise the same as the call with unbounded extents
    unb = dict(case, window_left=-1, window_right=-1)
    ref = gpu_varlen(gpu_lib, unb)
    for n in got:
        assert torch.equal(got[n], ref[n]), n


def test_no_tokens(gpu_lib):
    fa = gpu_lib
    q = torch.zeros((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    cu = torch.zeros(3, dtype=torch.int32, device=DEV)
    o, lse = fa.fa_fwd_varlen(q, q, q, cu, 0, 0.125, causal=True)
    assert o.shape == (0, 2, 64) and lse.shape == (2, 0)


def test_matches_dense_path(gpu_lib):
    # equal lengths without a window: the packed result equals the dense call on the
    # transposed layout, bit for bit (same kernels, same arithmetic order)
    fa = gpu_lib
    B, H, N, d = 3, 2, 300, 128
    case = workloads.make_varlen_case([N] * B, H, d, seed=9, causal=True)
    got = gpu_varlen(fa, case)
    dense = lambda x: x.view(B, N, H, d).transpose(1, 2).contiguous().to(DEV)
    q, k, v, do = (dense(case[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.fa_fwd(q, k, v, case["scale"], causal=True)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, case["scale"], causal=True)
    back = lambda x: x.transpose(1, 2).reshape(B * N, H, d).cpu()
    assert torch.equal(got["o"], back(o))
    assert torch.equal(got["lse"], lse.permute(1, 0, 2).reshape(H, B * N).cpu())
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(got[name], back(t)), name


def test_deterministic(gpu_lib):
    case = workloads.make_varlen_case([700, 33, 1000], 2, 64, seed=12, causal=True, window_left=200)
    a = gpu_varlen(gpu_lib, case)
    b = gpu_varlen(gpu_lib, case)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_workload_packed_full(gpu_lib):
    w = workloads.VARLEN_WORKLOADS["varlen_packed_causal"]
    case = workloads.generate_varlen(w)
    note(f"[varlen] {w.name}: {case['cu_seqlens'].numel() - 1} sequences, {case['q'].shape[0]} tokens")
    got = gpu_varlen(gpu_lib, case)
    cu = case["cu_seqlens"].tolist()
    ref_o, ref_lse = oracle.varlen_forward(case["q"], case["k"], case["v"], cu, case["scale"], **oracle_kw(case))
    parity.check_o(got["o"], ref_o, "bf16", "packed O")
    parity.check_lse(got["lse"], ref_lse, "packed lse")
    # gradients of two whole sequences (every head), compared element by element
    for s in (0, len(cu) - 2):
        c0, c1 = cu[s], cu[s + 1]
        g = oracle.varlen_backward(*(case[n][c0:c1] for n in ("q", "k", "v", "do")), [0, c1 - c0],
                                   case["scale"], **oracle_kw(case))
        check_grads({n: got[n][c0:c1] for n in ("dq", "dk", "dv")}, g, f"packed seq {s}")


def test_workload_sliding_window_sampled(gpu_lib):
    w = workloads.VARLEN_WORKLOADS["sliding_window_16k"]
    case = workloads.generate_varlen(w)
    got = gpu_varlen(gpu_lib, case)
    N, H, d = case["q"].shape
    wl = case["window_left"]
    rng = np.random.default_rng(3)
    to_dense = lambda x, h: x[:, h].unsqueeze(0).unsqueeze(0)   # [1, 1, N, d]
    for h in (0, H - 1):
        # rows near the start (window not yet full), across the middle and at the end
        rows = np.unique(np.r_[0:40, rng.integers(0, N, 60), N - 40:N])
        q1, k1, v1, do1 = (to_dense(case[n], h) for n in ("q", "k", "v", "do"))
        note(f"[varlen] sliding window head {h}: {rows.size} rows")
        allow = oracle.allowed_pairs(rows, N, causal=True, kv_len_b=None, block_mask=None, mask_block=128,
                                     window_left=wl)
        ref_o, ref_lse = oracle.forward_rows(parity.to64(q1[0, 0])[rows], parity.to64(k1[0, 0]),
                                             parity.to64(v1[0, 0]), case["scale"], allow)
        parity.check_o(got["o"][rows, h], ref_o, "bf16", f"window h{h} O")
        parity.check_lse(got["lse"][h, rows], ref_lse, f"window h{h} lse")
        # dK, dV of a block of 64 keys are exact from the rows that may see them: [j0, j0 + 63 + wl]
        j0 = int(rng.integers(N // 4, N // 2))
        krows = np.arange(j0, min(N, j0 + 64 + wl))
        dq, dk, dv = oracle.attention_backward(q1, k1, v1, do1, case["scale"], causal=True, window_left=wl,
                                               rows=krows)
        keys = np.arange(j0, j0 + 64)
        parity.check_grad(got["dk"][keys, h], dk[0, 0, keys], f"window h{h} dK")
        parity.check_grad(got["dv"][keys, h], dv[0, 0, keys], f"window h{h} dV")
        parity.check_grad(got["dq"][krows, h], dq[0, 0, krows], f"window h{h} dQ")
