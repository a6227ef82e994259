"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the same seeded inputs.

Bars: tests/parity.py. The sweep covers ragged and tiny shapes (N = 1 .. 300 across
several tiles and a ragged tail) in every mask mode; the named workloads run at their
full sizes, compared in full where the oracle finishes in seconds and on sampled rows /
keys otherwise (a sampled key's dK, dV is exact when every row that may attend to it is
included).
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


def gpu_run(fa, case, backward=True, sparse=None):
    """Run the HIP forward (and backward) on a case dict of CPU tensors; return CPU results."""
    q, k, v = (case[n].to(DEV) for n in ("q", "k", "v"))
    kv = None if case["kv_len"] is None else case["kv_len"].to(DEV)
    bm = case["block_mask"]
    use_sparse = (bm is not None) if sparse is None else sparse
    mb = case["mask_block"]
    if use_sparse:
        o, lse = fa.fa_fwd_blocksparse(q, k, v, case["scale"], bm.to(DEV), mb, case["causal"], kv)
    else:
        o, lse = fa.fa_fwd(q, k, v, case["scale"], case["causal"], kv)
    out = {"o": o, "lse": lse}
    if backward:
        do = case["do"].to(DEV)
        dq, dk, dv = fa.fa_bwd(q, k, v, o, do, lse, case["scale"], case["causal"], kv,
                               bm.to(DEV) if use_sparse else None, mb)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in out.items()}


def oracle_args(case):
    kv = None if case["kv_len"] is None else case["kv_len"].tolist()
    bm = None if case["block_mask"] is None else case["block_mask"].numpy()
    return dict(causal=case["causal"], kv_len=kv, block_mask=bm, mask_block=case["mask_block"])


def full_check(fa, case, dtype, backward=True, label="", sparse=None):
    note(f"[parity] {label}")
    got = gpu_run(fa, case, backward=backward, sparse=sparse)
    ref_o, ref_lse = oracle.attention_forward(case["q"], case["k"], case["v"], case["scale"], **oracle_args(case))
    raw = parity.check_o(got["o"], ref_o, dtype, f"{label} O")
    lse_err = parity.check_lse(got["lse"], ref_lse, f"{label} lse")
    note(f"[parity] {label}: O max-abs {raw:.3e}, lse max-abs {lse_err:.3e}")
    if backward:
        grads = oracle.attention_backward(case["q"], case["k"], case["v"], case["do"], case["scale"],
                                          **oracle_args(case))
        for name, ref in zip(("dq", "dk", "dv"), grads):
            if np.linalg.norm(ref) == 0:
                # zero by cancellation (e.g. a row with a single allowed key): rounding level
                m = float(got[name].abs().max())
                assert m <= parity.ZERO_REF_ABS, f"{label} {name}: {m:.2e} where the exact value is 0"
            else:
                parity.check_grad(got[name], ref, f"{label} {name}")
    return got


# ------------------------------------------------------------------------------------------
# sweep of small and ragged shapes
# ------------------------------------------------------------------------------------------
SWEEP_N = [1, 17, 64, 127, 128, 129, 200, 300, 520]


def _sweep_cases():
    cases = []
    for d in (16, 32, 64, 128):
        for N in SWEEP_N:
            cases.append((f"dense-N{N}-d{d}", dict(B=2, H=3, N=N, d=d)))
            cases.append((f"causal-N{N}-d{d}", dict(B=2, H=3, N=N, d=d, causal=True)))
            kv = [N, max(N // 2, 1), 1, 0] if N > 1 else [1, 0, 5, 1]
            cases.append((f"padded-N{N}-d{d}", dict(B=4, H=2, N=N, d=d, kv_len=kv)))
            cases.append((f"causal-padded-N{N}-d{d}", dict(B=4, H=2, N=N, d=d, causal=True, kv_len=kv)))
    return cases


SWEEP = _sweep_cases()


@pytest.mark.parametrize("name,params", SWEEP, ids=[c[0] for c in SWEEP])
def test_sweep_bf16(gpu_lib, name, params):
    p = dict(params)
    B, H, N, d = p.pop("B"), p.pop("H"), p.pop("N"), p.pop("d")
    case = workloads.make_case(B, H, N, d, seed=zlib.crc32(name.encode()) % 10000, **p)
    full_check(gpu_lib, case, "bf16", label=name)


def _random_dense(n=24, seed=4242):
    # fixed-seed random shapes for the dense path: head dimension, batch, heads, length,
    # mask mode and ragged key lengths (zeros included) drawn together
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([16, 32, 64, 128, 64, 64]))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 1300))
        causal = bool(rng.random() < 0.5)
        kv = None if rng.random() < 0.5 else [int(x) for x in rng.integers(0, N + 1, size=B)]
        out.append((f"rand{i}_d{d}_B{B}H{H}_N{N}_{'causal' if causal else 'full'}{'' if kv is None else '_padded'}",
                    dict(B=B, H=H, N=N, d=d, causal=causal, kv_len=kv)))
    return out


RANDOM_DENSE = _random_dense()


@pytest.mark.parametrize("name,params", RANDOM_DENSE, ids=[c[0] for c in RANDOM_DENSE])
def test_random_dense_shapes(gpu_lib, name, params):
    p = dict(params)
    B, H, N, d = p.pop("B"), p.pop("H"), p.pop("N"), p.pop("d")
    case = workloads.make_case(B, H, N, d, seed=zlib.crc32(name.encode()) % 10000, **p)
    full_check(gpu_lib, case, "bf16", label=name)


# The dense bf16 forward without dropout stages three K/V tiles deep up to N = 4096 at
# d <= 64 and two deep beyond (and at d = 128), and the dense d = 64 dK/dV kernel takes one
# query block per step (three workgroups per CU) up to N = 4096 and two beyond: both sides
# of those switches, with ragged ends.
STAGE_SWITCH = [
    ("stages-N4096-d64-causal", 4096, 64, True, None),
    ("stages-N4097-d64-causal", 4097, 64, True, None),
    ("stages-N4096-d64-padded", 4096, 64, False, [2501]),
    ("stages-N4097-d64-padded", 4097, 64, False, [4097]),
    ("stages-N4096-d32-padded", 4096, 32, False, [3001]),
    ("stages-N4097-d32-padded", 4097, 32, False, [4097]),
    ("stages-N4096-d16-causal", 4096, 16, True, None),
]


@pytest.mark.parametrize("name,N,d,causal,kv", STAGE_SWITCH, ids=[c[0] for c in STAGE_SWITCH])
def test_stage_depth_switch(gpu_lib, name, N, d, causal, kv):
    case = workloads.make_case(1, 2, N, d, seed=zlib.crc32(name.encode()) % 10000, causal=causal, kv_len=kv)
    full_check(gpu_lib, case, "bf16", label=name)


def _synthetic_mask(nb, seed):
    rng = np.random.default_rng(seed)
    m = (rng.random((nb, nb)) < 0.5).astype(np.uint8)
    np.fill_diagonal(m, 1)
    if nb >= 3:
        m[:, nb - 2] = 0  # a key block no query block keeps
        m[1, :] = 0       # a query block with no kept key block
    return m


SPARSE = [
    ("sparse-N129-d64", 129, 64, False, None),
    ("sparse-N300-d128", 300, 128, False, None),
    ("sparse-N640-d64", 640, 64, False, None),
    ("sparse-N640-d128-causal", 640, 128, True, None),
    ("sparse-N700-d64-padded", 700, 64, False, [700, 333]),
    ("sparse-N896-d64-mb256", 896, 64, False, None),
    ("sparse-N640-d32-causal", 640, 32, True, None),
    ("sparse-N384-d16-padded", 384, 16, False, [384, 200]),
]


@pytest.mark.parametrize("name,N,d,causal,kv", SPARSE, ids=[c[0] for c in SPARSE])
def test_sweep_blocksparse(gpu_lib, name, N, d, causal, kv):
    mb = 256 if "mb256" in name else 128
    nb = -(-N // mb)
    B = 1 if kv is None else len(kv)
    case = workloads.make_case(B, 2, N, d, seed=zlib.crc32(name.encode()) % 10000, causal=causal, kv_len=kv,
                               block_mask=_synthetic_mask(nb, nb), mask_block=mb)
    full_check(gpu_lib, case, "bf16", label=name)


def test_sparse_rule_medium_heavy_columns(gpu_lib):
    """The 64K workload's mask rule at N = 4096: heavy columns (j % 16 == 0) kept by every row."""
    N = 4096
    case = workloads.make_case(1, 2, N, 64, seed=77, block_mask=workloads.sparse_block_rule(N // 128).numpy(),
                               mask_block=128)
    full_check(gpu_lib, case, "bf16", label="sparse-rule-N4096")


@pytest.mark.parametrize("d", [16, 128])
def test_blocksparse_largest_n(gpu_lib, d):
    """Block-sparse forward and backward at the largest N the backward's tile lists take
    (131072: 4096 query steps of 32 rows, 1024 key tiles in the order table), banded mask
    |i - j| <= 1. A key block's dK, dV depend only on the query blocks next to it, so sampled
    blocks (first, second, middle, last) are compared with the oracle exactly."""
    N, mb = 131072, 128
    nb = N // mb
    i = np.arange(nb)
    mask = (np.abs(i[:, None] - i[None, :]) <= 1).astype(np.uint8)
    case = workloads.make_case(1, 1, N, d, seed=41 + d, block_mask=mask, mask_block=mb)
    note(f"[parity] sparse largest N={N} d={d}")
    got = gpu_run(gpu_lib, case)
    q64, k64, v64 = (parity.to64(case[n])[0, 0] for n in ("q", "k", "v"))
    for r in (0, 1, nb // 2, nb - 1):
        rows = np.arange(r * mb, (r + 1) * mb)
        allow = oracle.allowed_pairs(rows, N, causal=False, kv_len_b=None, block_mask=mask, mask_block=mb)
        ref_o, ref_lse = oracle.forward_rows(q64[rows], k64, v64, case["scale"], allow)
        parity.check_o(got["o"][0, 0, rows], ref_o, "bf16", f"block {r} O")
        parity.check_lse(got["lse"][0, 0, rows], ref_lse, f"block {r} lse")
        near = np.arange(max(r - 1, 0) * mb, min(r + 2, nb) * mb)  # query blocks that see key block r
        dq, dk, dv = oracle.attention_backward(case["q"], case["k"], case["v"], case["do"], case["scale"],
                                               block_mask=mask, mask_block=mb, rows=near)
        parity.check_grad(got["dk"][0, 0, rows], dk[0, 0, rows], f"block {r} dK")
        parity.check_grad(got["dv"][0, 0, rows], dv[0, 0, rows], f"block {r} dV")
        parity.check_grad(got["dq"][0, 0, near], dq[0, 0, near], f"blocks near {r} dQ")


@pytest.mark.parametrize("N,d", [(1, 64), (77, 64), (128, 64), (300, 128), (129, 128), (77, 32), (300, 32)])
def test_sweep_f32_forward(gpu_lib, N, d):
    case = workloads.make_case(2, 2, N, d, dtype="f32", seed=N + d, causal=(N % 2 == 1))
    full_check(gpu_lib, case, "f32", backward=False, label=f"f32-N{N}-d{d}")
    case = workloads.make_case(2, 1, N, d, dtype="f32", seed=N + d + 1, kv_len=[max(N - 3, 0), 1])
    full_check(gpu_lib, case, "f32", backward=False, label=f"f32-padded-N{N}-d{d}")


F32_SPARSE = [
    ("f32-sparse-N129-d64", 129, 64, False, None),
    ("f32-sparse-N640-d32-causal", 640, 32, True, None),
    ("f32-sparse-N700-d128-padded", 700, 128, False, [700, 333]),
    ("f32-sparse-N896-d64-mb256-causal", 896, 64, True, None),
]


@pytest.mark.parametrize("name,N,d,causal,kv", F32_SPARSE, ids=[c[0] for c in F32_SPARSE])
def test_sweep_f32_blocksparse_forward(gpu_lib, name, N, d, causal, kv):
    """The fp32 forward's key-tile list (fa_fwd_blocksparse with FA_F32), ragged N, a key block
    no query block keeps and a query block with no kept key block (O = 0, lse = -inf)."""
    mb = 256 if "mb256" in name else 128
    nb = -(-N // mb)
    B = 1 if kv is None else len(kv)
    case = workloads.make_case(B, 2, N, d, dtype="f32", seed=zlib.crc32(name.encode()) % 10000, causal=causal,
                               kv_len=kv, block_mask=_synthetic_mask(nb, nb + 1), mask_block=mb)
    full_check(gpu_lib, case, "f32", backward=False, label=name)


BF16_SPARSE_FWD = [
    ("bf16-sparse-fwd-N1-d64", 1, 64, False),
    ("bf16-sparse-fwd-N1000-d128-causal", 1000, 128, True),
    ("bf16-sparse-fwd-N2049-d16", 2049, 16, False),
]


@pytest.mark.parametrize("name,N,d,causal", BF16_SPARSE_FWD, ids=[c[0] for c in BF16_SPARSE_FWD])
def test_sweep_bf16_blocksparse_forward(gpu_lib, name, N, d, causal):
    """fa_fwd_blocksparse alone (bf16): a single token, a causal ragged tail, and a sequence
    one token past a whole number of mask blocks."""
    mb = 128
    nb = -(-N // mb)
    case = workloads.make_case(1, 3, N, d, seed=zlib.crc32(name.encode()) % 10000, causal=causal,
                               block_mask=_synthetic_mask(nb, nb + 2), mask_block=mb)
    full_check(gpu_lib, case, "bf16", backward=False, label=name)


@pytest.mark.parametrize("N", [300, 1000])
def test_large_score_magnitude(gpu_lib, N):
    """Q x30: scores with a standard deviation of ~30 make the running maximum jump by
    far more than the lazy-rescale threshold, many times per row."""
    for causal in (False, True):
        case = workloads.make_case(1, 2, N, 64, seed=5, causal=causal, q_magnitude=30.0)
        full_check(gpu_lib, case, "bf16", label=f"q-magnitude30-N{N}-causal{causal}")


def test_scale_sign_and_zero(gpu_lib):
    """A negative scale and a zero scale are valid softmax scales."""
    for s in (-0.125, 0.0, 0.7):
        case = workloads.make_case(1, 2, 200, 64, seed=9, causal=True)
        case["scale"] = s
        full_check(gpu_lib, case, "bf16", label=f"scale{s}")


def test_forward_deterministic(gpu_lib):
    case = workloads.make_case(2, 2, 333, 128, seed=3, causal=True)
    a = gpu_run(gpu_lib, case, backward=False)
    b = gpu_run(gpu_lib, case, backward=False)
    assert torch.equal(a["o"], b["o"]) and torch.equal(a["lse"], b["lse"])


@pytest.mark.parametrize("d", [64, 128])
def test_backward_deterministic(gpu_lib, d):
    """The backward accumulates without atomics: repeated calls are bitwise identical."""
    case = workloads.make_case(2, 3, 700, d, seed=5, causal=True, kv_len=[700, 450])
    a = gpu_run(gpu_lib, case)
    b = gpu_run(gpu_lib, case)
    for n in ("dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n


def test_blocksparse_pattern(gpu_lib):
    """Changing K, V inside blocks masked for query block r leaves block r's O and lse bitwise
    unchanged; keys no query block keeps get dK = dV = 0 exactly."""
    N, mb = 768, 128
    nb = N // mb
    m = _synthetic_mask(nb, 4)
    case = workloads.make_case(1, 2, N, 64, seed=21, block_mask=m, mask_block=mb)
    base = gpu_run(gpu_lib, case)
    for r in range(nb):
        masked = [j for j in range(nb) if not m[r, j]]
        if not masked:
            continue
        pert = dict(case)
        k2, v2 = case["k"].clone(), case["v"].clone()
        gen = torch.Generator("cpu").manual_seed(100 + r)
        for j in masked:
            blk = k2[:, :, j * mb:(j + 1) * mb]
            blk.copy_(torch.randn(blk.shape, generator=gen).to(k2.dtype))
            v2[:, :, j * mb:(j + 1) * mb] = 7.0
        pert["k"], pert["v"] = k2, v2
        got = gpu_run(gpu_lib, pert, backward=False)
        rows = slice(r * mb, (r + 1) * mb)
        assert torch.equal(got["o"][:, :, rows], base["o"][:, :, rows]), r
        assert torch.equal(got["lse"][:, :, rows], base["lse"][:, :, rows]), r
    dead = [j for j in range(nb) if not m[:, j].any()]
    assert dead
    for j in dead:
        assert torch.all(base["dk"][:, :, j * mb:(j + 1) * mb] == 0)
        assert torch.all(base["dv"][:, :, j * mb:(j + 1) * mb] == 0)


def test_padded_keys_get_zero_gradient(gpu_lib):
    case = workloads.make_case(3, 2, 257, 64, seed=8, kv_len=[100, 257, 0])
    got = gpu_run(gpu_lib, case)
    assert torch.all(got["dk"][0, :, 100:] == 0) and torch.all(got["dv"][0, :, 100:] == 0)
    assert torch.all(got["dk"][2] == 0) and torch.all(got["dv"][2] == 0) and torch.all(got["dq"][2] == 0)
    assert torch.all(got["o"][2] == 0) and torch.all(torch.isneginf(got["lse"][2]))


# ------------------------------------------------------------------------------------------
# the named workloads at full size
# ------------------------------------------------------------------------------------------
def test_workload_single_head_f32(gpu_lib):
    w = workloads.WORKLOADS["single_head_f32"]
    full_check(gpu_lib, workloads.generate(w), "f32", backward=False, label=w.name)


@pytest.mark.parametrize("name", ["bert_padded", "gpt2_causal"])
def test_workload_full_oracle(gpu_lib, name):
    w = workloads.WORKLOADS[name]
    full_check(gpu_lib, workloads.generate(w), "bf16", label=w.name)


def _sample_rows(N, rng, extra=()):
    rows = set(range(0, min(N, 40))) | set(range(max(0, N - 40), N)) | set(extra)
    rows |= set(rng.choice(N, size=min(N, 160), replace=False).tolist())
    return np.array(sorted(rows))


def _sampled_check(fa, w, rows, key_rows, key_sel, label):
    """O, lse, dQ on `rows` for every head; dK, dV on keys `key_sel`, using the
    contributions of `key_rows` (every row that may attend to those keys)."""
    note(f"[parity] {label}: generating inputs")
    case = workloads.generate(w)
    note(f"[parity] {label}: GPU forward + backward")
    got = gpu_run(fa, case)
    args = oracle_args(case)
    B, H, N, d = w.B, w.H, w.N, w.d
    note(f"[parity] {label}: oracle on {rows.size} sampled rows")
    q64, k64, v64, do64 = (parity.to64(case[n]) for n in ("q", "k", "v", "do"))
    bm = args["block_mask"]
    ref_o = np.zeros((B, H, rows.size, d))
    ref_l = np.zeros((B, H, rows.size))
    for b in range(B):
        allow = oracle.allowed_pairs(rows, N, causal=w.causal,
                                     kv_len_b=None if args["kv_len"] is None else args["kv_len"][b],
                                     block_mask=bm, mask_block=w.mask_block)
        for h in range(H):
            ref_o[b, h], ref_l[b, h] = oracle.forward_rows(q64[b, h, rows], k64[b, h], v64[b, h], w.scale, allow)
    raw = parity.check_o(got["o"][:, :, rows], ref_o, "bf16", f"{label} O[sampled]")
    lse_err = parity.check_lse(got["lse"][:, :, rows], ref_l, f"{label} lse[sampled]")
    note(f"[parity] {label}: O max-abs {raw:.3e}, lse max-abs {lse_err:.3e} on {rows.size} rows")
    dq, _, _ = oracle.attention_backward(q64, k64, v64, do64, w.scale, rows=rows, **args)
    parity.check_grad(got["dq"][:, :, rows], dq[:, :, rows], f"{label} dQ[sampled]")
    note(f"[parity] {label}: oracle dK/dV on {key_sel.size} keys from {key_rows.size} rows")
    _, dk, dv = oracle.attention_backward(q64, k64, v64, do64, w.scale, rows=key_rows, **args)
    parity.check_grad(got["dk"][:, :, key_sel], dk[:, :, key_sel], f"{label} dK[sampled]")
    parity.check_grad(got["dv"][:, :, key_sel], dv[:, :, key_sel], f"{label} dV[sampled]")


@pytest.mark.parametrize("name", ["long_causal_d64", "long_causal_d128", "long_causal_d32", "long_causal_d16"])
def test_workload_long_causal_sampled(gpu_lib, name):
    w = workloads.WORKLOADS[name]
    rng = np.random.default_rng(1)
    rows = _sample_rows(w.N, rng, extra=range(8191, 8260))
    tail = np.arange(w.N - 1024, w.N)  # causal: keys >= N-1024 are attended only by these rows
    _sampled_check(gpu_lib, w, rows, tail, tail, name)


def test_workload_block_sparse_sampled(gpu_lib):
    w = workloads.WORKLOADS["block_sparse_64k"]
    rng = np.random.default_rng(2)
    rows = _sample_rows(w.N, rng, extra=range(127, 131))
    mb = w.mask_block
    # key blocks 5 and 301 are kept only by query blocks 4..6 and 300..302 under the rule
    key_sel = np.concatenate([np.arange(5 * mb, 6 * mb), np.arange(301 * mb, 302 * mb)])
    key_rows = np.concatenate([np.arange(4 * mb, 7 * mb), np.arange(300 * mb, 303 * mb)])
    _sampled_check(gpu_lib, w, rows, key_rows, key_sel, w.name)


# ------------------------------------------------------------------------------------------
# the longest accumulations at full length: key tiles that every query tile reaches
# ------------------------------------------------------------------------------------------
def _heavy_keys_check(fa, w, keys, label):
    """dK, dV of `keys` in head (0, 0), from the oracle's backward over ALL query rows of that
    head (every row that may attend to them), and dQ of the same head in full."""
    note(f"[parity] {label}: generating inputs")
    case = workloads.generate(w)
    note(f"[parity] {label}: GPU forward + backward")
    got = gpu_run(fa, case)
    note(f"[parity] {label}: oracle backward of head (0, 0), all {w.N} rows")
    dq, dk, dv = oracle.attention_backward(case["q"], case["k"], case["v"], case["do"], w.scale,
                                           heads=[(0, 0)], **oracle_args(case))
    e_k = parity.check_grad(got["dk"][0, 0, keys], dk[0, 0, keys], f"{label} dK[heavy keys]")
    e_v = parity.check_grad(got["dv"][0, 0, keys], dv[0, 0, keys], f"{label} dV[heavy keys]")
    e_q = parity.check_grad(got["dq"][0, 0], dq[0, 0], f"{label} dQ[head 0]")
    e_k_all = parity.check_grad(got["dk"][0, 0], dk[0, 0], f"{label} dK[head 0]")
    e_v_all = parity.check_grad(got["dv"][0, 0], dv[0, 0], f"{label} dV[head 0]")
    note(f"[parity] {label}: rel-L2 heavy dK {e_k:.2e} dV {e_v:.2e}; head 0 dQ {e_q:.2e} dK {e_k_all:.2e} "
         f"dV {e_v_all:.2e}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["long_causal_d64", "long_causal_d128"])
def test_workload_long_causal_heavy_keys(gpu_lib, name):
    """Causal N = 16384: keys 0..127 are attended by all 16384 rows, so their dK/dV workgroup
    accumulates over every query step (at d = 128 the path with K held in registers)."""
    w = workloads.WORKLOADS[name]
    _heavy_keys_check(gpu_lib, w, np.arange(0, 128), name)


@pytest.mark.timeout(900)
def test_workload_block_sparse_global_column(gpu_lib):
    """N = 65536 block-sparse: key block 16 (j mod 16 == 0) is kept by all 512 query blocks,
    the longest dK/dV accumulation of the launch (the 8-wave layout's two-half reduction)."""
    w = workloads.WORKLOADS["block_sparse_64k"]
    mb = w.mask_block
    _heavy_keys_check(gpu_lib, w, np.arange(16 * mb, 17 * mb), w.name)


def test_binding_rejects_host_buffers(gpu_lib):
    """A host (CPU) lse or workspace, or one on the wrong dtype, is refused by the binding with
    ValueError before any call into the library, so no host pointer reaches a kernel."""
    fa = gpu_lib
    case = workloads.make_case(1, 2, 64, 64, seed=1, causal=True)
    q, k, v, do = (case[n].to(DEV) for n in ("q", "k", "v", "do"))
    lse_host = torch.empty((1, 2, 64), dtype=torch.float32)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, v, case["scale"], causal=True, lse=lse_host)
    with pytest.raises(ValueError):
        fa.fa_fwd_blocksparse(q, k, v, case["scale"], torch.ones((1, 1), dtype=torch.uint8, device=DEV),
                              lse=lse_host)
    o, lse = fa.fa_fwd(q, k, v, case["scale"], causal=True)
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, o, do, lse_host, case["scale"], causal=True)
    need = fa.fa_bwd_workspace_bytes(1, 2, 64, 64)
    for bad in (torch.empty(need, dtype=torch.uint8),                       # host memory
                torch.empty(need // 4, dtype=torch.float32, device=DEV)):   # wrong dtype
        with pytest.raises(ValueError):
            fa.fa_bwd(q, k, v, o, do, lse, case["scale"], causal=True, workspace=bad)
        with pytest.raises(ValueError):
            fa.fa_bwd_dropout(q, k, v, o, do, lse, case["scale"], 0.1, 7, causal=True, workspace=bad)
    with pytest.raises(ValueError):
        fa.fa_fwd_kvcache(q, k, v, case["scale"], workspace=torch.empty(1 << 20, dtype=torch.uint8))
    torch.cuda.synchronize()
