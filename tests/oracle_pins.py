"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Every pin takes the oracle module as an argument, so the same battery runs
against the real oracle (all must pass) and against copies with a planted
mistake (at least one must fail; see test_oracle_mutations.py).

None of the pins re-types the oracle's formula. Each checks something the
definition implies by other means:
  * closed forms (Q = 0 -> mean of the allowed values, ln |A_i|; one-hot keys;
    causal row 0),
  * invariants (permutation equivariance, shift invariance, linearity in V,
    rows of P summing to one, exposed through V = I),
  * central finite differences of the oracle's own forward (backward pins),
  * an independent library routine (torch scaled_dot_product_attention in
    float64 on the CPU, with autograd for the gradients), also for the decode
    function on a bottom-right mask built here,
  * brute-force scalar loops on tiny inputs (math.fsum over Python floats).

The allowed sets used by the expected values are built here, from the mask
rules stated in the pages (aiwiki "FlashAttention": causal and variable-length
masks; legiblepapers "Fast and Memory Efficient Exact Attention": predefined
block mask), not by calling the oracle's helper.
"""
from __future__ import annotations

import math

import numpy as np
import torch

RNG = np.random.default_rng


# ----------------------------------------------------------------------------------
# independent construction of the allowed set (scalar rules, Python loops)
# ----------------------------------------------------------------------------------
def allowed_lists(N, causal=False, kv_len_b=None, block_mask=None, mb=1):
    """For each query row i, the sorted list of keys j it may attend to."""
    out = []
    for i in range(N):
        js = []
        for j in range(N):
            if causal and j > i:
                continue
            if kv_len_b is not None and j >= kv_len_b:
                continue
            if block_mask is not None and not block_mask[i // mb][j // mb]:
                continue
            js.append(j)
        out.append(js)
    return out


def dense_bool(lists, N):
    a = np.zeros((len(lists), N), dtype=bool)
    for i, js in enumerate(lists):
        a[i, js] = True
    return a


MASK_CASES = [
    # (name, N, causal, kv_len list per batch, block mask (list of lists) or None, mb)
    ("none", 9, False, None, None, 1),
    ("causal", 9, True, None, None, 1),
    ("padding", 9, False, [5, 9], None, 1),
    ("block", 12, False, None, [[1, 0, 1], [0, 1, 0], [1, 1, 0]], 4),
    ("causal+padding+block", 12, True, [7, 12], [[1, 0, 1], [1, 1, 0], [1, 0, 1]], 4),
]


def _fwd(orc, q, k, v, scale, causal, kv_len, bm, mb):
    return orc.attention_forward(q, k, v, scale, causal=causal, kv_len=kv_len,
                                 block_mask=None if bm is None else np.array(bm), mask_block=mb)


def _bwd(orc, q, k, v, do, scale, causal, kv_len, bm, mb):
    return orc.attention_backward(q, k, v, do, scale, causal=causal, kv_len=kv_len,
                                  block_mask=None if bm is None else np.array(bm), mask_block=mb)


# ----------------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------------
def pin_zero_query(orc):
    """Q = 0: every allowed score is 0, so O_i = mean of the allowed v_j and lse_i = ln |A_i|."""
    for name, N, causal, kv, bm, mb in MASK_CASES:
        B = 1 if kv is None else len(kv)
        rng = RNG(11)
        d = 3
        q = np.zeros((B, 2, N, d))
        k = rng.standard_normal((B, 2, N, d))
        v = rng.standard_normal((B, 2, N, d))
        o, lse = _fwd(orc, q, k, v, 0.7, causal, kv, bm, mb)
        for b in range(B):
            lists = allowed_lists(N, causal, None if kv is None else kv[b], bm, mb)
            for h in range(2):
                for i, js in enumerate(lists):
                    if not js:
                        continue
                    exp_o = [math.fsum(v[b, h, j, c] for j in js) / len(js) for c in range(d)]
                    assert np.allclose(o[b, h, i], exp_o, rtol=0, atol=1e-12), (name, b, h, i)
                    assert abs(lse[b, h, i] - math.log(len(js))) < 1e-12, (name, b, h, i)
    # scale = 0 with a random Q is the same closed form
    rng = RNG(12)
    q, k, v = (rng.standard_normal((1, 1, 7, 4)) for _ in range(3))
    o, lse = orc.attention_forward(q, k, v, 0.0, causal=True)
    for i in range(7):
        assert np.allclose(o[0, 0, i], v[0, 0, : i + 1].mean(axis=0), atol=1e-12)
        assert abs(lse[0, 0, i] - math.log(i + 1)) < 1e-12


def pin_one_hot_keys(orc):
    """k_j = e_{h(j)}, q_i = t e_{g(i)}: the softmax has two levels, exp(a) and 1, a = scale*t."""
    N, d, t, scale = 10, 4, 3.0, 0.5
    hj = [j % d for j in range(N)]
    gi = [(3 * i + 1) % d for i in range(N)]
    k = np.zeros((1, 1, N, d))
    q = np.zeros((1, 1, N, d))
    for j in range(N):
        k[0, 0, j, hj[j]] = 1.0
    for i in range(N):
        q[0, 0, i, gi[i]] = t
    v = RNG(13).standard_normal((1, 1, N, 2))
    a = scale * t
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, scale, causal=causal)
        for i in range(N):
            js = range(i + 1) if causal else range(N)
            w = {j: (math.exp(a) if hj[j] == gi[i] else 1.0) for j in js}
            z = math.fsum(w.values())
            for c in range(2):
                exp_o = math.fsum(w[j] * v[0, 0, j, c] for j in js) / z
                assert abs(o[0, 0, i, c] - exp_o) < 1e-12, (causal, i, c)
            assert abs(lse[0, 0, i] - math.log(z)) < 1e-12, (causal, i)


def pin_causal_row0(orc):
    """Causal row 0 attends only to key 0: O_0 = v_0, lse_0 = scale q_0.k_0, dQ_0 = 0."""
    rng = RNG(14)
    q, k, v, do = (rng.standard_normal((2, 2, 6, 5)) for _ in range(4))
    o, lse = orc.attention_forward(q, k, v, 0.3, causal=True)
    dq, _, _ = orc.attention_backward(q, k, v, do, 0.3, causal=True)
    for b in range(2):
        for h in range(2):
            assert np.allclose(o[b, h, 0], v[b, h, 0], atol=1e-15)
            dot = math.fsum(float(x) * float(y) for x, y in zip(q[b, h, 0], k[b, h, 0]))
            assert abs(lse[b, h, 0] - 0.3 * dot) < 1e-13
            assert np.all(dq[b, h, 0] == 0.0)


def pin_empty_rows(orc):
    """A row with no allowed key: O = 0, lse = -inf; no gradient flows through it."""
    rng = RNG(15)
    q, k, v, do = (rng.standard_normal((2, 1, 5, 3)) for _ in range(4))
    o, lse = orc.attention_forward(q, k, v, 0.5, kv_len=[0, 2])
    dq, dk, dv = orc.attention_backward(q, k, v, do, 0.5, kv_len=[0, 2])
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(dq[0] == 0) and np.all(dk[0] == 0) and np.all(dv[0] == 0)
    assert np.all(np.isfinite(lse[1])) and np.all(dk[1, :, 2:] == 0) and np.all(dv[1, :, 2:] == 0)
    # a block mask with an all-zero block row empties those rows too
    bm = np.array([[1, 0], [0, 0]])
    o, lse = orc.attention_forward(q[:1], k[:1], v[:1], 0.5, block_mask=bm, mask_block=3)
    assert np.all(o[0, 0, 3:] == 0) and np.all(np.isneginf(lse[0, 0, 3:]))
    assert np.all(np.isfinite(lse[0, 0, :3]))


# ----------------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------------
def pin_identity_values(orc):
    """V = I exposes P as O: rows sum to 1, P_ij / P_ik = exp(s_ij - s_ik), lse_i = s_ij - ln P_ij."""
    for name, N, causal, kv, bm, mb in MASK_CASES:
        B = 1 if kv is None else len(kv)
        rng = RNG(16)
        d = 4
        q = rng.standard_normal((B, 1, N, d)) * 2
        k = rng.standard_normal((B, 1, N, d))
        v = np.broadcast_to(np.eye(N), (B, 1, N, N)).copy()
        scale = 0.6
        p, lse = _fwd(orc, q, k, v, scale, causal, kv, bm, mb)
        for b in range(B):
            lists = allowed_lists(N, causal, None if kv is None else kv[b], bm, mb)
            for i, js in enumerate(lists):
                row = p[b, 0, i]
                if not js:
                    assert np.all(row == 0)
                    continue
                assert abs(math.fsum(row) - 1.0) < 1e-12, (name, b, i)
                off = [j for j in range(N) if j not in js]
                assert np.all(row[off] == 0.0), (name, b, i)
                s = {j: scale * math.fsum(float(x) * float(y) for x, y in zip(q[b, 0, i], k[b, 0, j]))
                     for j in js}
                j0 = js[0]
                for j in js:
                    assert abs(row[j] / row[j0] - math.exp(s[j] - s[j0])) < 1e-11 * math.exp(s[j] - s[j0])
                    assert abs(lse[b, 0, i] - (s[j] - math.log(row[j]))) < 1e-11


def pin_permutation_equivariance(orc):
    """Non-causal, unmasked: permuting the rows of K and V leaves O, lse, dQ unchanged and permutes dK, dV."""
    rng = RNG(17)
    q, k, v, do = (rng.standard_normal((1, 2, 11, 5)) for _ in range(4))
    perm = rng.permutation(11)
    o1, l1 = orc.attention_forward(q, k, v, 0.4)
    o2, l2 = orc.attention_forward(q, k[:, :, perm], v[:, :, perm], 0.4)
    assert np.allclose(o1, o2, atol=1e-13) and np.allclose(l1, l2, atol=1e-13)
    g1 = orc.attention_backward(q, k, v, do, 0.4)
    g2 = orc.attention_backward(q, k[:, :, perm], v[:, :, perm], do, 0.4)
    assert np.allclose(g1[0], g2[0], atol=1e-12)
    assert np.allclose(g1[1][:, :, perm], g2[1], atol=1e-12)
    assert np.allclose(g1[2][:, :, perm], g2[2], atol=1e-12)
    # permuting the query rows permutes every per-row output
    o3, l3 = orc.attention_forward(q[:, :, perm], k, v, 0.4)
    assert np.allclose(o1[:, :, perm], o3, atol=1e-13) and np.allclose(l1[:, :, perm], l3, atol=1e-13)


def pin_shift_invariance(orc):
    """K <- K + c (same c for every key) leaves O unchanged and shifts lse_i by scale q_i.c."""
    rng = RNG(18)
    q, k, v = (rng.standard_normal((1, 1, 8, 3)) for _ in range(3))
    c = np.array([0.7, -1.3, 2.1])
    for causal in (False, True):
        o1, l1 = orc.attention_forward(q, k, v, 0.9, causal=causal)
        o2, l2 = orc.attention_forward(q, k + c, v, 0.9, causal=causal)
        assert np.allclose(o1, o2, atol=1e-12)
        assert np.allclose(l2 - l1, 0.9 * (q @ c), atol=1e-12)


def pin_linearity_in_v(orc):
    rng = RNG(19)
    q, k, v1, v2 = (rng.standard_normal((1, 2, 9, 4)) for _ in range(4))
    for causal in (False, True):
        o1, _ = orc.attention_forward(q, k, v1, 0.5, causal=causal)
        o2, _ = orc.attention_forward(q, k, v2, 0.5, causal=causal)
        o3, _ = orc.attention_forward(q, k, 2.5 * v1 - 0.75 * v2, 0.5, causal=causal)
        assert np.allclose(o3, 2.5 * o1 - 0.75 * o2, atol=1e-12)


# ----------------------------------------------------------------------------------
# backward: finite differences of the oracle's own forward
# ----------------------------------------------------------------------------------
def pin_finite_differences(orc):
    """Central differences of L = sum(O * dO) (h = 1e-6) against dQ, dK, dV, every mask type."""
    for name, N, causal, kv, bm, mb in MASK_CASES:
        B = 1 if kv is None else len(kv)
        rng = RNG(20)
        d = 3
        q, k, v, do = (rng.standard_normal((B, 1, N, d)) for _ in range(4))
        scale = 0.8
        grads = _bwd(orc, q, k, v, do, scale, causal, kv, bm, mb)

        def loss(qq, kk, vv):
            o, _ = _fwd(orc, qq, kk, vv, scale, causal, kv, bm, mb)
            return float(np.sum(o * do))

        hstep = 1e-6
        for which, g in zip(range(3), grads):
            base = [q, k, v]
            num = np.zeros_like(g)
            it = np.nditer(base[which], flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                args_p = [x.copy() for x in base]
                args_m = [x.copy() for x in base]
                args_p[which][idx] += hstep
                args_m[which][idx] -= hstep
                num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * hstep)
            err = np.max(np.abs(num - g)) / max(1.0, np.max(np.abs(g)))
            assert err < 1e-7, (name, "qkv"[which], err)


def pin_lse_gradient(orc):
    """d(sum_i lse_i)/dq_i = scale sum_j P_ij k_j, i.e. scale times the forward with V := K."""
    rng = RNG(21)
    q, k = (rng.standard_normal((1, 1, 7, 3)) for _ in range(2))
    scale = 0.7
    for causal in (False, True):
        o_k, _ = orc.attention_forward(q, k, k, scale, causal=causal)
        hstep = 1e-6
        for i in range(7):
            for c in range(3):
                qp, qm = q.copy(), q.copy()
                qp[0, 0, i, c] += hstep
                qm[0, 0, i, c] -= hstep
                lp = orc.attention_forward(qp, k, k, scale, causal=causal)[1].sum()
                lm = orc.attention_forward(qm, k, k, scale, causal=causal)[1].sum()
                assert abs((lp - lm) / (2 * hstep) - scale * o_k[0, 0, i, c]) < 1e-7


# ----------------------------------------------------------------------------------
# independent library routine: torch SDPA in float64 on the CPU, autograd gradients
# ----------------------------------------------------------------------------------
def _sdpa(q, k, v, do, scale, allow):
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.tensor(allow), scale=scale)
    out.backward(torch.tensor(do, dtype=torch.float64))
    return out.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_library_sdpa(orc, magnitude=1.0):
    """Agreement with torch's scaled_dot_product_attention (float64, CPU) on rows with >= 1 allowed key."""
    for name, N, causal, kv, bm, mb in MASK_CASES:
        B = 1 if kv is None else len(kv)
        rng = RNG(22)
        d = 5
        q, k, v, do = (rng.standard_normal((B, 3, N, d)) * magnitude for _ in range(4))
        scale = 1 / math.sqrt(d)
        o, _ = _fwd(orc, q, k, v, scale, causal, kv, bm, mb)
        dq, dk, dv = _bwd(orc, q, k, v, do, scale, causal, kv, bm, mb)
        for b in range(B):
            lists = allowed_lists(N, causal, None if kv is None else kv[b], bm, mb)
            allow = dense_bool(lists, N)
            live = allow.any(axis=1)
            # SDPA returns NaN on fully masked rows; feed it only the live rows' queries
            ro, rdq, rdk, rdv = _sdpa(q[b][:, live], k[b], v[b], do[b][:, live], scale, allow[live])
            tol = 1e-10 * max(1.0, magnitude)
            assert np.allclose(o[b][:, live], ro, atol=tol, rtol=1e-10), name
            assert np.allclose(dq[b][:, live], rdq, atol=tol, rtol=1e-9), name
            assert np.allclose(dk[b], rdk, atol=tol, rtol=1e-9), name
            assert np.allclose(dv[b], rdv, atol=tol, rtol=1e-9), name


def pin_restricted_backward(orc):
    """The sampling mode of the backward (``heads=``, ``rows=``), which the large-workload
    GPU checks rely on. Restricting the loss to rows R of the listed (b, h) is the same as
    L = sum over those rows of O * dO, i.e. dO zeroed everywhere else; torch's SDPA with
    autograd on that dO gives the expected dQ (rows R), dK and dV (every key: the
    contributions of rows R alone). Everything outside the restriction must be exactly 0.
    Masks: causal, key padding, block mask (every row keeps key block 0) and a sliding
    window; a row chunk of 2 puts chunk boundaries inside R."""
    B, H, N, d, mb = 2, 3, 11, 4, 4
    bm = [[1, 0, 1], [1, 1, 0], [1, 0, 1]]
    cases = [
        dict(causal=True, kv_len=[9, 11], block_mask=bm, wl=-1),
        dict(causal=False, kv_len=None, block_mask=None, wl=3),
    ]
    rows = np.array([0, 3, 4, 7, 10])
    heads = [(1, 2), (0, 0), (1, 0)]
    rng = RNG(24)
    for c in cases:
        q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
        scale = 0.6
        dq, dk, dv = orc.attention_backward(
            q, k, v, do, scale, causal=c["causal"], kv_len=c["kv_len"],
            block_mask=None if c["block_mask"] is None else np.array(c["block_mask"]), mask_block=mb,
            window_left=c["wl"], heads=heads, rows=rows, row_chunk=2)
        for b in range(B):
            lists = allowed_lists(N, c["causal"], None if c["kv_len"] is None else c["kv_len"][b],
                                  c["block_mask"], mb if c["block_mask"] is not None else 1)
            allow = dense_bool(lists, N)
            if c["wl"] >= 0:
                allow &= dense_bool(window_lists(N, False, c["wl"], -1), N)
            assert allow.any(axis=1).all()
            for h in range(H):
                if (b, h) not in heads:
                    assert not dq[b, h].any() and not dk[b, h].any() and not dv[b, h].any(), (b, h)
                    continue
                do_r = np.zeros_like(do[b, h])
                do_r[rows] = do[b, h, rows]
                _, rdq, rdk, rdv = _sdpa(q[b, h], k[b, h], v[b, h], do_r, scale, allow)
                assert np.allclose(dq[b, h, rows], rdq[rows], atol=1e-12, rtol=1e-9), (b, h)
                other = np.setdiff1d(np.arange(N), rows)
                assert not dq[b, h, other].any(), (b, h)
                assert np.allclose(dk[b, h], rdk, atol=1e-12, rtol=1e-9), (b, h)
                assert np.allclose(dv[b, h], rdv, atol=1e-12, rtol=1e-9), (b, h)


def pin_large_magnitude(orc):
    """Inputs x30 (scores in the hundreds): still finite and equal to the library routine."""
    pin_library_sdpa(orc, magnitude=30.0)


def pin_block_rule_medium(orc):
    """N = 2048 with causal + block mask (mb = 128) + padding against SDPA on a dense boolean mask."""
    N, d, mb = 2048, 8, 128
    nb = N // mb
    bm = [[1 if (abs(i - j) <= 1 or j % 5 == 0) else 0 for j in range(nb)] for i in range(nb)]
    rng = RNG(23)
    q, k, v, do = (rng.standard_normal((1, 1, N, d)) for _ in range(4))
    scale = 1 / math.sqrt(d)
    o, lse = orc.attention_forward(q, k, v, scale, causal=True, kv_len=[1900],
                                   block_mask=np.array(bm), mask_block=mb)
    ii = np.arange(N)[:, None]
    jj = np.arange(N)[None, :]
    allow = (jj <= ii) & (jj < 1900) & np.kron(np.array(bm, dtype=bool), np.ones((mb, mb), dtype=bool))
    ro, _, _, _ = _sdpa(q[0], k[0], v[0], do[0], scale, allow)
    assert np.allclose(o[0], ro, atol=1e-11)


# ----------------------------------------------------------------------------------
# decode against a key/value cache (kvcache_forward)
# ----------------------------------------------------------------------------------
def _cache_allowed(Nq, Nk, L, causal):
    """Scalar rule: query i (position L - Nq + i) may see key j < L, and j <= L - Nq + i
    when causal."""
    a = np.zeros((Nq, Nk), dtype=bool)
    for i in range(Nq):
        for j in range(Nk):
            if j >= L:
                continue
            if causal and j > L - Nq + i:
                continue
            a[i, j] = True
    return a


def pin_kvcache_zero_query(orc):
    """Q = 0: every allowed key has the same score, so O_i is the mean of the values the
    query may see and lse_i = ln(count); with causal alignment query i sees the first
    L - Nq + i + 1 keys (none when that is <= 0)."""
    rng = RNG(31)
    B, H, Nq, Nk, d = 3, 2, 5, 19, 4
    lens = [19, 7, 3]
    q = np.zeros((B, H, Nq, d))
    k, v = rng.standard_normal((B, H, Nk, d)), rng.standard_normal((B, H, Nk, d))
    for causal in (False, True):
        o, lse = orc.kvcache_forward(q, k, v, 0.37, causal=causal, kv_len=lens)
        for b, L in enumerate(lens):
            for i in range(Nq):
                n = min(L, L - Nq + i + 1) if causal else L
                for h in range(H):
                    if n <= 0:
                        assert np.all(o[b, h, i] == 0) and np.isneginf(lse[b, h, i])
                    else:
                        assert np.allclose(o[b, h, i], v[b, h, :n].mean(axis=0), atol=1e-13)
                        assert abs(lse[b, h, i] - math.log(n)) < 1e-13


def pin_kvcache_single_query(orc):
    """Nq = 1 (one decode step): the query sees every cached key, causal or not; checked
    against a brute-force scalar softmax."""
    rng = RNG(32)
    Nk, d, L = 23, 3, 17
    q, k, v = rng.standard_normal((1, 1, 1, d)), rng.standard_normal((1, 1, Nk, d)), rng.standard_normal((1, 1, Nk, d))
    for causal in (False, True):
        o, lse = orc.kvcache_forward(q, k, v, 0.8, causal=causal, kv_len=[L])
        sc = [0.8 * math.fsum(q[0, 0, 0, t] * k[0, 0, j, t] for t in range(d)) for j in range(L)]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        z = math.fsum(w)
        ref = [math.fsum(w[j] * v[0, 0, j, t] for j in range(L)) / z for t in range(d)]
        assert np.allclose(o[0, 0, 0], ref, atol=1e-13)
        assert abs(lse[0, 0, 0] - (m + math.log(z))) < 1e-12


def pin_kvcache_library_sdpa(orc):
    """Agreement with torch SDPA (float64) on the explicitly built bottom-right mask."""
    rng = RNG(33)
    B, H, Nq, Nk, d = 2, 2, 6, 40, 5
    lens = [40, 29]
    q = rng.standard_normal((B, H, Nq, d))
    k, v = rng.standard_normal((B, H, Nk, d)), rng.standard_normal((B, H, Nk, d))
    for causal in (False, True):
        o, _ = orc.kvcache_forward(q, k, v, 0.45, causal=causal, kv_len=lens)
        for b, L in enumerate(lens):
            allow = _cache_allowed(Nq, Nk, L, causal)
            live = allow.any(axis=1)
            ro, _, _, _ = _sdpa(q[b][:, live], k[b], v[b], np.zeros_like(q[b][:, live]), 0.45, allow[live])
            assert np.allclose(o[b][:, live], ro, atol=1e-12), (causal, b)


# ----------------------------------------------------------------------------------
# sliding window and packed variable-length sequences
# ----------------------------------------------------------------------------------
def window_lists(N, causal, wl, wr):
    """Allowed keys per query under the causal and sliding-window rules (scalar loops)."""
    out = []
    for i in range(N):
        js = []
        for j in range(N):
            if causal and j > i:
                continue
            if wl >= 0 and j < i - wl:
                continue
            if wr >= 0 and j > i + wr:
                continue
            js.append(j)
        out.append(js)
    return out


def _lse_loop(q, k, scale, js):
    """ln sum_j exp(scale q . k_j) by scalar loops (shifted by the maximum for range)."""
    if not js:
        return -math.inf
    s = [scale * math.fsum(float(a) * float(b) for a, b in zip(q, k[j])) for j in js]
    m = max(s)
    return m + math.log(math.fsum(math.exp(x - m) for x in s))


WINDOW_CASES = [  # (N, causal, window_left, window_right)
    (11, False, 3, 2),
    (11, True, 4, -1),
    (11, False, -1, 0),
    (11, False, 0, 5),
    (11, True, 2, 7),
    (11, False, 20, 20),
]


def pin_window_library_sdpa(orc):
    """Sliding windows (with and without causal) against torch SDPA on masks built here."""
    rng = RNG(40)
    for N, causal, wl, wr in WINDOW_CASES:
        d, scale = 4, 0.6
        q, k, v, do = (rng.standard_normal((2, 2, N, d)) for _ in range(4))
        o, lse = orc.attention_forward(q, k, v, scale, causal=causal, window_left=wl, window_right=wr)
        dq, dk, dv = orc.attention_backward(q, k, v, do, scale, causal=causal, window_left=wl,
                                            window_right=wr)
        lists = window_lists(N, causal, wl, wr)
        allow = dense_bool(lists, N)
        live = allow.any(axis=1)
        for b in range(2):
            ro, rdq, rdk, rdv = _sdpa(q[b][:, live], k[b], v[b], do[b][:, live], scale, allow[live])
            case = (N, causal, wl, wr, b)
            assert np.allclose(o[b][:, live], ro, atol=1e-12), case
            assert np.allclose(dq[b][:, live], rdq, atol=1e-11), case
            assert np.allclose(dk[b], rdk, atol=1e-11), case
            assert np.allclose(dv[b], rdv, atol=1e-11), case
            for h in range(2):
                for i in range(N):
                    ref = _lse_loop(q[b, h, i], k[b, h], scale, lists[i])
                    assert (ref == -math.inf and lse[b, h, i] == -math.inf) or abs(lse[b, h, i] - ref) < 1e-12, case


def pin_window_self_only(orc):
    """Left extent 0 with causal (or both extents 0): each query sees only its own key, so
    O_i = v_i and lse_i = scale q_i . k_i; the same inside every packed sequence."""
    rng = RNG(41)
    q, k, v = (rng.standard_normal((1, 2, 9, 3)) for _ in range(3))
    for causal, wl, wr in ((True, 0, -1), (False, 0, 0)):
        o, lse = orc.attention_forward(q, k, v, 0.9, causal=causal, window_left=wl, window_right=wr)
        assert np.allclose(o, v, atol=1e-15)
        assert np.allclose(lse, 0.9 * np.einsum("bhnd,bhnd->bhn", q, k), atol=1e-14)
    cu = [0, 3, 3, 8, 9]
    qp, kp, vp = (rng.standard_normal((9, 2, 3)) for _ in range(3))
    o, lse = orc.varlen_forward(qp, kp, vp, cu, 0.9, causal=True, window_left=0)
    assert np.allclose(o, vp, atol=1e-15)
    assert np.allclose(lse, 0.9 * np.einsum("thd,thd->ht", qp, kp), atol=1e-14)


VARLEN_CU = [0, 5, 5, 12, 13, 20]  # lengths 5, 0, 7, 1, 7


def pin_varlen_library_sdpa(orc):
    """Packed sequences: every sequence against torch SDPA on its own slice (forward, lse by
    scalar loops, gradients), for full, causal and windowed masks."""
    rng = RNG(42)
    total, H, d, scale = VARLEN_CU[-1], 2, 3, 0.7
    q, k, v, do = (rng.standard_normal((total, H, d)) for _ in range(4))
    for causal, wl, wr in ((False, -1, -1), (True, -1, -1), (False, 2, 1), (True, 3, -1)):
        o, lse = orc.varlen_forward(q, k, v, VARLEN_CU, scale, causal=causal, window_left=wl, window_right=wr)
        dq, dk, dv = orc.varlen_backward(q, k, v, do, VARLEN_CU, scale, causal=causal, window_left=wl,
                                         window_right=wr)
        assert o.shape == (total, H, d) and lse.shape == (H, total)
        for c0, c1 in zip(VARLEN_CU[:-1], VARLEN_CU[1:]):
            n = c1 - c0
            if n == 0:
                continue
            lists = window_lists(n, causal, wl, wr)
            allow = dense_bool(lists, n)
            sl = [x[c0:c1].transpose(1, 0, 2) for x in (q, k, v, do)]  # [H, n, d]
            ro, rdq, rdk, rdv = _sdpa(*sl, scale, allow)
            case = (causal, wl, wr, c0)
            assert np.allclose(o[c0:c1].transpose(1, 0, 2), ro, atol=1e-12), case
            assert np.allclose(dq[c0:c1].transpose(1, 0, 2), rdq, atol=1e-11), case
            assert np.allclose(dk[c0:c1].transpose(1, 0, 2), rdk, atol=1e-11), case
            assert np.allclose(dv[c0:c1].transpose(1, 0, 2), rdv, atol=1e-11), case
            for h in range(H):
                for i in range(n):
                    ref = _lse_loop(q[c0 + i, h], k[c0:c1, h], scale, lists[i])
                    assert abs(lse[h, c0 + i] - ref) < 1e-12, case


def pin_varlen_isolation(orc):
    """Changing one sequence's keys and values changes no other sequence's results."""
    rng = RNG(43)
    total, H, d = VARLEN_CU[-1], 2, 3
    q, k, v, do = (rng.standard_normal((total, H, d)) for _ in range(4))
    k2, v2 = k.copy(), v.copy()
    k2[5:12] += 3.0
    v2[5:12] -= 2.0
    a = orc.varlen_forward(q, k, v, VARLEN_CU, 0.5, causal=True)
    b = orc.varlen_forward(q, k2, v2, VARLEN_CU, 0.5, causal=True)
    ga = orc.varlen_backward(q, k, v, do, VARLEN_CU, 0.5, causal=True)
    gb = orc.varlen_backward(q, k2, v2, do, VARLEN_CU, 0.5, causal=True)
    other = np.r_[0:5, 12:20]
    assert np.array_equal(a[0][other], b[0][other]) and np.array_equal(a[1][:, other], b[1][:, other])
    for x, y in zip(ga, gb):
        assert np.array_equal(x[other], y[other])
    assert not np.allclose(a[0][5:12], b[0][5:12])


# ----------------------------------------------------------------------------------
# dropout: the counter-based generator and the mask it defines
# ----------------------------------------------------------------------------------
def _philox_scalar(c, k):
    """Philox4x32-10 on Python integers, one block at a time (a second implementation of
    the published definition, written independently of the oracle's array version)."""
    mask = 0xFFFFFFFF
    x0, x1, x2, x3 = (int(v) & mask for v in c)
    k0, k1 = int(k[0]) & mask, int(k[1]) & mask
    for _ in range(10):
        prod0 = 0xD2511F53 * x0
        prod1 = 0xCD9E8D57 * x2
        x0, x1, x2, x3 = ((prod1 >> 32) ^ x1 ^ k0) & mask, prod1 & mask, ((prod0 >> 32) ^ x3 ^ k1) & mask, prod0 & mask
        k0 = (k0 + 0x9E3779B9) & mask
        k1 = (k1 + 0xBB67AE85) & mask
    return [x0, x1, x2, x3]


def pin_philox_known_answers(orc):
    """The generator reproduces the known-answer vectors published with it
    (tests/golden/philox4x32_10_kat.json), and so does the scalar re-implementation."""
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "philox4x32_10_kat.json")
    for vec in json.load(open(path))["vectors"]:
        c = [int(x, 16) for x in vec["counter"]]
        k = [int(x, 16) for x in vec["key"]]
        want = [int(x, 16) for x in vec["output"]]
        got = [int(w) for w in orc.philox4x32_10(*c, *k)]
        assert got == want, (vec, [hex(g) for g in got])
        assert _philox_scalar(c, k) == want


def _keep_scalar(b, h, i, j, seed, p):
    """The keep rule for one pair, on Python integers: the call for the block of keys
    4 (j // 4) .. + 3 and queries 2 (i // 2), + 1; of its eight 16-bit values (two per
    word, low half first) the pair takes value number 2 (j % 4) + i % 2."""
    words = _philox_scalar((j // 4, i // 2, h, b), (seed & 0xFFFFFFFF, seed >> 32))
    values = [(wd >> shift) & 0xFFFF for wd in words for shift in (0, 16)]
    return values[2 * (j % 4) + i % 2] >= min(math.floor(p * 65536), 65535)


def pin_dropout_mask_rule(orc):
    """dropout_keep follows the stated rule element by element (scalar generator calls)."""
    for b, h, seed, p in ((0, 0, 1, 0.5), (3, 5, 0x1234567890ABCDEF, 0.1), (1, 2, 77, 0.9)):
        rows, cols = [0, 1, 2, 5, 130, 131], list(range(0, 23)) + [64, 127, 1000]
        keep = orc.dropout_keep(b, h, rows, cols, seed, p)
        for a, i in enumerate(rows):
            for c, j in enumerate(cols):
                assert bool(keep[a, c]) == _keep_scalar(b, h, i, j, seed, p), (b, h, seed, p, i, j)


def pin_dropout_keep_rate(orc):
    """Over 512 x 512 elements the kept fraction is 1 - p within 6 binomial standard
    deviations, and different heads and seeds give different masks."""
    n = 512 * 512
    for p in (0.1, 0.5, 0.9):
        keep = orc.dropout_keep(0, 1, np.arange(512), np.arange(512), 2024, p)
        sd = math.sqrt(n * p * (1 - p))
        assert abs(keep.sum() - n * (1 - p)) < 6 * sd, (p, keep.mean())
    a = orc.dropout_keep(0, 0, np.arange(64), np.arange(64), 5, 0.5)
    assert not np.array_equal(a, orc.dropout_keep(0, 1, np.arange(64), np.arange(64), 5, 0.5))
    assert not np.array_equal(a, orc.dropout_keep(1, 0, np.arange(64), np.arange(64), 5, 0.5))
    assert not np.array_equal(a, orc.dropout_keep(0, 0, np.arange(64), np.arange(64), 6, 0.5))
    assert orc.dropout_keep(0, 0, np.arange(64), np.arange(64), 5, 0.0).all()


def pin_dropout_identity_values(orc):
    """V = I exposes P o M: O_ij = P_ij keep_ij / (1 - p), P from a scalar softmax loop and
    keep from the scalar generator; lse is that of the undropped softmax."""
    rng = RNG(50)
    N, d, scale, p, seed = 12, 3, 0.8, 0.4, 99
    q, k = rng.standard_normal((2, 1, N, d)), rng.standard_normal((2, 1, N, d))
    v = np.broadcast_to(np.eye(N), (2, 1, N, N)).copy()
    for causal in (False, True):
        o, lse = orc.attention_forward(q, k, v, scale, causal=causal, dropout_p=p, dropout_seed=seed)
        for b in range(2):
            for i in range(N):
                js = list(range(i + 1)) if causal else list(range(N))
                ss = [scale * math.fsum(float(x) * float(y) for x, y in zip(q[b, 0, i], k[b, 0, j])) for j in js]
                mx = max(ss)
                den = math.fsum(math.exp(x - mx) for x in ss)
                for j in range(N):
                    want = 0.0
                    if j in js and _keep_scalar(b, 0, i, j, seed, p):
                        want = math.exp(ss[js.index(j)] - mx) / den / (1 - p)
                    assert abs(o[b, 0, i, j] - want) < 1e-12, (causal, b, i, j)
                assert abs(lse[b, 0, i] - (mx + math.log(den))) < 1e-12


def pin_dropout_finite_differences(orc):
    """The mask does not depend on the inputs: central differences of L = sum(O * dO)
    against dQ, dK, dV with dropout, causal and padded."""
    rng = RNG(51)
    B, N, d, scale, p, seed = 2, 7, 3, 0.7, 0.3, 4242
    q, k, v, do = (rng.standard_normal((B, 1, N, d)) for _ in range(4))
    kw = dict(causal=True, kv_len=[7, 5], dropout_p=p, dropout_seed=seed)
    grads = orc.attention_backward(q, k, v, do, scale, **kw)

    def loss(qq, kk, vv):
        return float(np.sum(orc.attention_forward(qq, kk, vv, scale, **kw)[0] * do))

    for which, g in enumerate(grads):
        base = [q, k, v]
        num = np.zeros_like(g)
        it = np.nditer(base[which], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            pp = [x.copy() for x in base]
            mm = [x.copy() for x in base]
            pp[which][idx] += 1e-6
            mm[which][idx] -= 1e-6
            num[idx] = (loss(*pp) - loss(*mm)) / 2e-6
        err = np.max(np.abs(num - g)) / max(1.0, np.max(np.abs(g)))
        assert err < 1e-7, ("qkv"[which], err)


ALL_PINS = [
    pin_zero_query,
    pin_one_hot_keys,
    pin_causal_row0,
    pin_empty_rows,
    pin_identity_values,
    pin_permutation_equivariance,
    pin_shift_invariance,
    pin_linearity_in_v,
    pin_finite_differences,
    pin_lse_gradient,
    pin_library_sdpa,
    pin_restricted_backward,
    pin_large_magnitude,
    pin_block_rule_medium,
    pin_kvcache_zero_query,
    pin_kvcache_single_query,
    pin_kvcache_library_sdpa,
    pin_window_library_sdpa,
    pin_window_self_only,
    pin_varlen_library_sdpa,
    pin_varlen_isolation,
    pin_philox_known_answers,
    pin_dropout_mask_rule,
    pin_dropout_keep_rate,
    pin_dropout_identity_values,
    pin_dropout_finite_differences,
]
