"""Plain, slow fp64 CPU oracle of exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it. It shares no code with the HIP path (no kernels,
headers, helpers, tables or pre/post-processing); both sides see the same
seeded inputs and nothing else.

What it computes, and where the pages define it
------------------------------------------------
* Forward — aiwiki.page "FlashAttention", section "Attention and the memory
  bottleneck": the output is the row-wise softmax of the scaled score matrix
  ``Q K^T / sqrt(d)`` applied to ``V``; masks restrict which query–key pairs
  may interact. The scale is a caller argument (the configs use 1/sqrt(d)).
  The same page, section "Tiling and online normalization", states that the
  tiled algorithm reaches this plain result up to floating-point reordering,
  so the oracle is the plain definition: it materialises the score rows,
  takes a two-pass (max, then sum) softmax and multiplies by V. It does NOT
  use the online (running max / running sum) recurrence.
* Row statistics — sendsoonai.com "FlashAttention: IO-aware explained",
  section "Recomputation and IO complexity": only the per-row softmax
  statistics (m, l) are kept. The oracle reports them in the combined form
  ``lse_i = m_i + ln l_i`` (natural log, since the page's update equations
  use e^x), i.e. ``lse_i = ln sum_{j allowed} exp(scale * q_i . k_j)``.
* Masks — aiwiki "FlashAttention", sections "Attention and the memory
  bottleneck" (masks restrict pairs) and "Software integration and
  limitations" (causal masks, variable-length sequences); legiblepapers.com
  "Fast and Memory Efficient Exact Attention", summary paragraph (block-sparse
  attention skips the zero blocks of a predefined block mask). The allowed set
  is the AND of the three predicates:
      causal:   j <= i                       (square self-attention)
      padding:  j <  L_b                     (key padding per batch entry)
      block:    mask[i // mb][j // mb] != 0  (block-sparse, mb = mask block)
  Query rows are never masked; a row with no allowed key has O = 0,
  lse = -inf and zero gradient (the pages are silent; plainest reading).
* Sliding window — aiwiki "FlashAttention", section "Software integration and
  limitations", lists sliding-window masks among the interfaces; the cochat.ai
  audit's citation check of the Longformer reference describes sliding-window
  attention as each query attending a fixed window of w keys (O(n w) work).
  Plainest reading: a left extent wl and a right extent wr, each unbounded when
  negative; key j is allowed for query i iff i - wl <= j <= i + wr (another
  predicate in the AND above; causal is the same as wr = 0).
* Variable-length packed sequences — same aiwiki section ("variable-length
  sequences"). Plainest reading, used by ``varlen_forward`` / ``varlen_backward``:
  sequences are packed along one token axis, q/k/v of shape [total, H, d], with
  sequence s owning tokens cu_seqlens[s] .. cu_seqlens[s+1] - 1; attention (and
  every mask, with positions counted from the sequence's first token) acts
  within a sequence only. lse is returned as [H, total].
* Decode against a key/value cache — aiwiki "FlashAttention", section "Software
  integration and limitations", lists inference with cached keys and values
  among the interfaces but defines no semantics. Plainest reading, used by
  ``kvcache_forward``: Nq new queries are the last Nq positions of a sequence
  whose first L_b keys and values are in the cache (the new tokens' own keys
  included); query i sits at position L_b - Nq + i and, when causal, attends
  key j iff j <= L_b - Nq + i; always j < L_b. With Nq = Nk = L_b this is the
  square causal mask above.
* Dropout — the cochat.ai audit of "FlashAttention: Fast and Memory-Efficient
  Exact Attention with IO-Awareness" quotes the fused kernel applying dropout to
  the attention probabilities and the backward regenerating the same mask from
  the generator state instead of storing it. The pages give no generator, so
  the oracle fixes one: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
  random numbers: as easy as 1, 2, 3", SC 2011), a counter-based generator
  written here from its published definition (``philox4x32_10``). One call
  covers a block of 4 keys x 2 queries: its counter is (j // 4, i // 2, h, b)
  and its key (seed mod 2^32, seed // 2^32); its four 32-bit words hold eight
  16-bit values, and key j of query i in batch b, head h takes word (j mod 4),
  16-bit half (i mod 2) (0 = low). The pair is kept iff that value is
  >= floor(p 2^16); kept probabilities are scaled by 1 / (1 - p).
  lse stays that of the undropped softmax: O = (P o M) V with M = keep / (1 - p).
* Backward — the pages say only that the backward is simplified analytically
  and recomputes the attention matrix from the saved statistics
  (cochat.ai audit of "FlashAttention: Fast and Memory-Efficient Exact
  Attention with IO-Awareness", quoted App. B.2/B.4 and Theorem 5 proof). The
  oracle is the chain rule of the definition, written out with the softmax
  Jacobian (no rowsum(dO*O) shortcut):
      dV = (P o M)^T dO                    (M = 1 without dropout)
      dP = dO V^T
      dS_ij = P_ij (M_ij dP_ij - sum_k P_ik M_ik dP_ik)
      dQ = scale * dS K
      dK = scale * dS^T Q

Evaluation order: rows are processed in independent chunks (each row of the
definition depends only on its own query), and for a chunk only the key
columns that at least one of its rows may attend to are gathered. A dropped
column has P = 0 exactly, so both are exact rewrites of the definition, not
reorderings of any sum over allowed keys.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "allowed_pairs",
    "forward_rows",
    "attention_forward",
    "attention_backward",
    "kvcache_forward",
    "varlen_forward",
    "varlen_backward",
    "philox4x32_10",
    "dropout_keep",
]

_ROW_CHUNK = 256


def _as_f64(x) -> np.ndarray:
    """Exact widening of the caller's values (fp32 / bf16-as-fp32) to fp64."""
    if hasattr(x, "detach"):  # a torch tensor: go through float32, exact for bf16/fp32
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


_PHILOX_M = (0xD2511F53, 0xCD9E8D57)   # round multipliers (Salmon et al., SC 2011)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)   # key schedule increments (same source)
_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on arrays of 32-bit counter words (broadcast together).

    One round: the products M0 x0 and M1 x2 (64-bit) split into high and low words;
    the new state is (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)),
    then the key is bumped by the two Weyl constants. Returns the four output words.
    """
    x = [np.asarray(v, dtype=np.uint64) & _U32 for v in (c0, c1, c2, c3)]
    x = list(np.broadcast_arrays(*x))
    k0, k1 = np.uint64(k0 & 0xFFFFFFFF), np.uint64(k1 & 0xFFFFFFFF)
    m0, m1 = np.uint64(_PHILOX_M[0]), np.uint64(_PHILOX_M[1])
    for _ in range(10):
        p0, p1 = m0 * x[0], m1 * x[2]                     # exact: both factors < 2^32
        x = [((p1 >> np.uint64(32)) ^ x[1] ^ k0) & _U32, p1 & _U32,
             ((p0 >> np.uint64(32)) ^ x[3] ^ k1) & _U32, p0 & _U32]
        k0 = (k0 + np.uint64(_PHILOX_W[0])) & _U32
        k1 = (k1 + np.uint64(_PHILOX_W[1])) & _U32
    return x


def dropout_keep(b: int, h: int, rows, cols, seed: int, p: float) -> np.ndarray:
    """Boolean [len(rows), len(cols)]: is key j of query i kept (module docstring)."""
    rows = np.asarray(rows, dtype=np.int64)[:, None]
    cols = np.asarray(cols, dtype=np.int64)[None, :]
    words = philox4x32_10(cols >> 2, rows >> 1, h, b, seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.choose(np.broadcast_to(cols & 3, words[0].shape), words)        # word j mod 4
    half = (w >> (np.uint64(16) * (rows & 1).astype(np.uint64))) & np.uint64(0xFFFF)  # half i mod 2
    threshold = min(int(np.floor(p * 65536.0)), 65535)
    return half >= np.uint64(threshold)


def _dropout_scale(b, h, rows, cols, dropout_p, dropout_seed):
    """M = keep / (1 - p) on the given rows and key columns, or None without dropout."""
    if dropout_p == 0.0:
        return None
    return dropout_keep(b, h, rows, cols, dropout_seed, dropout_p) / (1.0 - dropout_p)


def allowed_pairs(rows: np.ndarray, n_keys: int, *, causal: bool, kv_len_b,
                  block_mask, mask_block: int, window_left: int = -1,
                  window_right: int = -1) -> np.ndarray:
    """Boolean [len(rows), n_keys]: may query ``i`` attend to key ``j``.

    The AND of the causal (j <= i), key-padding (j < L_b), block-mask
    (mask[i // mb][j // mb] != 0) and sliding-window (i - wl <= j <= i + wr, a
    negative extent being unbounded) predicates; see the module docstring for
    the passages that define each.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(n_keys, dtype=np.int64)
    allow = np.ones((rows.size, n_keys), dtype=bool)
    if causal:
        allow &= cols[None, :] <= rows[:, None]
    if kv_len_b is not None:
        allow &= cols[None, :] < int(kv_len_b)
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0
        allow &= bm[rows[:, None] // mask_block, cols[None, :] // mask_block]
    if window_left >= 0:
        allow &= cols[None, :] >= rows[:, None] - window_left
    if window_right >= 0:
        allow &= cols[None, :] <= rows[:, None] + window_right
    return allow


def forward_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 allow: np.ndarray, drop: np.ndarray | None = None):
    """Exact attention for a set of query rows of one (batch, head).

    q_rows [R, d], k [Nk, d], v [Nk, dv], allow [R, Nk] -> (O [R, dv], lse [R]).
    Two-pass softmax of the materialised score rows (aiwiki "FlashAttention",
    section "Attention and the memory bottleneck"). ``drop``: optional [R, Nk]
    dropout multipliers M (keep / (1 - p)) applied to P before it meets V.
    """
    cols = np.nonzero(allow.any(axis=0))[0]
    R = q_rows.shape[0]
    out = np.zeros((R, v.shape[1]), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    if cols.size == 0:
        return out, lse
    a = allow[:, cols]
    s = scale * (q_rows @ k[cols].T)                 # scores S = scale * Q K^T
    s = np.where(a, s, -np.inf)                      # masked pairs leave the softmax
    m = s.max(axis=1)                                # pass 1: row maximum
    live = np.isfinite(m)                            # rows with at least one allowed key
    m_safe = np.where(live, m, 0.0)
    e = np.exp(s - m_safe[:, None])                  # exp(-inf) = 0 for masked pairs
    l = e.sum(axis=1)                                # pass 2: row sum
    p = np.where(live[:, None], e / np.where(live, l, 1.0)[:, None], 0.0)
    if drop is not None:
        p = p * drop[:, cols]
    out[:] = p @ v[cols]
    lse[live] = m[live] + np.log(l[live])
    return out, lse


def attention_forward(q, k, v, scale: float, *, causal: bool = False, kv_len=None,
                      block_mask=None, mask_block: int = 128, window_left: int = -1,
                      window_right: int = -1, dropout_p: float = 0.0, dropout_seed: int = 0,
                      row_chunk: int = _ROW_CHUNK):
    """O, lse for q/k/v of shape [B, H, N, d] (any float dtype, widened to fp64).

    kv_len: None or length-B integers (key padding). block_mask: None or a 2-D
    array [ceil(N/mb), ceil(N/mb)] shared by every (b, h), nonzero = keep.
    window_left / window_right: sliding-window extents (negative = unbounded).
    dropout_p / dropout_seed: dropout on the probabilities (module docstring).
    Returns O [B, H, N, d] fp64 and lse [B, H, N] fp64 (natural log).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, N, _ = q.shape
    out = np.zeros(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    lse = np.full((B, H, N), -np.inf, dtype=np.float64)
    lens = None if kv_len is None else [int(x) for x in np.asarray(kv_len).reshape(-1)]
    for b in range(B):
        for r0 in range(0, N, row_chunk):
            rows = np.arange(r0, min(N, r0 + row_chunk))
            allow = allowed_pairs(rows, k.shape[2], causal=causal,
                                  kv_len_b=None if lens is None else lens[b],
                                  block_mask=block_mask, mask_block=mask_block,
                                  window_left=window_left, window_right=window_right)
            for h in range(H):
                drop = _dropout_scale(b, h, rows, np.arange(k.shape[2]), dropout_p, dropout_seed)
                o_r, l_r = forward_rows(q[b, h, rows], k[b, h], v[b, h], scale, allow, drop)
                out[b, h, rows] = o_r
                lse[b, h, rows] = l_r
    return out, lse


def attention_backward(q, k, v, dout, scale: float, *, causal: bool = False, kv_len=None,
                       block_mask=None, mask_block: int = 128, window_left: int = -1,
                       window_right: int = -1, dropout_p: float = 0.0, dropout_seed: int = 0,
                       heads=None, rows=None, row_chunk: int = _ROW_CHUNK):
    """dQ, dK, dV of L = sum(O * dO) for the forward above, all fp64.

    The probabilities are recomputed from the definition (two-pass softmax);
    the softmax Jacobian-vector product is written out in full. ``heads``
    optionally restricts the work to a list of (b, h) pairs, and ``rows`` to a
    sorted list of query rows: only those rows get dQ, and dK / dV then hold
    the contributions of those rows alone (exact for every key that no other
    row may attend to). Entries outside the restriction stay zero. Both serve
    to sample a large workload.
    """
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    B, H, N, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    lens = None if kv_len is None else [int(x) for x in np.asarray(kv_len).reshape(-1)]
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)
    all_rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    for b, h in pairs:
        for r0 in range(0, all_rows.size, row_chunk):
            rows = all_rows[r0:r0 + row_chunk]
            allow = allowed_pairs(rows, k.shape[2], causal=causal,
                                  kv_len_b=None if lens is None else lens[b],
                                  block_mask=block_mask, mask_block=mask_block,
                                  window_left=window_left, window_right=window_right)
            cols = np.nonzero(allow.any(axis=0))[0]
            if cols.size == 0:
                continue
            a = allow[:, cols]
            kc, vc, qr, dor = k[b, h, cols], v[b, h, cols], q[b, h, rows], dout[b, h, rows]
            s = np.where(a, scale * (qr @ kc.T), -np.inf)
            m = s.max(axis=1)
            live = np.isfinite(m)
            e = np.exp(s - np.where(live, m, 0.0)[:, None])
            l = e.sum(axis=1)
            p = np.where(live[:, None], e / np.where(live, l, 1.0)[:, None], 0.0)
            mm = _dropout_scale(b, h, rows, cols, dropout_p, dropout_seed)
            mm = np.ones_like(p) if mm is None else mm         # dropout multipliers M
            dv[b, h, cols] += (p * mm).T @ dor                 # dV = (P o M)^T dO
            dp = (dor @ vc.T) * mm                             # dP = dO V^T, through M
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))  # softmax Jacobian
            dq[b, h, rows] = scale * (ds @ kc)                 # dQ = scale dS K
            dk[b, h, cols] += scale * (ds.T @ qr)              # dK = scale dS^T Q
    return dq, dk, dv


def kvcache_forward(q, k, v, scale: float, *, causal: bool = False, kv_len=None):
    """O, lse of Nq queries against a key/value cache (module docstring, "Decode").

    q [B, H, Nq, d]; k, v [B, H, Nk, d]; kv_len None (L_b = Nk) or length-B integers,
    clamped to [0, Nk]. Query i of batch b attends key j iff j < L_b and, if causal,
    j <= L_b - Nq + i. Returns O [B, H, Nq, d] and lse [B, H, Nq] in fp64; a query with
    no allowed key gets O = 0, lse = -inf.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    out = np.zeros(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    lse = np.full((B, H, Nq), -np.inf, dtype=np.float64)
    lens = [Nk] * B if kv_len is None else [min(max(int(x), 0), Nk) for x in np.asarray(kv_len).reshape(-1)]
    cols = np.arange(Nk, dtype=np.int64)
    for b in range(B):
        L = lens[b]
        allow = np.broadcast_to(cols[None, :] < L, (Nq, Nk)).copy()
        if causal:
            pos = L - Nq + np.arange(Nq, dtype=np.int64)      # absolute query positions
            allow &= cols[None, :] <= pos[:, None]
        for h in range(H):
            out[b, h], lse[b, h] = forward_rows(q[b, h], k[b, h], v[b, h], scale, allow)
    return out, lse


def _segments(cu_seqlens, total: int):
    cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
    if len(cu) < 2 or cu[0] != 0 or cu[-1] != total or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0, be nondecreasing and end at the token count")
    return list(zip(cu[:-1], cu[1:]))


def varlen_forward(q, k, v, cu_seqlens, scale: float, *, causal: bool = False,
                   window_left: int = -1, window_right: int = -1):
    """O [total, H, d] and lse [H, total] of packed sequences (module docstring).

    q, k, v [total, H, d]; sequence s is tokens cu_seqlens[s] .. cu_seqlens[s+1] - 1
    and attends within itself, with the causal and sliding-window masks counted from
    its first token.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    total, H, _ = q.shape
    out = np.zeros((total, H, v.shape[2]), dtype=np.float64)
    lse = np.full((H, total), -np.inf, dtype=np.float64)
    for c0, c1 in _segments(cu_seqlens, total):
        if c1 == c0:
            continue
        seq = [x[c0:c1].transpose(1, 0, 2)[None] for x in (q, k, v)]   # [1, H, n, d]
        o_s, l_s = attention_forward(*seq, scale, causal=causal, window_left=window_left,
                                     window_right=window_right)
        out[c0:c1] = o_s[0].transpose(1, 0, 2)
        lse[:, c0:c1] = l_s[0]
    return out, lse


def varlen_backward(q, k, v, dout, cu_seqlens, scale: float, *, causal: bool = False,
                    window_left: int = -1, window_right: int = -1):
    """dQ, dK, dV [total, H, d] of L = sum(O * dout) for ``varlen_forward``."""
    q, k, v, dout = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(dout)
    total = q.shape[0]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for c0, c1 in _segments(cu_seqlens, total):
        if c1 == c0:
            continue
        seq = [x[c0:c1].transpose(1, 0, 2)[None] for x in (q, k, v, dout)]
        g = attention_backward(*seq, scale, causal=causal, window_left=window_left,
                               window_right=window_right)
        for dst, src in zip((dq, dk, dv), g):
            dst[c0:c1] = src[0].transpose(1, 0, 2)
    return dq, dk, dv
