"""Plant plausible mistakes in copies of the oracle; the pin battery must catch every one.

Each mutant is the oracle's source with one textual change (a dropped term, a
wrong sign, index or operand), executed as a fresh module. This shows the pins
are strong enough that such a mistake in the oracle could not pass unnoticed.
"""
import os
import types

import pytest

from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

MUTANTS = {
    "fwd_scale_dropped": ("s = scale * (q_rows @ k[cols].T)", "s = (q_rows @ k[cols].T)"),
    "fwd_keys_reversed": ("s = scale * (q_rows @ k[cols].T)", "s = scale * (q_rows @ k[cols][::-1].T)"),
    "fwd_values_from_keys": ("out[:] = p @ v[cols]", "out[:] = p @ v[cols][::-1]"),
    "causal_off_by_one": ("cols[None, :] <= rows[:, None]", "cols[None, :] < rows[:, None] + 2"),
    "causal_flipped": ("cols[None, :] <= rows[:, None]", "cols[None, :] >= rows[:, None]"),
    "padding_off_by_one": ("cols[None, :] < int(kv_len_b)", "cols[None, :] <= int(kv_len_b)"),
    "block_mask_transposed": ("bm[rows[:, None] // mask_block, cols[None, :] // mask_block]",
                              "bm[cols[None, :] // mask_block, rows[:, None] // mask_block]"),
    "lse_log2": ("lse[live] = m[live] + np.log(l[live])", "lse[live] = m[live] + np.log2(l[live])"),
    "lse_missing_max": ("lse[live] = m[live] + np.log(l[live])", "lse[live] = np.log(l[live])"),
    "no_max_subtraction": ("e = np.exp(s - m_safe[:, None])", "e = np.exp(s)"),
    "normaliser_dropped": ("p = np.where(live[:, None], e / np.where(live, l, 1.0)[:, None], 0.0)\n    if drop",
                           "p = np.where(live[:, None], e, 0.0)\n    if drop"),
    "bwd_jacobian_sign": ("ds = p * (dp - (p * dp)", "ds = p * (dp + (p * dp)"),
    "bwd_jacobian_term_dropped": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "bwd_dk_scale_dropped": ("dk[b, h, cols] += scale * (ds.T @ qr)", "dk[b, h, cols] += (ds.T @ qr)"),
    "bwd_dq_scale_dropped": ("dq[b, h, rows] = scale * (ds @ kc)", "dq[b, h, rows] = (ds @ kc)"),
    "bwd_dv_wrong_operand": ("dv[b, h, cols] += (p * mm).T @ dor", "dv[b, h, cols] += (p * mm).T @ qr"),
    "bwd_dp_wrong_operand": ("dp = (dor @ vc.T) * mm", "dp = (dor @ kc.T) * mm"),
    "bwd_dk_wrong_operand": ("dk[b, h, cols] += scale * (ds.T @ qr)", "dk[b, h, cols] += scale * (ds.T @ dor)"),
    "bwd_scale_dropped_in_recompute": ("s = np.where(a, scale * (qr @ kc.T), -np.inf)",
                                       "s = np.where(a, (qr @ kc.T), -np.inf)"),
    "kvcache_causal_top_left": ("allow &= cols[None, :] <= pos[:, None]",
                                "allow &= cols[None, :] <= np.arange(Nq)[:, None]"),
    "kvcache_causal_off_by_one": ("pos = L - Nq + np.arange(Nq, dtype=np.int64)",
                                  "pos = L - Nq - 1 + np.arange(Nq, dtype=np.int64)"),
    "kvcache_length_ignored": ("allow = np.broadcast_to(cols[None, :] < L, (Nq, Nk)).copy()",
                               "allow = np.ones((Nq, Nk), dtype=bool)"),
    "bwd_causal_ignored": ("allow = allowed_pairs(rows, k.shape[2], causal=causal,\n"
                           "                                  kv_len_b=None if lens is None else lens[b],\n"
                           "                                  block_mask=block_mask, mask_block=mask_block,\n"
                           "                                  window_left=window_left, window_right=window_right)\n"
                           "            cols",
                           "allow = allowed_pairs(rows, k.shape[2], causal=False,\n"
                           "                                  kv_len_b=None if lens is None else lens[b],\n"
                           "                                  block_mask=block_mask, mask_block=mask_block,\n"
                           "                                  window_left=window_left, window_right=window_right)\n"
                           "            cols"),
    "window_left_off_by_one": ("allow &= cols[None, :] >= rows[:, None] - window_left",
                               "allow &= cols[None, :] > rows[:, None] - window_left"),
    "window_right_ignored": ("allow &= cols[None, :] <= rows[:, None] + window_right",
                             "allow &= cols[None, :] <= rows[:, None] + window_right + 10**6"),
    "window_mirrored": ("allow &= cols[None, :] >= rows[:, None] - window_left",
                        "allow &= cols[None, :] >= rows[:, None] - window_right"),
    "bwd_window_ignored": ("                                  window_left=window_left, window_right=window_right)\n"
                           "            cols",
                           "                                  window_left=-1, window_right=-1)\n"
                           "            cols"),
    "varlen_keys_shifted": ("seq = [x[c0:c1].transpose(1, 0, 2)[None] for x in (q, k, v)]",
                            "seq = [x[c0:c1].transpose(1, 0, 2)[None] for x in (q,)] + "
                            "[np.roll(x, 1, axis=0)[c0:c1].transpose(1, 0, 2)[None] for x in (k, v)]"),
    "varlen_lse_misplaced": ("lse[:, c0:c1] = l_s[0]", "lse[:, c0:c1] = l_s[0][:, ::-1]"),
    "dropout_scale_missing": ("return dropout_keep(b, h, rows, cols, dropout_seed, dropout_p) / (1.0 - dropout_p)",
                              "return dropout_keep(b, h, rows, cols, dropout_seed, dropout_p) * 1.0"),
    "dropout_word_shifted": ("np.broadcast_to(cols & 3,", "np.broadcast_to((cols + 1) & 3,"),
    "dropout_half_from_key": ("(np.uint64(16) * (rows & 1).astype(np.uint64))",
                              "(np.uint64(16) * (cols & 1).astype(np.uint64))"),
    "dropout_half_swapped": ("(np.uint64(16) * (rows & 1).astype(np.uint64))",
                             "(np.uint64(16) * ((rows + 1) & 1).astype(np.uint64))"),
    "dropout_query_pair_ignored": ("philox4x32_10(cols >> 2, rows >> 1, h, b,", "philox4x32_10(cols >> 2, rows, h, b,"),
    "dropout_counter_transposed": ("philox4x32_10(cols >> 2, rows >> 1, h, b,", "philox4x32_10(rows >> 2, cols >> 1, h, b,"),
    "dropout_threshold_flipped": ("return half >= np.uint64(threshold)", "return half < np.uint64(threshold)"),
    "dropout_heads_swapped": ("philox4x32_10(cols >> 2, rows >> 1, h, b,", "philox4x32_10(cols >> 2, rows >> 1, b, h,"),
    "philox_weyl_constant": ("_PHILOX_W = (0x9E3779B9, 0xBB67AE85)", "_PHILOX_W = (0x9E3779B9, 0xBB67AE86)"),
    "philox_output_order": ("x = [((p1 >> np.uint64(32)) ^ x[1] ^ k0) & _U32, p1 & _U32,",
                            "x = [((p1 >> np.uint64(32)) ^ x[3] ^ k0) & _U32, p1 & _U32,"),
    "fwd_dropout_ignored": ("p = p * drop[:, cols]", "p = p * 1.0"),
    "bwd_dropout_dv_unmasked": ("dv[b, h, cols] += (p * mm).T @ dor", "dv[b, h, cols] += p.T @ dor"),
    "bwd_dropout_dp_unmasked": ("dp = (dor @ vc.T) * mm", "dp = (dor @ vc.T)"),
    "bwd_rows_ignored": ("all_rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)",
                         "all_rows = np.arange(N)"),
    "bwd_heads_truncated": ("for b in range(B) for h in range(H)] if heads is None else list(heads)",
                            "for b in range(B) for h in range(H)] if heads is None else list(heads)[:1]"),
    "bwd_last_row_chunk_dropped": ("for r0 in range(0, all_rows.size, row_chunk):",
                                   "for r0 in range(0, all_rows.size - 1, row_chunk):"),
    "varlen_bwd_dk_dv_swapped": ("for dst, src in zip((dq, dk, dv), g):", "for dst, src in zip((dq, dv, dk), g):"),
}


def _mutant(old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # an assertion or a crash both count as caught
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"no pin catches mutant {name}"
