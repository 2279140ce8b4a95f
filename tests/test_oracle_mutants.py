"""Planted mistakes: a copy of the oracle with one plausible error must fail a pin.

Each mutant edits the oracle's source text on the CPU, loads it as a separate module
and runs every pin; the test passes when at least one pin rejects the mutant.  This
shows the pins constrain every part of the oracle (a dropped term, a wrong sign or
index, a transposed operand)."""
import types
from pathlib import Path

import pytest

from tests.oracle_pins import ALL_PINS

SRC = (Path(__file__).resolve().parent.parent / "oracle" / "lcv_oracle.py").read_text()

MUTANTS = {
    "rope_sign": [("out[..., c0 + 2 * p] = a * cos - b * sin", "out[..., c0 + 2 * p] = a * cos + b * sin")],
    "rope_rotate_half_pairing": [("b = x[..., c0 + 2 * p + 1]", "b = x[..., c0 + p + width // 2]"),
                                 ("out[..., c0 + 2 * p + 1] = a * sin + b * cos",
                                  "out[..., c0 + p + width // 2] = a * sin + b * cos"),
                                 ("a = x[..., c0 + 2 * p]", "a = x[..., c0 + p]"),
                                 ("out[..., c0 + 2 * p] = a * cos - b * sin", "out[..., c0 + p] = a * cos - b * sin")],
    "rope_freq_exponent": [("theta ** (-2.0 * p / width)", "theta ** (-1.0 * p / width)")],
    "rope_axes_swapped": [("((0, 16, 0), (16, 24, 1), (40, 24, 2))", "((0, 16, 0), (16, 24, 2), (40, 24, 1))")],
    "rope_section_bounds": [("((0, 16, 0), (16, 24, 1), (40, 24, 2))", "((0, 16, 0), (16, 16, 1), (32, 32, 2))")],
    "coords_row_major_swapped": [("return n // (h * w), (n // w) % h, n % w", "return n // (h * w), (n // h) % w, n % h")],
    "window_strict": [("mb = np.abs(i - j) <= local", "mb = np.abs(i - j) < local")],
    "global_offset": [("mb = mb | (j % stride == 0)", "mb = mb | (j % stride == stride - 1)")],
    "global_rows_not_cols": [("mb = mb | (j % stride == 0)", "mb = mb | (i % stride == 0)")],
    "condition_reversed": [("cond_ok = (rows[:, None] >= cond_len) | (keys[None, :] < cond_len)",
                            "cond_ok = (rows[:, None] < cond_len) | (keys[None, :] >= cond_len)")],
    "condition_dropped": [("return mb & cond_ok", "return mb")],
    "block_pair_noise_test": [("has_noise_row = last_row >= cond_len", "has_noise_row = last_row > cond_len")],
    "softmax_scale": [("SOFTMAX_SCALE = 1.0 / math.sqrt(HEAD_DIM)", "SOFTMAX_SCALE = 1.0 / HEAD_DIM")],
    "lse_base2": [("lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))",
                   "lse = np.where(empty, -np.inf, m_safe + np.log2(l_safe))")],
    "lse_missing_max": [("lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))",
                         "lse = np.where(empty, -np.inf, np.log(l_safe))")],
    "scores_use_v": [("s = (q @ k.T) * SOFTMAX_SCALE", "s = (q @ v.T) * SOFTMAX_SCALE")],
    "no_normalisation": [("out = (e @ v) / l_safe[:, None]", "out = (e @ v)")],
    "rope_transpose_sign": [("out[..., c0 + 2 * p] = a * cos + b * sin", "out[..., c0 + 2 * p] = a * cos - b * sin")],
    "prologue_bwd_no_projection": [("dx = (dn - n * np.mean(dn * n, axis=-1, keepdims=True)) / r", "dx = dn / r")],
    "prologue_bwd_dgamma_before_rotation": [("dgamma = np.sum((dy_pre * n).reshape(-1, HEAD_DIM), axis=0)",
                                             "dgamma = np.sum((np.asarray(dy) * n).reshape(-1, HEAD_DIM), axis=0)")],
    "prologue_bwd_gain_dropped": [("dn = dy_pre * gamma", "dn = dy_pre")],
    "cross_bwd_padding_ignored": [("        length = n_kv if kv_lens is None else int(kv_lens[b])\n        mask = np.broadcast_to(np.arange(n_kv)[None, :] < length, (n_q, n_kv))\n        for h in range(heads):\n            dq[b, h], dk[b, h], dv[b, h]",
                                   "        length = n_kv\n        mask = np.broadcast_to(np.arange(n_kv)[None, :] < length, (n_q, n_kv))\n        for h in range(heads):\n            dq[b, h], dk[b, h], dv[b, h]")],
    "merge_weight_not_normalised": [("out += (wgt / total_safe)[..., None] * o", "out += wgt[..., None] * o")],
    "merge_lse_without_max": [("lse = np.where(empty, -np.inf, m_safe + np.log(total_safe))",
                               "lse = np.where(empty, -np.inf, np.log(total_safe))")],
    "merge_lse_mean": [("total = np.sum(np.stack(weights), axis=0)", "total = np.mean(np.stack(weights), axis=0)")],
    "cross_padding_inclusive": [("mask = np.broadcast_to(np.arange(n_kv)[None, :] < length, (rows.size, n_kv))",
                                 "mask = np.broadcast_to(np.arange(n_kv)[None, :] <= length, (rows.size, n_kv))")],
    "cross_padding_ignored": [("length = n_kv if kv_lens is None else int(kv_lens[b])", "length = n_kv")],
    "cross_lens_of_first_item": [("length = n_kv if kv_lens is None else int(kv_lens[b])",
                                  "length = n_kv if kv_lens is None else int(kv_lens[0])")],
    "cross_rows_ignored": [("out[b, h], lse[b, h] = masked_attention(q[b, h, rows], k[b, h], v[b, h], mask)",
                            "out[b, h], lse[b, h] = masked_attention(q[b, h, :rows.size], k[b, h], v[b, h], mask)")],
    "pairs_count_cond": [("n_cond[:, None] * n_cond[None, :]", "n_cond[:, None] * size[None, :]")],
    "cached_kv_order": [("k_full = np.concatenate([np.asarray(k_cond, np.float64), np.asarray(k_noise, np.float64)], axis=2)",
                         "k_full = np.concatenate([np.asarray(k_noise, np.float64), np.asarray(k_cond, np.float64)], axis=2)")],
    "cached_q_positions": [("tokens = local_rows + cond_len", "tokens = local_rows")],
    "rmsnorm_sum_not_mean": [("mean_sq = np.mean(x * x, axis=-1, keepdims=True)",
                              "mean_sq = np.sum(x * x, axis=-1, keepdims=True)")],
    "rmsnorm_no_sqrt": [("return x / np.sqrt(mean_sq + eps) * np.asarray(gamma, dtype=np.float64)",
                         "return x / (mean_sq + eps) * np.asarray(gamma, dtype=np.float64)")],
    "rmsnorm_eps_outside": [("return x / np.sqrt(mean_sq + eps) * np.asarray(gamma, dtype=np.float64)",
                             "return x / (np.sqrt(mean_sq) + eps) * np.asarray(gamma, dtype=np.float64)")],
    "rmsnorm_wrong_axis": [("mean_sq = np.mean(x * x, axis=-1, keepdims=True)",
                            "mean_sq = np.mean(x * x, axis=0, keepdims=True)")],
    "rmsnorm_gain_inside": [("x = np.asarray(x, dtype=np.float64)\n    mean_sq",
                             "x = np.asarray(x, dtype=np.float64) * np.asarray(gamma, dtype=np.float64)\n    mean_sq")],
    "prologue_rope_first": [("return rope3d(rmsnorm(x, gamma, eps), grid, theta, token_offset)",
                             "return rmsnorm(rope3d(x, grid, theta, token_offset), gamma, eps)")],
    "prologue_no_offset": [("return rope3d(rmsnorm(x, gamma, eps), grid, theta, token_offset)",
                            "return rope3d(rmsnorm(x, gamma, eps), grid, theta, 0)")],
    "blocks_drop_last_column": [("cols = col_idx[row_ptr[i]:row_ptr[i + 1]]", "cols = col_idx[row_ptr[i]:row_ptr[i + 1] - 1]")],
    "blocks_row_of_next_block": [("cols = col_idx[row_ptr[i]:row_ptr[i + 1]]",
                                  "cols = col_idx[row_ptr[min(i + 1, n - 1)]:row_ptr[min(i + 1, n - 1) + 1]]")],
    "blocks_no_condition_mask": [("mask = token_mask(rows, keys, cond_len, local, stride)",
                                  "mask = np.ones((rows.size, keys.size), dtype=bool)")],
    "bwd_delta_sign": [("ds = p * (dp - delta[:, None])", "ds = p * (dp + delta[:, None])")],
    "bwd_delta_dropped": [("ds = p * (dp - delta[:, None])", "ds = p * dp")],
    "bwd_dq_scale": [("dq = (ds @ k) * SOFTMAX_SCALE", "dq = ds @ k")],
    "bwd_dk_uses_k": [("dk = (ds.T @ q) * SOFTMAX_SCALE", "dk = (ds.T @ k) * SOFTMAX_SCALE")],
    "bwd_dv_no_transpose": [("dv = p.T @ dout", "dv = p @ dout")],
    "bwd_dp_uses_q": [("dp = dout @ v.T", "dp = dout @ q.T")],
    "bwd_unnormalised_p": [("p = e / np.where(empty, 1.0, l)[:, None]", "p = e")],
}


def _load_mutant(name):
    src = SRC
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation anchor not found: {old}"
        src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"oracle_mutant_{name}", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _load_mutant(name)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin rejects the planted mistake {name}"
