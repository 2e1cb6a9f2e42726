"""Each plausible mistake planted in a copy of the oracle must fail a pin.

The mistakes are planted on the CPU, in a private copy of the oracle's source
text; the real oracle module is never modified.  A mutation "fails a pin"
when at least one check raises.
"""
import types
from pathlib import Path

import pytest

from oracle_pins import ALL_CHECKS

SRC = (Path(__file__).resolve().parent.parent / "oracle" / "gqa_oracle.py").read_text()

MUTATIONS = {
    "interleaved_group_map": [
        ("Qg = q[b, k * G:(k + 1) * G, :]", "Qg = q[b, k::K, :]"),
        ("out[b, k * G:(k + 1) * G, :] = p @ Vc", "out[b, k::K, :] = p @ Vc")],
    "kv_head_of_modulo": [("return h // (H // K)", "return h % K")],
    "weights_group_map": [("k_cache[b, h // G, :L, :]", "k_cache[b, h % K, :L, :]")],
    "decode_length_short": [("k_cache[b, k, :L, :]", "k_cache[b, k, :max(L - 1, 1), :]"),
                            ("v_cache[b, k, :L, :]", "v_cache[b, k, :max(L - 1, 1), :]")],
    "decode_length_long": [("k_cache[b, k, :L, :]", "k_cache[b, k, :L + 1, :]"),
                           ("v_cache[b, k, :L, :]", "v_cache[b, k, :L + 1, :]")],
    "decode_scale_dropped": [("p = _softmax_rows(float(scale) * (Qg @ Kc.T))",
                              "p = _softmax_rows(Qg @ Kc.T)")],
    "decode_scale_sqrt": [("p = _softmax_rows(float(scale) * (Qg @ Kc.T))",
                           "p = _softmax_rows(float(scale) ** 0.5 * (Qg @ Kc.T))")],
    "decode_values_are_keys": [("out[b, k * G:(k + 1) * G, :] = p @ Vc",
                                "out[b, k * G:(k + 1) * G, :] = p @ Kc")],
    "softmax_wrong_axis": [("s = s - s.max(axis=-1, keepdims=True)", "s = s - s.max(axis=0, keepdims=True)"),
                           ("return e / e.sum(axis=-1, keepdims=True)", "return e / e.sum(axis=0, keepdims=True)")],
    "softmax_unnormalised": [("return e / e.sum(axis=-1, keepdims=True)", "return e")],
    "softmax_sign_flip": [("e = np.exp(s)", "e = np.exp(-s)")],
    "causal_strict": [("keep = np.arange(S)[None, :] <= rows[:, None]",
                       "keep = np.arange(S)[None, :] < rows[:, None]")],
    "causal_reversed": [("keep = np.arange(S)[None, :] <= rows[:, None]",
                         "keep = np.arange(S)[None, :] >= rows[:, None]")],
    "causal_no_mask": [("s = np.where(keep, s, -np.inf)", "s = s")],
    "prefill_group_map": [("for h in range(g * G, (g + 1) * G):", "for h in range(g, H, K):")],
    "prefill_values_are_keys": [("out[b, h] = _softmax_rows(s) @ Vc", "out[b, h] = _softmax_rows(s) @ Kc")],
    "prefill_scale_dropped": [("s = float(scale) * (q[b, h, rows, :] @ Kc.T)", "s = q[b, h, rows, :] @ Kc.T")],
    "meanpool_interleaved": [("return src.reshape(outer, K, G, inner).mean(axis=2)",
                              "return src.reshape(outer, G, K, inner).mean(axis=1)")],
    "meanpool_first_head": [("return src.reshape(outer, K, G, inner).mean(axis=2)",
                             "return src.reshape(outer, K, G, inner)[:, :, 0, :]")],
    "meanpool_sum": [("return src.reshape(outer, K, G, inner).mean(axis=2)",
                      "return src.reshape(outer, K, G, inner).sum(axis=2)")],
    "kv_bytes_no_factor_two": [("return 2 * int(layers)", "return int(layers)")],
    "kv_bytes_query_heads": [("return 2 * int(layers) * int(kv_heads)", "return 2 * int(layers) * int(kv_heads) * 4")],
    "append_wrong_row": [("kc[b, :, L, :] = k_new[b]", "kc[b, :, max(L - 1, 0), :] = k_new[b]")],
    "append_no_increment": [("sl[b] = L + 1", "sl[b] = L")],
    "append_v_from_k": [("vc[b, :, L, :] = v_new[b]", "vc[b, :, L, :] = k_new[b]")],
    "append_full_cache": [("if L >= S_max:\n            continue", "if L > S_max:\n            continue")],
    "paged_row_from_block_index": [("out[b, :, j, :] = pool[n, :, j % bs, :]",
                                    "out[b, :, j, :] = pool[n, :, j // bs, :]")],
    "paged_table_by_row": [("n = int(block_table[b, j // bs])", "n = int(block_table[b, j % bs])")],
    "paged_table_transposed": [("n = int(block_table[b, j // bs])",
                                "n = int(block_table.ravel()[(j // bs) * B + b])")],
    "paged_v_gathered_from_k": [("vc = paged_gather_ref(v_pool, block_table, seq_lens)",
                                 "vc = paged_gather_ref(k_pool, block_table, seq_lens)")],
    "paged_append_row": [("kp[n, :, L % bs, :] = k_new[b]", "kp[n, :, L // bs, :] = k_new[b]")],
    "paged_append_block": [("n = int(block_table[b, L // bs])", "n = int(block_table[b, L % max_blocks])")],
    "paged_append_no_increment": [("        vp[n, :, L % bs, :] = v_new[b]\n        sl[b] = L + 1",
                                   "        vp[n, :, L % bs, :] = v_new[b]")],
    "paged_append_ignores_bad_id": [("        if not 0 <= n < num_blocks:\n            continue\n        kp",
                                     "        n = n % num_blocks\n        kp")],
    "int8_scale_over_128": [("scales[nz] = amax[nz] / np.float32(127)", "scales[nz] = amax[nz] / np.float32(128)")],
    "int8_inv_128": [("inv = np.float32(127) / amax[nz]", "inv = np.float32(128) / amax[nz]")],
    "int8_truncate": [("c = np.rint(x[nz] * inv[..., None])", "c = np.trunc(x[nz] * inv[..., None])")],
    "int8_round_half_up": [("c = np.rint(x[nz] * inv[..., None])", "c = np.floor(x[nz] * inv[..., None] + 0.5)")],
    "int8_per_tensor_amax": [("amax = np.max(np.abs(x), axis=-1)",
                              "amax = np.full(x.shape[:-1], np.max(np.abs(x)), dtype=np.float32)")],
    "int8_v_uses_k_scales": [("dequantize_int8_ref(v_codes, v_scales), seq_lens, scale)",
                              "dequantize_int8_ref(v_codes, k_scales), seq_lens, scale)")],
    "int8_dequant_ignores_scale": [("return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]",
                                    "return np.asarray(codes, dtype=np.float64) / 127.0")],
    "int8_append_unquantised": [("        kc[b, :, L, :] = kq[b]\n", "        kc[b, :, L, :] = k_new[b]\n")],
    "int8_append_scale_swapped": [("        ks[b, :, L] = kqs[b]\n", "        ks[b, :, L] = vqs[b]\n")],
    "chunk_offset_plus_one": [("pos = L - Sq + np.arange(Sq)", "pos = L - Sq + 1 + np.arange(Sq)")],
    "chunk_offset_from_zero": [("pos = L - Sq + np.arange(Sq)", "pos = np.arange(Sq)")],
    "chunk_strict_mask": [("keep = np.arange(L)[None, :] <= pos[:, None]", "keep = np.arange(L)[None, :] < pos[:, None]")],
    "cross_causal": [("keep = np.ones((Sq, L), dtype=bool)", "keep = np.arange(L)[None, :] <= np.arange(Sq)[:, None]")],
    "cross_drops_last_row": [("Kc = np.asarray(k[b, g, :L, :], dtype=np.float64)",
                              "Kc = np.asarray(k[b, g, :max(L - 1, 0), :], dtype=np.float64)"),
                             ("Vc = np.asarray(v[b, g, :L, :], dtype=np.float64)",
                              "Vc = np.asarray(v[b, g, :max(L - 1, 0), :], dtype=np.float64)"),
                             ("keep = np.ones((Sq, L), dtype=bool)", "keep = np.ones((Sq, max(L - 1, 0)), dtype=bool)")],
    "cross_group_interleaved": [("        keep = np.ones((Sq, L), dtype=bool)\n        for g in range(K):\n            Kc = np.asarray(k[b, g, :L, :], dtype=np.float64)\n            Vc = np.asarray(v[b, g, :L, :], dtype=np.float64)\n            for h in range(g * G, (g + 1) * G):",
                                 "        keep = np.ones((Sq, L), dtype=bool)\n        for g in range(K):\n            Kc = np.asarray(k[b, g, :L, :], dtype=np.float64)\n            Vc = np.asarray(v[b, g, :L, :], dtype=np.float64)\n            for h in range(g, H, K):")],
    "attend_rows_unmasked": [("    s = np.where(keep, s, -np.inf)\n    has", "    has")],
    "append_rows_partial": [("        if L + T > S_max:\n            continue\n        kc[b, :, L:L + T, :] = k_new[b]",
                             "        if L >= S_max:\n            continue\n        T2 = min(T, S_max - L)\n        kc[b, :, L:L + T2, :] = k_new[b, :, :T2]")],
    "append_rows_no_increment": [("        sl[b] = L + T\n", "        sl[b] = L + 1\n")],
    "project_k_v_swapped": [("    return y[..., :d], y[..., d:]", "    return y[..., d:], y[..., :d]")],
    "project_transposed_weight": [('y = np.einsum("btm,kjm->bktj", x, w)', 'y = np.einsum("btm,kjm->bktj", x, w[:, ::-1, :])')],
    "project_heads_interleaved": [('y = np.einsum("btm,kjm->bktj", x, w)',
                                   'y = np.einsum("btm,kjm->bktj", x, w.reshape(2, K, d, dm).transpose(1, 0, 2, 3).reshape(K, 2 * d, dm))')],
    "merge_without_rescale": [("    num = (w[..., None] * acc).sum(axis=-2)", "    num = acc.sum(axis=-2)")],
    "merge_unweighted_denominator": [("    den = (w * l).sum(axis=-1)", "    den = l.sum(axis=-1)")],
    "partials_unshifted_sum": [("                l[b, h, p] = e.sum()", "                l[b, h, p] = np.exp(s).sum()")],
    "partials_end_inclusive": [("                t0, t1 = max(t0, 0), min(t1, L)", "                t0, t1 = max(t0, 0), min(t1 + 1, L)")],
    "empty_length_nan": [("        if L == 0:\n            continue\n        for k in range(K):",
                          "        for k in range(K):")],
}


def _mutant(edits):
    src = SRC
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(MUTATIONS[name])
    caught = []
    for check in ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as detection
            caught.append(f"{check.__name__}: {type(e).__name__}")
    assert caught, f"mutation {name} passed every pin"
