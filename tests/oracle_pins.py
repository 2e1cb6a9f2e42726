"""Pins of the CPU oracle against facts that do not come from the oracle.

Every ``check_*`` takes the oracle module ``O`` as its argument (so that the
mutation tests can hand it a copy with a planted mistake) and raises
AssertionError (or any exception) when the oracle disagrees with:

* numbers the pages print (KV-cache bytes, tests/golden/kv_cache_bytes.json);
* a pure-Python brute force written from the 1-based group formula;
* torch's fp64 CPU scaled_dot_product_attention (a library special case:
  pinghaoyang.com.cn "GQA 完全拆解", section 工程实现 (engineering), names
  PyTorch SDPA with fewer KV heads than query heads);
* closed forms (softmax of known scores, one cached row, zero query, constant
  values, prefix means, identical heads under mean pooling);
* invariants the pages state (K = H is MHA and K = 1 is MQA; expanding each
  KV head G times and running MHA gives GQA; incremental decode equals the
  last row of causal attention; weight pooling commutes with projection).
"""
from __future__ import annotations

import json
import math
from pathlib import Path

import numpy as np
import torch

from oracle import bruteforce as BF

GOLDEN = Path(__file__).resolve().parent / "golden"


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_decode(seed, B, H, K, d, lens, s_max=None, nan_tail=True):
    r = _rng(seed)
    s_max = s_max or (max(lens) + 1)
    q = r.standard_normal((B, H, d))
    kc = r.standard_normal((B, K, s_max, d))
    vc = r.standard_normal((B, K, s_max, d))
    if nan_tail:
        for b, L in enumerate(lens):
            kc[b, :, L:] = np.nan
            vc[b, :, L:] = np.nan
    return q, kc, vc, np.array(lens)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------
# numbers printed on the pages
# --------------------------------------------------------------------------
def check_kv_bytes_golden(O):
    data = json.loads((GOLDEN / "kv_cache_bytes.json").read_text())
    for e in data["entries"]:
        got = O.kv_cache_bytes(e["layers"], e["kv_heads"], e["head_dim"], e["elem_bytes"], e["tokens"])
        if "exact_bytes" in e:
            assert got == e["exact_bytes"], (e["what"], got)
        else:
            val = round(got / e["unit_bytes"], e["round_to"])
            assert val == e["approx"], (e["what"], got, val)
    for r in data["ratios"]:
        full = O.kv_cache_bytes(80, r["mha_kv_heads"], 128, 2, 2048)
        grp = O.kv_cache_bytes(80, r["gqa_kv_heads"], 128, 2, 2048)
        assert grp / full == r["ratio"], r["what"]


def check_kv_head_map(O):
    for H, K in [(8, 2), (16, 4), (6, 3), (56, 8), (71, 1), (5, 5)]:
        for h in range(H):
            assert O.kv_head_of(h, H, K) == BF.group_of_head(h + 1, H, K) - 1, (H, K, h)


# --------------------------------------------------------------------------
# brute force on tiny inputs
# --------------------------------------------------------------------------
def check_bruteforce_decode(O):
    for seed, (B, H, K, d, lens) in enumerate([
            (2, 6, 3, 4, [5, 1]), (1, 8, 2, 3, [7]), (2, 4, 4, 5, [3, 0]),
            (1, 5, 1, 4, [6]), (2, 9, 3, 2, [2, 9])]):
        q, kc, vc, sl = _rand_decode(100 + seed, B, H, K, d, lens)
        ref = BF.decode_bruteforce(q.tolist(), kc.tolist(), vc.tolist(), sl.tolist(), 0.37)
        _close(O.decode_ref(q, kc, vc, sl, 0.37), ref, 1e-13, f"decode brute force {seed}")


def check_bruteforce_prefill(O):
    for seed, (B, H, K, S, d) in enumerate([(1, 4, 2, 5, 3), (2, 6, 3, 4, 2), (1, 3, 1, 6, 4)]):
        r = _rng(200 + seed)
        q = r.standard_normal((B, H, S, d))
        k = r.standard_normal((B, K, S + 2, d))
        v = r.standard_normal((B, K, S + 2, d))
        k[:, :, S:] = np.nan
        v[:, :, S:] = np.nan
        ref = BF.prefill_bruteforce(q.tolist(), k[:, :, :S].tolist(), v[:, :, :S].tolist(), 0.6)
        _close(O.prefill_causal_ref(q, k, v, 0.6), ref, 1e-13, f"prefill brute force {seed}")


def check_bruteforce_meanpool(O):
    for seed, (outer, H, K, inner) in enumerate([(2, 6, 3, 5), (1, 8, 2, 3), (3, 4, 4, 2), (1, 7, 1, 4)]):
        src = _rng(300 + seed).standard_normal((outer, H, inner))
        _close(O.meanpool_convert_ref(src, K), BF.meanpool_bruteforce(src.tolist(), K), 1e-14,
               f"meanpool brute force {seed}")


# --------------------------------------------------------------------------
# library special case: torch fp64 CPU SDPA
# --------------------------------------------------------------------------
def _sdpa(q, k, v, scale, causal=False, gqa=True):
    F = torch.nn.functional
    return F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=scale, enable_gqa=gqa).numpy()


def check_sdpa_decode(O):
    for seed, (B, H, K, d, lens) in enumerate([(3, 32, 8, 16, [40, 1, 17]), (2, 12, 4, 8, [9, 33])]):
        q, kc, vc, sl = _rand_decode(400 + seed, B, H, K, d, lens)
        got = O.decode_ref(q, kc, vc, sl, 0.25)
        for b, L in enumerate(lens):
            ref = _sdpa(q[b][None, :, None, :], kc[b][None, :, :L], vc[b][None, :, :L], 0.25)
            _close(got[b], ref[0, :, 0, :], 1e-12, f"SDPA decode b={b}")


def check_sdpa_prefill(O):
    r = _rng(500)
    B, H, K, S, d = 2, 8, 2, 24, 8
    q = r.standard_normal((B, H, S, d))
    k = r.standard_normal((B, K, S, d))
    v = r.standard_normal((B, K, S, d))
    _close(O.prefill_causal_ref(q, k, v, 0.3), _sdpa(q, k, v, 0.3, causal=True), 1e-12, "SDPA prefill")
    rows = [0, 5, 23]
    _close(O.prefill_causal_ref(q, k, v, 0.3, rows=rows),
           _sdpa(q, k, v, 0.3, causal=True)[:, :, rows], 1e-12, "SDPA prefill rows")


def check_mha_special_case(O):
    """K = H: every query head has its own KV head (plain multi-head)."""
    q, kc, vc, sl = _rand_decode(600, 2, 6, 6, 8, [11, 4])
    got = O.decode_ref(q, kc, vc, sl, 0.5)
    for b, L in enumerate(sl):
        ref = _sdpa(q[b][None, :, None, :], kc[b][None, :, :L], vc[b][None, :, :L], 0.5, gqa=False)
        _close(got[b], ref[0, :, 0, :], 1e-12, "MHA special case")


def check_mqa_special_case(O):
    """K = 1: all query heads share one K/V head, which has no head axis
    (pinghaoyang.com.cn 'GQA 完全拆解', MQA section: [b, n, d_k])."""
    q, kc, vc, sl = _rand_decode(700, 2, 7, 1, 8, [13, 2])
    got = O.decode_ref(q, kc, vc, sl, 0.5)
    for b, L in enumerate(sl):
        kk = np.broadcast_to(kc[b, 0, :L], (7, L, 8)).copy()[None]
        vv = np.broadcast_to(vc[b, 0, :L], (7, L, 8)).copy()[None]
        ref = _sdpa(q[b][None, :, None, :], kk, vv, 0.5, gqa=False)
        _close(got[b], ref[0, :, 0, :], 1e-12, "MQA special case")


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def check_expanded_kv_equivalence(O):
    """GQA equals MHA on KV heads materialised G times each (the repeat_kv
    route described in the engineering section), with explicit copies."""
    B, H, K, d = 2, 12, 3, 8
    q, kc, vc, sl = _rand_decode(800, B, H, K, d, [10, 6])
    G = H // K
    kx = np.empty((B, H) + kc.shape[2:])
    vx = np.empty((B, H) + vc.shape[2:])
    for h in range(H):
        kx[:, h] = kc[:, h // G]
        vx[:, h] = vc[:, h // G]
    _close(O.decode_ref(q, kc, vc, sl, 0.4), O.decode_ref(q, kx, vx, sl, 0.4), 1e-13,
           "expanded-KV equivalence")


def check_identical_heads_meanpool(O):
    """An MHA cache whose heads are identical within each group gives the
    same outputs as GQA on the mean-pooled cache, and mean pooling returns
    that shared head exactly."""
    B, H, K, d, L = 2, 8, 2, 6, 9
    r = _rng(900)
    base_k = r.standard_normal((B, K, L, d))
    base_v = r.standard_normal((B, K, L, d))
    G = H // K
    kx = np.repeat(base_k, G, axis=1)
    vx = np.repeat(base_v, G, axis=1)
    q = r.standard_normal((B, H, d))
    pooled_k = O.meanpool_convert_ref(kx.transpose(0, 2, 1, 3).reshape(B * L, H, d), K)
    pooled_k = pooled_k.reshape(B, L, K, d).transpose(0, 2, 1, 3)
    pooled_v = O.meanpool_convert_ref(vx.transpose(0, 2, 1, 3).reshape(B * L, H, d), K)
    pooled_v = pooled_v.reshape(B, L, K, d).transpose(0, 2, 1, 3)
    assert np.array_equal(pooled_k, base_k) and np.array_equal(pooled_v, base_v)
    sl = np.array([L, L - 3])
    _close(O.decode_ref(q, pooled_k, pooled_v, sl, 0.3), O.decode_ref(q, kx, vx, sl, 0.3), 1e-13,
           "identical heads vs MHA")


def check_softmax_closed_form(O):
    """Known scores: with q = e0, k_j = (ln(j+1)/scale) e0 the scores are
    ln(j+1), so p_j = (j+1) / sum(1..L) exactly; one-hot value rows make the
    output equal to p, which must also sum to one."""
    L, d, scale = 7, 8, 0.125
    q = np.zeros((1, 2, d))
    q[0, :, 0] = 1.0
    kc = np.zeros((1, 1, L, d))
    vc = np.zeros((1, 1, L, d))
    for j in range(L):
        kc[0, 0, j, 0] = math.log(j + 1) / scale
        vc[0, 0, j, j] = 1.0
    want = np.array([(j + 1) / (L * (L + 1) / 2) for j in range(L)] + [0.0] * (d - L))
    out = O.decode_ref(q, kc, vc, [L], scale)
    _close(out[0, 0], want, 1e-15, "closed-form softmax")
    _close(out[0, 1], want, 1e-15, "closed-form softmax head 1")
    w = O.decode_weights_ref(q, kc, [L], scale)
    _close(w[0][0], want[:L], 1e-15, "weights closed form")
    assert abs(math.fsum(w[0][1]) - 1.0) < 1e-15


def check_weights_sum_to_one(O):
    q, kc, vc, sl = _rand_decode(1000, 2, 8, 2, 8, [12, 3])
    for row in O.decode_weights_ref(q, kc, sl, 0.7):
        for p in row:
            assert np.all(p >= 0) and abs(math.fsum(p) - 1.0) < 1e-14


def check_weights_sdpa(O):
    """The weights equal SDPA's output when the value rows are the identity."""
    q, kc, vc, sl = _rand_decode(1050, 2, 8, 4, 6, [5, 3])
    w = O.decode_weights_ref(q, kc, sl, 0.6)
    for b, L in enumerate(sl):
        eye = np.broadcast_to(np.eye(L), (4, L, L)).copy()[None]
        ref = _sdpa(q[b][None, :, None, :], kc[b][None, :, :L], eye, 0.6)[0, :, 0, :]
        _close(np.stack(w[b]), ref, 1e-13, "weights vs SDPA")


def check_single_row(O):
    """L = 1: the softmax has one term, so the output is that value row exactly."""
    q, kc, vc, sl = _rand_decode(1100, 3, 8, 4, 8, [1, 1, 1])
    out = O.decode_ref(q, kc, vc, sl, 0.3)
    for b in range(3):
        for h in range(8):
            assert np.array_equal(out[b, h], vc[b, h // 2, 0])


def check_zero_query_mean(O):
    """q = 0: all scores equal, so the output is the mean of rows [0, L)."""
    q, kc, vc, sl = _rand_decode(1200, 2, 6, 3, 5, [17, 4], s_max=20)
    q[:] = 0.0
    out = O.decode_ref(q, kc, vc, sl, 0.9)
    for b, L in enumerate(sl):
        for h in range(6):
            _close(out[b, h], vc[b, h // 2, :L].mean(axis=0), 1e-14, "zero-query mean")


def check_constant_values(O):
    q, kc, vc, sl = _rand_decode(1300, 2, 4, 2, 6, [9, 5])
    c = _rng(1301).standard_normal(6)
    for b, L in enumerate(sl):
        vc[b, :, :L] = c
    out = O.decode_ref(q, kc, vc, sl, 1.1)
    _close(out, np.broadcast_to(c, out.shape), 1e-14, "constant values")


def check_empty_length(O):
    q, kc, vc, sl = _rand_decode(1400, 2, 4, 2, 4, [0, 3])
    out = O.decode_ref(q, kc, vc, sl, 0.5)
    assert np.array_equal(out[0], np.zeros((4, 4))) and np.all(np.isfinite(out[1]))


def check_incremental_equals_causal(O):
    """Appending token i and then decoding it reproduces causal row i."""
    r = _rng(1500)
    B, H, K, S, d = 2, 6, 2, 9, 4
    q = r.standard_normal((B, H, S, d))
    k = r.standard_normal((B, K, S, d))
    v = r.standard_normal((B, K, S, d))
    full = O.prefill_causal_ref(q, k, v, 0.45)
    kc = np.full((B, K, S, d), np.nan)
    vc = np.full((B, K, S, d), np.nan)
    sl = np.zeros(B, dtype=np.int64)
    for i in range(S):
        kc, vc, sl = O.kv_append_ref(k[:, :, i], v[:, :, i], kc, vc, sl)
        assert list(sl) == [i + 1] * B
        _close(O.decode_ref(q[:, :, i], kc, vc, sl, 0.45), full[:, :, i], 1e-13,
               f"incremental row {i}")


def check_prefill_closed_forms(O):
    r = _rng(1600)
    B, H, K, S, d = 1, 4, 2, 8, 3
    q = r.standard_normal((B, H, S, d))
    k = r.standard_normal((B, K, S, d))
    v = r.standard_normal((B, K, S, d))
    out = O.prefill_causal_ref(q, k, v, 0.8)
    for h in range(H):
        assert np.array_equal(out[0, h, 0], v[0, h // 2, 0]), "row 0 must equal V_0"
    out0 = O.prefill_causal_ref(np.zeros_like(q), k, v, 0.8)
    for h in range(H):
        for i in range(S):
            _close(out0[0, h, i], v[0, h // 2, :i + 1].mean(axis=0), 1e-14, "prefix mean")


def check_append_semantics(O):
    r = _rng(1700)
    B, K, S_max, d = 3, 2, 5, 4
    kc = r.integers(-30000, 30000, (B, K, S_max, d), dtype=np.int16)
    vc = r.integers(-30000, 30000, (B, K, S_max, d), dtype=np.int16)
    kn = r.integers(-30000, 30000, (B, K, d), dtype=np.int16)
    vn = r.integers(-30000, 30000, (B, K, d), dtype=np.int16)
    sl = np.array([0, 3, S_max])
    k2, v2, s2 = O.kv_append_ref(kn, vn, kc, vc, sl)
    assert list(s2) == [1, 4, S_max]
    for b, L in enumerate(sl):
        for pos in range(S_max):
            if pos == L:
                assert np.array_equal(k2[b, :, pos], kn[b]) and np.array_equal(v2[b, :, pos], vn[b])
            else:
                assert np.array_equal(k2[b, :, pos], kc[b, :, pos])
                assert np.array_equal(v2[b, :, pos], vc[b, :, pos])
    assert list(sl) == [0, 3, S_max], "inputs must not be modified"


def check_meanpool_linearity(O):
    """Pooling the per-head key projections W_K [H, d_k, d_model] and then
    projecting X equals projecting X with every head and pooling the results
    (the einsum 'bd,hdk->bhk' form of the MQA section)."""
    r = _rng(1800)
    H, K, dk, dm, n = 8, 2, 5, 7, 3
    W = r.standard_normal((H, dm, dk))
    X = r.standard_normal((n, dm))
    per_head = np.einsum("bd,hdk->bhk", X, W)                  # [n, H, dk]
    pooled_after = O.meanpool_convert_ref(per_head, K)          # [n, K, dk]
    Wp = O.meanpool_convert_ref(W.reshape(1, H, dm * dk), K).reshape(K, dm, dk)
    pooled_before = np.einsum("bd,hdk->bhk", X, Wp)
    _close(pooled_after, pooled_before, 1e-12, "meanpool linearity")


def check_meanpool_identity_g1(O):
    src = _rng(1900).standard_normal((3, 5, 4))
    assert np.array_equal(O.meanpool_convert_ref(src, 5), src)


# --------------------------------------------------------------------------
# paged KV cache
# --------------------------------------------------------------------------
def _paged_from_contiguous(cache, bs):
    """Cut a contiguous cache [B, K, S, d] into blocks of ``bs`` positions:
    block b * (S // bs) + i holds positions [i * bs, (i + 1) * bs) of
    sequence b, so the identity table arange(B * S // bs) maps back."""
    B, K, S, d = cache.shape
    mb = S // bs
    pool = cache.reshape(B, K, mb, bs, d).transpose(0, 2, 1, 3, 4).reshape(B * mb, K, bs, d)
    return pool, np.arange(B * mb, dtype=np.int32).reshape(B, mb)


def check_paged_worked_example(O):
    g = json.loads((GOLDEN / "paged_gather_example.json").read_text())
    bs = g["block_size"]
    pool = np.array(g["pool_markers"], dtype=np.float64).reshape(g["num_blocks"], 1, bs, 1)
    table = np.array(g["block_table"], dtype=np.int32)
    got = O.paged_gather_ref(pool, table, np.array(g["seq_lens"]))
    for b, want in enumerate(g["gathered"]):
        assert list(got[b, 0, :len(want), 0]) == want, f"sequence {b}: {got[b, 0, :, 0]}"
        assert np.all(np.isnan(got[b, 0, len(want):, 0]))
    a = g["append"]
    pool_i = np.array(g["pool_markers"], dtype=np.int32).reshape(g["num_blocks"], 1, bs, 1)
    new = np.full((2, 1, 1), 99, dtype=np.int32)
    kp, vp, sl = O.kv_append_paged_ref(new, new, pool_i, pool_i, table, np.array(a["seq_lens"]))
    assert list(sl) == a["new_seq_lens"]
    assert kp[:, 0, :, 0].tolist() == a["pool_after"] and vp[:, 0, :, 0].tolist() == a["pool_after"]


def check_paged_identity_table(O):
    """A pool cut from a contiguous cache, read through the identity table,
    is that cache: the gather returns it and decode matches the brute force."""
    B, H, K, d, bs = 2, 4, 2, 3, 2
    lens = [5, 8]
    q, kc, vc, sl = _rand_decode(2000, B, H, K, d, lens, s_max=8, nan_tail=False)
    kp, table = _paged_from_contiguous(kc, bs)
    vp, _ = _paged_from_contiguous(vc, bs)
    g = O.paged_gather_ref(kp, table, sl)
    for b, L in enumerate(lens):
        assert np.array_equal(g[b, :, :L], kc[b, :, :L])
    ref = BF.decode_bruteforce(q.tolist(), kc.tolist(), vc.tolist(), lens, 0.7)
    _close(O.decode_paged_ref(q, kp, vp, table, sl, 0.7), ref, 1e-13, "paged decode vs brute force")


def check_paged_block_permutation(O):
    """Relabelling physical blocks (and the table with them) changes nothing;
    two sequences sharing one table give identical rows."""
    r = _rng(2100)
    B, H, K, d, bs, nb, mb = 3, 6, 3, 4, 4, 9, 3
    kp = r.standard_normal((nb, K, bs, d))
    vp = r.standard_normal((nb, K, bs, d))
    q = r.standard_normal((B, H, d))
    q[2] = q[0]
    table = np.array([[4, 0, 7], [2, 2, 5], [4, 0, 7]], dtype=np.int32)
    sl = np.array([10, 9, 10])
    out = O.decode_paged_ref(q, kp, vp, table, sl, 0.5)
    assert np.array_equal(out[0], out[2])
    perm = r.permutation(nb)                         # new id of old block n is perm[n]
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    out2 = O.decode_paged_ref(q, kp2, vp2, perm[table].astype(np.int32), sl, 0.5)
    _close(out2, out, 1e-15, "block relabelling")
    # sequence 1 reads block 2 twice: rows [0, 4) and [4, 8) are the same
    g = O.paged_gather_ref(kp, table, sl)
    assert np.array_equal(g[1, :, 0:4], g[1, :, 4:8]) and np.array_equal(g[1, :, 8], kp[5, :, 0])


def check_paged_append_identity(O):
    """Appending through the identity table is the contiguous append, full
    tables and invalid block ids are left alone."""
    r = _rng(2200)
    B, K, S, d, bs = 3, 2, 8, 4, 4
    kc = r.integers(-30000, 30000, (B, K, S, d), dtype=np.int16)
    vc = r.integers(-30000, 30000, (B, K, S, d), dtype=np.int16)
    kn = r.integers(-30000, 30000, (B, K, d), dtype=np.int16)
    vn = r.integers(-30000, 30000, (B, K, d), dtype=np.int16)
    sl = np.array([3, 4, S])
    k2, v2, s2 = O.kv_append_ref(kn, vn, kc, vc, sl)
    kp, table = _paged_from_contiguous(kc, bs)
    vp, _ = _paged_from_contiguous(vc, bs)
    kp2, vp2, sp2 = O.kv_append_paged_ref(kn, vn, kp, vp, table, sl)
    assert list(sp2) == list(s2) == [4, 5, S]
    assert np.array_equal(kp2, _paged_from_contiguous(k2, bs)[0])
    assert np.array_equal(vp2, _paged_from_contiguous(v2, bs)[0])
    bad = table.copy()
    bad[1, 1] = -1
    kp3, _, sp3 = O.kv_append_paged_ref(kn, vn, kp, vp, bad, sl)
    assert sp3[1] == 4 and np.array_equal(kp3[table[1, 1]], kp[table[1, 1]])


# --------------------------------------------------------------------------
# int8 KV cache
# --------------------------------------------------------------------------
def check_int8_exact_grid(O):
    """Rows on the quantisation grid come back exactly: x = c * 0.5 with
    max |c| = 127 gives inv = 2, codes c and scale 0.5."""
    c = np.array([[127, -64, 0, 1, -127, 3, 100, -1]], dtype=np.int8)
    x = c.astype(np.float32) * np.float32(0.5)
    codes, scales = O.quantize_int8_ref(x)
    assert np.array_equal(codes, c) and scales.dtype == np.float32 and scales[0] == np.float32(0.5)
    assert np.array_equal(O.dequantize_int8_ref(codes, scales), x.astype(np.float64))


def check_int8_ties_to_even(O):
    """amax = 127 makes inv = 1, so x itself is rounded: ties go to even."""
    x = np.array([[127.0, 2.5, -2.5, 3.5, 0.5, -0.5, 1.5, 126.5]], dtype=np.float32)
    codes, scales = O.quantize_int8_ref(x)
    assert codes[0].tolist() == [127, 2, -2, 4, 0, 0, 2, 126]
    assert scales[0] == np.float32(1.0)


def check_int8_bounds_and_invariants(O):
    r = _rng(2300)
    x = (r.standard_normal((5, 7, 64)) * r.uniform(0.01, 100, (5, 7, 1))).astype(np.float32)
    x[1, 2] = 0.0
    codes, scales = O.quantize_int8_ref(x)
    assert codes.dtype == np.int8 and scales.shape == (5, 7)
    deq = O.dequantize_int8_ref(codes, scales)
    err = np.abs(deq - x.astype(np.float64))
    # half a step, plus float32 rounding of inv, the product and the scale
    assert np.all(err <= scales[..., None].astype(np.float64) * (0.5 + 1e-5) + 1e-30)
    amax = np.abs(x).max(axis=-1)
    nz = amax > 0
    assert np.all(np.abs(codes.astype(np.int32)).max(axis=-1)[nz] == 127)
    assert np.all(codes[1, 2] == 0) and scales[1, 2] == 0
    assert np.allclose(scales[nz], amax[nz] / 127.0, rtol=1e-6)
    # powers of two change the scale, not the codes
    c2, s2 = O.quantize_int8_ref(x * np.float32(8.0))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales * np.float32(8.0))
    assert np.array_equal(O.quantize_int8_ref(-x)[0], -codes)


def check_int8_halves_cache(O):
    """aicoding.csdn.net, section 3 (deployment tips): 8-bit KV quantisation
    halves the cache; with one fp32 scale per row of d = 128 the cache is
    (128 + 4) / 256 of the bf16 one."""
    ratio = O.kv_cache_bytes(32, 8, 128, 1, 8192) / O.kv_cache_bytes(32, 8, 128, 2, 8192)
    assert ratio == 0.5
    codes, scales = O.quantize_int8_ref(np.ones((8, 64, 128), dtype=np.float32))
    assert (codes.nbytes + scales.nbytes) / (8 * 64 * 128 * 2) == (128 + 4) / 256


def check_int8_decode_composition(O):
    """With unit scales the int8 decode is the plain decode of the integer
    caches (brute force); with per-row scales it is the decode of the
    dequantised rows, position by position."""
    r = _rng(2400)
    B, H, K, d, lens = 2, 4, 2, 6, [5, 3]
    q = r.standard_normal((B, H, d)) * 0.05
    kc = r.integers(-127, 128, (B, K, 6, d)).astype(np.int8)
    vc = r.integers(-127, 128, (B, K, 6, d)).astype(np.int8)
    ones = np.ones((B, K, 6), dtype=np.float32)
    ref = BF.decode_bruteforce(q.tolist(), kc.astype(float).tolist(), vc.astype(float).tolist(), lens, 0.5)
    _close(O.decode_int8_ref(q, kc, vc, ones, ones, np.array(lens), 0.5), ref, 1e-11, "int8 unit scales")
    ks = r.uniform(0.001, 0.1, (B, K, 6)).astype(np.float32)
    vs = r.uniform(0.001, 0.1, (B, K, 6)).astype(np.float32)
    kf = [[[[float(kc[b, k, j, i]) * float(ks[b, k, j]) for i in range(d)] for j in range(6)]
           for k in range(K)] for b in range(B)]
    vf = [[[[float(vc[b, k, j, i]) * float(vs[b, k, j]) for i in range(d)] for j in range(6)]
           for k in range(K)] for b in range(B)]
    ref = BF.decode_bruteforce(q.tolist(), kf, vf, lens, 0.5)
    _close(O.decode_int8_ref(q, kc, vc, ks, vs, np.array(lens), 0.5), ref, 1e-13, "int8 scaled rows")


def check_int8_append(O):
    r = _rng(2500)
    B, K, S, d = 3, 2, 4, 8
    kc = r.integers(-127, 128, (B, K, S, d)).astype(np.int8)
    vc = r.integers(-127, 128, (B, K, S, d)).astype(np.int8)
    ks = r.uniform(0.1, 1, (B, K, S)).astype(np.float32)
    vs = r.uniform(0.1, 1, (B, K, S)).astype(np.float32)
    kn = r.standard_normal((B, K, d)).astype(np.float32)
    vn = r.standard_normal((B, K, d)).astype(np.float32)
    sl = np.array([0, 2, S])
    k2, v2, ks2, vs2, s2 = O.kv_append_int8_ref(kn, vn, kc, vc, ks, vs, sl)
    assert list(s2) == [1, 3, S]
    kq, kqs = O.quantize_int8_ref(kn)
    vq, vqs = O.quantize_int8_ref(vn)
    for b, L in enumerate(sl):
        for pos in range(S):
            new = pos == L
            assert np.array_equal(k2[b, :, pos], kq[b] if new else kc[b, :, pos])
            assert np.array_equal(v2[b, :, pos], vq[b] if new else vc[b, :, pos])
            assert np.array_equal(ks2[b, :, pos], kqs[b] if new else ks[b, :, pos])
            assert np.array_equal(vs2[b, :, pos], vqs[b] if new else vs[b, :, pos])
    # appended rows dequantise to within half a step of the new rows
    assert np.all(np.abs(O.dequantize_int8_ref(kq, kqs) - kn) <= kqs[..., None] * 0.50001)


# --------------------------------------------------------------------------
# chunked prefill over a cache, cross-attention, multi-row append
# --------------------------------------------------------------------------
def check_chunk_equals_causal_rows(O):
    """A chunk of S_q queries at the end of a cache of L_b rows gives rows
    [L_b - S_q, L_b) of causal prefill over the whole sequence (the pages:
    prefill row i is what decode step i computes)."""
    r = _rng(2600)
    B, H, K, d, Sq, S = 3, 6, 2, 8, 5, 14
    lens = [14, 9, 5]
    qf = r.standard_normal((B, H, S, d))
    k = r.standard_normal((B, K, S, d))
    v = r.standard_normal((B, K, S, d))
    qc = np.stack([qf[b, :, L - Sq:L] for b, L in enumerate(lens)])
    got = O.prefill_chunk_ref(qc, k, v, np.array(lens), 0.4)
    for b, L in enumerate(lens):
        want = O.prefill_causal_ref(qf[b:b + 1, :, :L], k[b:b + 1, :, :L], v[b:b + 1, :, :L], 0.4,
                                    rows=range(L - Sq, L))
        _close(got[b], want[0], 1e-13, f"chunk rows of sequence {b}")


def check_chunk_single_token_is_decode(O):
    q, kc, vc, sl = _rand_decode(2700, 3, 8, 2, 6, [7, 1, 12], nan_tail=False)
    got = O.prefill_chunk_ref(q[:, :, None, :], kc, vc, sl, 0.3)
    _close(got[:, :, 0], O.decode_ref(q, kc, vc, sl, 0.3), 1e-14, "chunk of one = decode")
    ref = BF.decode_bruteforce(q.tolist(), kc.tolist(), vc.tolist(), sl.tolist(), 0.3)
    _close(got[:, :, 0], ref, 1e-13, "chunk of one vs brute force")


def check_cross_attention_sdpa(O):
    """Non-causal GQA: torch's fp64 scaled_dot_product_attention with
    enable_gqa (no mask) on each sequence's valid rows."""
    r = _rng(2800)
    B, H, K, d, Sq, S = 3, 8, 2, 16, 7, 20
    lens = [20, 3, 11]
    q = r.standard_normal((B, H, Sq, d))
    k = r.standard_normal((B, K, S, d))
    v = r.standard_normal((B, K, S, d))
    got = O.cross_attention_ref(q, k, v, np.array(lens), 0.25)
    for b, L in enumerate(lens):
        want = _sdpa(q[b:b + 1], k[b:b + 1, :, :L].copy(), v[b:b + 1, :, :L].copy(), 0.25)
        _close(got[b], want[0], 1e-12, f"cross-attention sequence {b}")


def check_cross_rows_are_decodes(O):
    """Each query row of cross-attention is a decode step over all L_b rows;
    L_b = 0 gives zeros, and the rows do not depend on each other."""
    q, kc, vc, sl = _rand_decode(2900, 2, 4, 4, 8, [6, 0], nan_tail=False)
    qq = np.stack([q, -q, 2 * q], axis=2)                                     # [B, H, 3, d]
    got = O.cross_attention_ref(qq, kc, vc, sl, 0.5)
    for i in range(3):
        _close(got[:, :, i], O.decode_ref(qq[:, :, i], kc, vc, sl, 0.5), 1e-14, f"cross row {i}")
    assert np.all(got[1] == 0)


def check_append_rows(O):
    r = _rng(3000)
    B, K, S, d, T = 3, 2, 9, 4, 3
    kc = r.integers(-9999, 9999, (B, K, S, d), dtype=np.int16)
    vc = r.integers(-9999, 9999, (B, K, S, d), dtype=np.int16)
    kn = r.integers(-9999, 9999, (B, K, T, d), dtype=np.int16)
    vn = r.integers(-9999, 9999, (B, K, T, d), dtype=np.int16)
    sl = np.array([0, 6, 7])                          # the last has no room for 3 rows
    k2, v2, s2 = O.kv_append_rows_ref(kn, vn, kc, vc, sl)
    assert list(s2) == [3, 9, 7]
    # the same as T single-row appends (for the sequences with room)
    k3, v3, s3 = kc, vc, sl
    for t in range(T):
        k3, v3, s3 = O.kv_append_ref(kn[:, :, t], vn[:, :, t], k3, v3, s3)
    for b in (0, 1):
        assert np.array_equal(k2[b], k3[b]) and np.array_equal(v2[b], v3[b])
    assert np.array_equal(k2[2], kc[2]) and np.array_equal(v2[2], vc[2])


# --------------------------------------------------------------------------
# fused K/V projection
# --------------------------------------------------------------------------
def check_project_identity_weights(O):
    """d_model = d, W_K = I and W_V = 2 I for every head: K rows are the
    tokens themselves and V rows twice them."""
    r = _rng(3100)
    B, T, K, d = 2, 3, 4, 8
    x = r.standard_normal((B, T, d))
    w = np.concatenate([np.broadcast_to(np.eye(d), (K, d, d)), np.broadcast_to(2 * np.eye(d), (K, d, d))], axis=1)
    kr, vr = O.kv_project_ref(x, w)
    for k in range(K):
        assert np.array_equal(kr[:, k], x) and np.array_equal(vr[:, k], 2 * x)


def check_project_linear_library(O):
    """torch.nn.functional.linear (fp64) on W_KV flattened to [K * 2d, d_model]."""
    r = _rng(3200)
    B, T, K, d, dm = 2, 5, 3, 4, 16
    x = r.standard_normal((B, T, dm))
    w = r.standard_normal((K, 2 * d, dm))
    y = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w.reshape(K * 2 * d, dm))).numpy()
    y = y.reshape(B, T, K, 2 * d).transpose(0, 2, 1, 3)          # [B, K, T, 2d]
    kr, vr = O.kv_project_ref(x, w)
    _close(kr, y[..., :d], 1e-12, "K rows")
    _close(vr, y[..., d:], 1e-12, "V rows")


def check_project_append(O):
    r = _rng(3300)
    B, T, K, d, dm, S = 3, 2, 2, 4, 8, 6
    x = r.standard_normal((B, T, dm))
    w = r.standard_normal((K, 2 * d, dm))
    kc = r.standard_normal((B, K, S, d))
    vc = r.standard_normal((B, K, S, d))
    sl = np.array([0, 3, 5])                      # the last has no room for two rows
    k2, v2, s2 = O.kv_project_append_ref(x, w, kc, vc, sl)
    assert list(s2) == [2, 5, 5]
    for b, L in enumerate([0, 3]):
        for t in range(T):
            for k in range(K):
                _close(k2[b, k, L + t], w[k, :d] @ x[b, t], 1e-12, "appended K")
                _close(v2[b, k, L + t], w[k, d:] @ x[b, t], 1e-12, "appended V")
    assert np.array_equal(k2[2], kc[2]) and np.array_equal(v2[2], vc[2])
    assert np.array_equal(k2[1, :, :3], kc[1, :, :3])


# --------------------------------------------------------------------------
# split model of the two-pass decode
# --------------------------------------------------------------------------
def check_split_merge_equals_decode(O):
    """Any partition plan -- equal, ragged, with empty partitions, one
    position per partition -- merges to the plain decode (1e-12)."""
    q, kc, vc, sl = _rand_decode(3400, 3, 8, 2, 16, [37, 0, 100], nan_tail=False)
    ref = O.decode_ref(q, kc, vc, sl, 0.3)
    plans = [[(0, 101)], [(0, 32), (32, 64), (64, 96), (96, 128)], [(0, 7), (7, 50), (50, 51), (51, 200)],
             [(0, 5), (300, 400), (5, 101)], [(j, j + 1) for j in range(101)]]
    for bounds in plans:
        out = O.combine_partials_ref(*O.decode_partials_ref(q, kc, vc, sl, 0.3, bounds))
        _close(out, ref, 1e-12, f"merge over {len(bounds)} partitions")
        assert np.all(out[1] == 0), "an empty sequence merges to zeros"


def check_split_partials_closed_form(O):
    """One position per partition: m is the score, l = 1 and acc = v."""
    q, kc, vc, sl = _rand_decode(3500, 1, 2, 1, 4, [3], nan_tail=False)
    m, l, acc = O.decode_partials_ref(q, kc, vc, sl, 0.5, [(0, 1), (1, 2), (2, 3), (3, 4)])
    for h in range(2):
        for j in range(3):
            _close(m[0, h, j], 0.5 * kc[0, 0, j] @ q[0, h], 1e-15, "score")
            assert l[0, h, j] == 1.0 and np.array_equal(acc[0, h, j], vc[0, 0, j])
        assert m[0, h, 3] == -np.inf and l[0, h, 3] == 0 and not acc[0, h, 3].any()


ALL_CHECKS = [
    check_kv_bytes_golden, check_kv_head_map,
    check_bruteforce_decode, check_bruteforce_prefill, check_bruteforce_meanpool,
    check_sdpa_decode, check_sdpa_prefill, check_mha_special_case, check_mqa_special_case,
    check_expanded_kv_equivalence, check_identical_heads_meanpool,
    check_softmax_closed_form, check_weights_sum_to_one, check_weights_sdpa, check_single_row,
    check_zero_query_mean, check_constant_values, check_empty_length,
    check_incremental_equals_causal, check_prefill_closed_forms, check_append_semantics,
    check_meanpool_linearity, check_meanpool_identity_g1,
    check_paged_worked_example, check_paged_identity_table, check_paged_block_permutation,
    check_paged_append_identity,
    check_int8_exact_grid, check_int8_ties_to_even, check_int8_bounds_and_invariants,
    check_int8_halves_cache, check_int8_decode_composition, check_int8_append,
    check_chunk_equals_causal_rows, check_chunk_single_token_is_decode, check_cross_attention_sdpa,
    check_cross_rows_are_decodes, check_append_rows,
    check_project_identity_weights, check_project_linear_library, check_project_append,
    check_split_merge_equals_decode, check_split_partials_closed_form,
]
