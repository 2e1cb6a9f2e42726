"""Float64 NumPy oracle for grouped-query attention (GQA) over a KV cache.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the product path.

Sources (web pages; cited by host, title and section heading):

* [CAI]  compassingai.com, concept page "分組查詢注意力" (Grouped-Query
  Attention), sections "技術原理" (technical principle) and "關鍵引數"
  (key parameters).
* [PHY]  pinghaoyang.com.cn/aigc/posts/gqa, "GQA 完全拆解", sections
  "解码推理的内存账本" (the decode memory ledger), "MQA：一次性把 KV 头砍到只剩一个"
  (MQA), "GQA：插值在 MHA 与 MQA 之间的分组共享" (GQA as interpolation),
  "Uptraining：把现成 MHA 检查点改造成 GQA" (uptraining / mean pooling),
  "主流模型里的 GQA：KV 缓存账本" (KV ledger of mainstream models) and
  "工程实现：权重布局、repeat 与 Kernel 融合" (engineering).
* [CSDN] aicoding.csdn.net, "LLaMa3与DeepSeek采用的GQA技术", section
  "2. KV Cache的数学本质与工程挑战" (the mathematics of the KV cache).

Notation: B batch, H query heads, K KV heads, G = H / K query heads per KV
head, d head dimension, S_max cache capacity, L_b valid length of sequence b.

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* Query head h uses KV head floor(h / G): the groups are consecutive runs of
  G query heads ([PHY] GQA section gives the 1-based range of group g; [CAI]
  technical principle reshapes [.., H, d] into [.., K, H/K, d]).
* Decode attends over cache rows [0, L_b) and the new token's row is
  appended *before* attending, so that one decode step equals the last row
  of causal attention ([PHY] memory ledger: the step-t query meets keys 1..t).
* L_b = 0 gives a zero output row; append into a full cache writes nothing.
* The scale is an input (the pages use 1/sqrt(d_k)); callers pass the
  float32 value and the oracle uses it exactly.
* The causal mask keeps key j for query i iff j <= i (diagonal included).
"""
from __future__ import annotations

import numpy as np


def kv_head_of(h: int, H: int, K: int) -> int:
    """KV head shared by query head ``h`` (0-based).

    [PHY] GQA section: group g (1-based) holds the consecutive query heads
    (g-1)*H/K + 1 .. g*H/K, i.e. in 0-based terms head h belongs to group
    floor(h / (H/K)).
    """
    if H % K != 0:
        raise ValueError("H must be divisible by K")
    return h // (H // K)


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis; subtracting the row max changes nothing
    mathematically and keeps exp() finite."""
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def decode_weights_ref(q, k_cache, seq_lens, scale) -> list:
    """Attention weights of one decode step, per (b, h): a float64 vector of
    length L_b that is softmax(scale * q[b,h] . k_cache[b, kv(h), j]) over
    j in [0, L_b).

    [CSDN] section 2 (scores = q k^T / sqrt(d_k), then softmax) applied per
    group as in [CAI] technical principle.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, d = q.shape
    K = k_cache.shape[1]
    G = H // K
    w = []
    for b in range(B):
        L = int(seq_lens[b])
        row = []
        for h in range(H):
            if L == 0:
                row.append(np.zeros(0))
                continue
            kc = np.asarray(k_cache[b, h // G, :L, :], dtype=np.float64)
            row.append(_softmax_rows(float(scale) * (kc @ q[b, h])))
        w.append(row)
    return w


def decode_ref(q, k_cache, v_cache, seq_lens, scale) -> np.ndarray:
    """One GQA decode step: out[b, h] = sum_j p_j * V[b, kv(h), j] with
    p = softmax_j(scale * q[b, h] . K[b, kv(h), j]), j in [0, L_b).

    q        [B, H, d]        (any real dtype; converted to float64)
    k_cache  [B, K, S_max, d] (rows >= L_b are never read)
    v_cache  [B, K, S_max, d]
    seq_lens [B] integers, 0 <= L_b <= S_max
    returns  [B, H, d] float64; a row with L_b = 0 is zero.

    Follows [CAI] technical principle (per group g the G query heads attend
    to the one shared K_g, V_g with softmax(Q_g K_g^T / sqrt(d_k)) V_g),
    [PHY] memory ledger (the step-t query meets all cached rows) and [CSDN]
    section 2 (scores, softmax, weighted sum of cached values).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, d = q.shape
    Bk, K, S_max, dk = k_cache.shape
    if Bk != B or dk != d or H % K != 0:
        raise ValueError("shape mismatch")
    G = H // K
    out = np.zeros((B, H, d), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if not 0 <= L <= S_max:
            raise ValueError("seq_lens out of range")
        if L == 0:
            continue
        for k in range(K):
            Qg = q[b, k * G:(k + 1) * G, :]                          # [G, d]
            Kc = np.asarray(k_cache[b, k, :L, :], dtype=np.float64)  # [L, d]
            Vc = np.asarray(v_cache[b, k, :L, :], dtype=np.float64)  # [L, d]
            p = _softmax_rows(float(scale) * (Qg @ Kc.T))            # [G, L]
            out[b, k * G:(k + 1) * G, :] = p @ Vc
    return out


def prefill_causal_ref(q, k, v, scale, rows=None) -> np.ndarray:
    """Causal GQA attention over a whole prefix (prefill).

    out[b, h, i] = sum_{j <= i} softmax_j(scale * q[b,h,i] . k[b,kv(h),j]) v[b,kv(h),j]

    q     [B, H, S, d]
    k, v  [B, K, S_kv, d] with S_kv >= S; only rows [0, S) are used
    rows  optional sequence of query positions to evaluate (default: all S)
    returns [B, H, len(rows), d] float64

    [PHY] memory ledger (prefill processes the whole prefix in parallel; row
    i is exactly what decode step i computes), [CAI] technical principle for
    the grouping; the lower-triangular mask keeps the diagonal.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, S, d = q.shape
    K = k.shape[1]
    if H % K != 0 or k.shape[2] < S:
        raise ValueError("shape mismatch")
    G = H // K
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((B, H, len(rows), d), dtype=np.float64)
    keep = np.arange(S)[None, :] <= rows[:, None]                    # [R, S]
    for b in range(B):
        for g in range(K):
            Kc = np.asarray(k[b, g, :S, :], dtype=np.float64)           # [S, d]
            Vc = np.asarray(v[b, g, :S, :], dtype=np.float64)
            for h in range(g * G, (g + 1) * G):
                s = float(scale) * (q[b, h, rows, :] @ Kc.T)            # [R, S]
                s = np.where(keep, s, -np.inf)
                out[b, h] = _softmax_rows(s) @ Vc
    return out


def kv_append_ref(k_new, v_new, k_cache, v_cache, seq_lens):
    """Append one token's K and V rows per (b, kv head) at position L_b.

    k_new, v_new [B, K, d]; caches [B, K, S_max, d]; seq_lens [B].
    Returns new (k_cache, v_cache, seq_lens) copies: rows L_b of every (b, k)
    are replaced bit-for-bit by the new rows and L_b becomes L_b + 1; a
    sequence whose cache is full (L_b == S_max) is left unchanged.

    Works on any element dtype (pass integer views to compare bits).
    [CAI] technical principle (each generated token writes a [batch, 1, K,
    d_k] row), [PHY] memory ledger (the new K, V row is appended each step).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    sl = np.array(seq_lens, copy=True)
    S_max = kc.shape[2]
    for b in range(kc.shape[0]):
        L = int(sl[b])
        if L >= S_max:
            continue
        kc[b, :, L, :] = k_new[b]
        vc[b, :, L, :] = v_new[b]
        sl[b] = L + 1
    return kc, vc, sl


def meanpool_convert_ref(src, K: int) -> np.ndarray:
    """Mean-pool H per-head blocks into K group blocks.

    src [outer, H, inner] -> [outer, K, inner] float64 with
    dst[o, g, i] = (1/G) * sum_{r < G} src[o, g*G + r, i].

    [PHY] uptraining section (the new key projection of group g is the mean
    of the original key-head projections in that group; the same for values)
    and [CAI] technical principle (arithmetic mean over the H/K heads of a
    group; query projections unchanged).
    """
    src = np.asarray(src, dtype=np.float64)
    outer, H, inner = src.shape
    if H % K != 0:
        raise ValueError("H must be divisible by K")
    G = H // K
    return src.reshape(outer, K, G, inner).mean(axis=2)


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int,
                   elem_bytes: int, tokens: int = 1) -> int:
    """KV-cache size in bytes: 2 * layers * kv_heads * head_dim * bytes per
    element * tokens (one K and one V row per layer, KV head and token).

    [PHY] memory ledger and GQA section (S_KV = 2 L G d_k B, with G the number
    of KV heads in that page's notation).
    """
    return 2 * int(layers) * int(kv_heads) * int(head_dim) * int(elem_bytes) * int(tokens)


# --------------------------------------------------------------------------
# Paged KV cache
# --------------------------------------------------------------------------
# [CAI] downstream-schedulers section: a paged scheduler keeps blocks of
# K * s rows (KV heads, not query heads) and broadcasts each block to the H/K
# query heads of its group.  [PHY] engineering section: the paged blocks are
# organised by KV head and the kernel broadcasts inside the group; [PHY]
# memory ledger: paging removes allocation waste and is orthogonal to GQA.
#
# Reading (the pages give no index formula): a pool is [num_blocks, K,
# block_size, d]; a block table is [B, max_blocks]; logical position j of
# sequence b is row j % block_size of physical block block_table[b, j //
# block_size].


def paged_gather_ref(pool, block_table, seq_lens) -> np.ndarray:
    """Contiguous float64 cache [B, K, max_blocks * block_size, d] holding
    rows [0, L_b) of every (b, kv head) gathered from the paged ``pool``
    through ``block_table``; rows >= L_b are NaN (they must never be read)."""
    pool = np.asarray(pool)
    num_blocks, K, bs, d = pool.shape
    B, max_blocks = block_table.shape
    out = np.full((B, K, max_blocks * bs, d), np.nan)
    for b in range(B):
        L = int(seq_lens[b])
        if not 0 <= L <= max_blocks * bs:
            raise ValueError("seq_lens out of range")
        for j in range(L):
            n = int(block_table[b, j // bs])
            if not 0 <= n < num_blocks:
                raise ValueError("block id out of range")
            out[b, :, j, :] = pool[n, :, j % bs, :]
    return out


def decode_paged_ref(q, k_pool, v_pool, block_table, seq_lens, scale) -> np.ndarray:
    """One GQA decode step over a paged cache: ``decode_ref`` applied to the
    caches that ``paged_gather_ref`` assembles (the paging changes where rows
    live, not what is computed)."""
    kc = paged_gather_ref(k_pool, block_table, seq_lens)
    vc = paged_gather_ref(v_pool, block_table, seq_lens)
    return decode_ref(q, kc, vc, seq_lens, scale)


def kv_append_paged_ref(k_new, v_new, k_pool, v_pool, block_table, seq_lens):
    """Append one token's K and V rows per (b, kv head) into a paged cache.

    Returns new (k_pool, v_pool, seq_lens) copies: with L = L_b and
    n = block_table[b, L // block_size], row L % block_size of block n gets
    the new rows bit-for-bit and L_b becomes L + 1.  A sequence whose table
    is full (L == max_blocks * block_size) or whose block id lies outside
    [0, num_blocks) is left unchanged.  Any element dtype.
    """
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    sl = np.array(seq_lens, copy=True)
    num_blocks, _, bs, _ = kp.shape
    max_blocks = block_table.shape[1]
    for b in range(len(sl)):
        L = int(sl[b])
        if L >= max_blocks * bs:
            continue
        n = int(block_table[b, L // bs])
        if not 0 <= n < num_blocks:
            continue
        kp[n, :, L % bs, :] = k_new[b]
        vp[n, :, L % bs, :] = v_new[b]
        sl[b] = L + 1
    return kp, vp, sl


# --------------------------------------------------------------------------
# int8 KV cache
# --------------------------------------------------------------------------
# [PHY] section on related work after the KV ledger: quantising the cached K
# and V from 16-bit floats to INT8 / INT4 is orthogonal to GQA (GQA cuts the
# number of heads, quantisation the bytes per element; the savings
# multiply).  [CSDN] section 3 (practical deployment tips): 8-bit KV-cache
# quantisation cuts the cache memory by a further 50%.
#
# Reading (the pages give no quantisation rule): symmetric absmax
# quantisation per cached row, i.e. per (sequence, KV head, position) over
# the d elements, all in IEEE float32:
#     amax  = max_i |x_i|
#     inv   = 127 / amax                     (float32 division)
#     c_i   = clamp(rint(x_i * inv), -127, 127)  (float32 product, ties to even)
#     scale = amax / 127                     (float32 division)
# and the dequantised value is c_i * scale.  A row of zeros gets codes 0 and
# scale 0.  Rows must be finite.


def quantize_int8_ref(x):
    """Per-row int8 codes and float32 scales of ``x`` [..., d] (the rule
    above).  Returns (codes int8 [..., d], scales float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("rows must be finite")
    amax = np.max(np.abs(x), axis=-1)
    codes = np.zeros(x.shape, dtype=np.int8)
    scales = np.zeros(amax.shape, dtype=np.float32)
    nz = amax > 0
    inv = np.float32(127) / amax[nz]
    c = np.rint(x[nz] * inv[..., None])
    codes[nz] = np.clip(c, -127, 127).astype(np.int8)
    scales[nz] = amax[nz] / np.float32(127)
    return codes, scales


def dequantize_int8_ref(codes, scales) -> np.ndarray:
    """float64 values c_i * scale of int8 rows (exact in float64)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def decode_int8_ref(q, k_codes, v_codes, k_scales, v_scales, seq_lens, scale) -> np.ndarray:
    """One GQA decode step over an int8 cache: ``decode_ref`` on the
    dequantised caches.  Codes [B, K, S_max, d], scales [B, K, S_max]."""
    return decode_ref(q, dequantize_int8_ref(k_codes, k_scales),
                      dequantize_int8_ref(v_codes, v_scales), seq_lens, scale)


def kv_append_int8_ref(k_new, v_new, k_codes, v_codes, k_scales, v_scales, seq_lens):
    """Quantise each new K and V row and append it at position L_b of an
    int8 cache; returns new (k_codes, v_codes, k_scales, v_scales, seq_lens).
    A full cache (L_b == S_max) is left unchanged."""
    kc = np.array(k_codes, copy=True)
    vc = np.array(v_codes, copy=True)
    ks = np.array(k_scales, copy=True)
    vs = np.array(v_scales, copy=True)
    sl = np.array(seq_lens, copy=True)
    kq, kqs = quantize_int8_ref(k_new)
    vq, vqs = quantize_int8_ref(v_new)
    S_max = kc.shape[2]
    for b in range(kc.shape[0]):
        L = int(sl[b])
        if L >= S_max:
            continue
        kc[b, :, L, :] = kq[b]
        vc[b, :, L, :] = vq[b]
        ks[b, :, L] = kqs[b]
        vs[b, :, L] = vqs[b]
        sl[b] = L + 1
    return kc, vc, ks, vs, sl


# --------------------------------------------------------------------------
# Prefill over an existing cache (chunked prefill) and cross-attention
# --------------------------------------------------------------------------
# [PHY] memory ledger: the query at position t attends to cached rows 1..t;
# prefill computes a whole run of positions at once.  Reading: a chunk of
# S_q new tokens whose K/V rows have been appended, so that the cache of
# sequence b holds L_b rows ending with the chunk, puts query i at absolute
# position L_b - S_q + i; it attends causally to rows j <= L_b - S_q + i.
# [PHY] GQA section: GQA is used for decoder self-attention and for
# cross-attention (not for encoder self-attention); cross-attention has no
# causal mask: every query attends to all L_b rows of its (encoder) K/V.
# A query with no visible row gets a zero output row.


def _attend_rows(q_rows, Kc, Vc, keep, scale):
    """softmax(scale * q_rows @ Kc^T) @ Vc over the kept keys; rows with no
    kept key are zero.  q_rows [R, d], Kc/Vc [L, d], keep [R, L] bool."""
    out = np.zeros((q_rows.shape[0], Vc.shape[1]))
    if Kc.shape[0] == 0:
        return out
    s = float(scale) * (q_rows @ Kc.T)
    s = np.where(keep, s, -np.inf)
    has = keep.any(axis=1)
    if has.any():
        out[has] = _softmax_rows(s[has]) @ Vc
    return out


def prefill_chunk_ref(q, k_cache, v_cache, seq_lens, scale) -> np.ndarray:
    """Causal GQA attention of a chunk of S_q queries over a cache that
    already holds the chunk: q [B, H, S_q, d], caches [B, K, S_max, d],
    seq_lens [B] = L_b (rows in the cache, chunk included).  Query i of
    sequence b sits at position L_b - S_q + i and sees rows
    j <= L_b - S_q + i (j < L_b).  Returns [B, H, S_q, d] float64."""
    q = np.asarray(q, dtype=np.float64)
    B, H, Sq, d = q.shape
    K = k_cache.shape[1]
    if H % K != 0:
        raise ValueError("H must be divisible by K")
    G = H // K
    out = np.zeros((B, H, Sq, d))
    for b in range(B):
        L = int(seq_lens[b])
        if not 0 <= L <= k_cache.shape[2]:
            raise ValueError("seq_lens out of range")
        pos = L - Sq + np.arange(Sq)                                  # absolute positions
        keep = np.arange(L)[None, :] <= pos[:, None]                  # [S_q, L]
        for g in range(K):
            Kc = np.asarray(k_cache[b, g, :L, :], dtype=np.float64)
            Vc = np.asarray(v_cache[b, g, :L, :], dtype=np.float64)
            for h in range(g * G, (g + 1) * G):
                out[b, h] = _attend_rows(q[b, h], Kc, Vc, keep, scale)
    return out


def cross_attention_ref(q, k, v, kv_lens, scale) -> np.ndarray:
    """Non-causal GQA attention: q [B, H, S_q, d] over rows [0, L_b) of
    k, v [B, K, S_max, d], L_b = kv_lens[b].  Returns [B, H, S_q, d]."""
    q = np.asarray(q, dtype=np.float64)
    B, H, Sq, d = q.shape
    K = k.shape[1]
    if H % K != 0:
        raise ValueError("H must be divisible by K")
    G = H // K
    out = np.zeros((B, H, Sq, d))
    for b in range(B):
        L = int(kv_lens[b])
        if not 0 <= L <= k.shape[2]:
            raise ValueError("kv_lens out of range")
        keep = np.ones((Sq, L), dtype=bool)
        for g in range(K):
            Kc = np.asarray(k[b, g, :L, :], dtype=np.float64)
            Vc = np.asarray(v[b, g, :L, :], dtype=np.float64)
            for h in range(g * G, (g + 1) * G):
                out[b, h] = _attend_rows(q[b, h], Kc, Vc, keep, scale)
    return out


def kv_append_rows_ref(k_new, v_new, k_cache, v_cache, seq_lens):
    """Append T rows per (b, KV head): k_new, v_new [B, K, T, d] go to
    positions [L_b, L_b + T) and L_b becomes L_b + T; a sequence without room
    for all T rows (L_b + T > S_max) is left unchanged.  Any dtype."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    sl = np.array(seq_lens, copy=True)
    T = k_new.shape[2]
    S_max = kc.shape[2]
    for b in range(kc.shape[0]):
        L = int(sl[b])
        if L + T > S_max:
            continue
        kc[b, :, L:L + T, :] = k_new[b]
        vc[b, :, L:L + T, :] = v_new[b]
        sl[b] = L + T
    return kc, vc, sl


# --------------------------------------------------------------------------
# Fused K/V projection and append
# --------------------------------------------------------------------------
# [PHY] engineering section: GQA's W_K and W_V are [G, d_k, d_model] (G KV
# heads in that page's notation); inference frameworks merge them into one
# W_KV of shape [G, 2 d_k, d_model] so that a single GEMM yields both K and
# V.  Reading: for head k, rows [0, d) of W_KV[k] are W_K[k] and rows
# [d, 2d) are W_V[k]; a token's hidden state x (length d_model) gives
# K_k = W_KV[k, :d] x and V_k = W_KV[k, d:] x, which are appended to the
# cache (no bias; positional rotation, which the same section leaves to the
# unchanged rest of the model, is not part of this step).


def kv_project_ref(x, w_kv):
    """K and V rows of T tokens per sequence: x [B, T, d_model], w_kv
    [K, 2d, d_model] -> (k_rows, v_rows), each [B, K, T, d] float64."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_kv, dtype=np.float64)
    K, d2, dm = w.shape
    d = d2 // 2
    y = np.einsum("btm,kjm->bktj", x, w)                 # [B, K, T, 2d]
    return y[..., :d], y[..., d:]


def kv_project_append_ref(x, w_kv, k_cache, v_cache, seq_lens):
    """Project the T new tokens of every sequence and append their K/V rows
    at positions [L_b, L_b + T) (float64 caches returned, with the new
    lengths); a sequence without room for T rows is left unchanged."""
    kr, vr = kv_project_ref(x, w_kv)
    return kv_append_rows_ref(kr, vr, np.asarray(k_cache, dtype=np.float64),
                              np.asarray(v_cache, dtype=np.float64), seq_lens)


# --------------------------------------------------------------------------
# Split model (test infrastructure for the two-pass decode)
# --------------------------------------------------------------------------
# The decode is computed in partitions of the cached positions whose partial
# states are merged afterwards (the block-wise online softmax the foundit.cn
# article and the engineering section of pinghaoyang.com.cn name, via
# FlashAttention).  For a partition P the partial state of a query is
#     m_P = max_{j in P} s_j,  l_P = sum_{j in P} e^{s_j - m_P},
#     acc_P = sum_{j in P} e^{s_j - m_P} v_j
# (m = -inf, l = 0, acc = 0 for an empty partition) and the merge is
#     M = max_P m_P,  out = sum_P e^{m_P - M} acc_P / sum_P e^{m_P - M} l_P,
# which equals the softmax-weighted sum over all positions because
# e^{s - m_P} e^{m_P - M} = e^{s - M}.


def decode_partials_ref(q, k_cache, v_cache, seq_lens, scale, bounds):
    """float64 partial states of every query head for the position ranges
    ``bounds`` = [(t0, t1), ...] (clipped to [0, L_b)).
    Returns (m [B, H, P], l [B, H, P], acc [B, H, P, d])."""
    q = np.asarray(q, dtype=np.float64)
    B, H, d = q.shape
    K = k_cache.shape[1]
    G = H // K
    P = len(bounds)
    m = np.full((B, H, P), -np.inf)
    l = np.zeros((B, H, P))
    acc = np.zeros((B, H, P, d))
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(H):
            k = h // G
            for p, (t0, t1) in enumerate(bounds):
                t0, t1 = max(t0, 0), min(t1, L)
                if t0 >= t1:
                    continue
                s = float(scale) * (np.asarray(k_cache[b, k, t0:t1], dtype=np.float64) @ q[b, h])
                m[b, h, p] = s.max()
                e = np.exp(s - m[b, h, p])
                l[b, h, p] = e.sum()
                acc[b, h, p] = e @ np.asarray(v_cache[b, k, t0:t1], dtype=np.float64)
    return m, l, acc


def combine_partials_ref(m, l, acc) -> np.ndarray:
    """Merge partial states over the last partition axis; a query whose
    partitions are all empty gets a zero row."""
    M = m.max(axis=-1, keepdims=True)
    w = np.where(np.isfinite(m), np.exp(m - np.where(np.isfinite(M), M, 0.0)), 0.0)
    num = (w[..., None] * acc).sum(axis=-2)
    den = (w * l).sum(axis=-1)
    out = np.zeros_like(num)
    nz = den > 0
    out[nz] = num[nz] / den[nz][..., None]
    return out
