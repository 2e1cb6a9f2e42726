"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds no attention arithmetic: it only draws random numbers and
lays them out.  Every draw comes from one CPU ``torch.Generator`` seeded by
the caller, in a fixed order, so the GPU path and the CPU oracle consume the
very same bits.

Paged caches (``paged_layout``) re-lay those caches into blocks whose
physical order is a seeded random permutation.

Recipe (per call):
  1. ragged lengths, if requested: ``torch.randint(lo, hi + 1, (B,))``;
  2. q: float32 ``randn`` [B, H, d] (times ``q_scale``), then cast;
  3. k_cache: float32 ``randn`` [K, S_max, d] for b = 0..B-1 in turn, cast;
  4. v_cache: likewise;
  5. k_new, v_new: float32 ``randn`` [B, K, d] each, then cast.
Cache rows at positions >= L_b are then overwritten with NaN, so that any
read of an unused row poisons the output.

The named workloads mirror the model shapes the pages discuss: a 16-head /
4-group toy example, Llama-3-8B (32 query heads, 8 KV heads, d = 128),
Llama-2/3-70B (64 query heads, 8 KV heads), a 128K-token context, and a
4096-token causal prefill.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str               # "decode", "prefill", "chunk", "cross", "project" or "meanpool"
    B: int
    H: int
    K: int
    d: int
    dtype: str              # "f32" or "bf16"
    L: int = 0              # uniform cached length (decode) or S (prefill)
    ragged: tuple | None = None   # (lo, hi) inclusive for ragged decode
    q_scale: float = 1.0
    append: bool = False    # decode step preceded by one cache append
    note: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "decode_tiny_f32": Workload(
        "decode_tiny_f32", "decode", B=1, H=16, K=4, d=64, dtype="f32", L=256,
        note="16 query heads in 4 groups, fp32; also run with K=16 (MHA) and K=1 (MQA)"),
    "decode_llama3_8b": Workload(
        "decode_llama3_8b", "decode", B=16, H=32, K=8, d=128, dtype="bf16", L=8192,
        append=True, note="Llama-3-8B-shaped layer, 8192 cached tokens + 1 appended"),
    "decode_70b_ragged": Workload(
        "decode_70b_ragged", "decode", B=64, H=64, K=8, d=128, dtype="bf16",
        ragged=(512, 4096), note="Llama-2/3-70B-shaped layer, lengths U{512..4096}"),
    "decode_long_131k": Workload(
        "decode_long_131k", "decode", B=4, H=32, K=8, d=128, dtype="bf16", L=131072,
        q_scale=2.0, note="131072-token context, q scaled by 2"),
    "decode_mqa_71h": Workload(
        "decode_mqa_71h", "decode", B=32, H=71, K=1, d=64, dtype="bf16", L=32768,
        append=True, note="multi-query layer: 71 query heads sharing one KV head (the Falcon-7B head "
                          "layout), d=64, 32768 cached tokens + 1 appended"),
    "decode_f32_mqa_71h": Workload(
        "decode_f32_mqa_71h", "decode", B=8, H=71, K=1, d=128, dtype="f32", L=16384,
        note="fp32 multi-query layer: 71 query heads sharing one KV head, d=128, 16384 cached "
             "tokens (the fp32 pass reads each KV byte once for all five head blocks)"),
    "decode_paged_llama3_8b": Workload(
        "decode_paged_llama3_8b", "decode", B=16, H=32, K=8, d=128, dtype="bf16", L=8192,
        append=True, note="decode_llama3_8b over a paged cache: 16-token blocks in shuffled order",
        extra={"block_size": 16}),
    "decode_int8_llama3_8b": Workload(
        "decode_int8_llama3_8b", "decode", B=16, H=32, K=8, d=128, dtype="bf16", L=8192,
        append=True, note="decode_llama3_8b with the cache quantised to int8 (one fp32 scale per row)",
        extra={"kv_dtype": "int8"}),
    "prefill_chunk_8k": Workload(
        "prefill_chunk_8k", "chunk", B=2, H=64, K=8, d=128, dtype="bf16", L=8192,
        note="a 2048-token chunk continuing a 6144-row cache (queries at positions 6144..8191)",
        extra={"chunk": 2048}),
    "cross_attention_4k": Workload(
        "cross_attention_4k", "cross", B=4, H=32, K=8, d=128, dtype="bf16", L=4096,
        note="1024 decoder queries over 4096 encoder rows, no mask", extra={"S_q": 1024}),
    "kv_project_llama3_8b": Workload(
        "kv_project_llama3_8b", "project", B=16, H=32, K=8, d=128, dtype="bf16", L=8192,
        note="fused K/V projection of one decode token per sequence, d_model 4096, appended at 8192",
        extra={"d_model": 4096, "T": 1}),
    "meanpool_t5xxl": Workload(
        "meanpool_t5xxl", "meanpool", B=1, H=64, K=8, d=64, dtype="bf16",
        note="mean-pool conversion of a T5-XXL-shaped projection weight [64 heads x d_k 64, d_model 4096] "
             "to 8 KV heads (outer 1, inner d_k * d_model = 262144)",
        extra={"d_model": 4096, "matrices": 48}),
    "prefill_causal_4k": Workload(
        "prefill_causal_4k", "prefill", B=2, H=64, K=8, d=128, dtype="bf16", L=4096,
        note="causal prefill, S=4096, 64 query heads over 8 KV heads"),
    "prefill_causal_4k_f32": Workload(
        "prefill_causal_4k_f32", "prefill", B=2, H=64, K=8, d=128, dtype="f32", L=4096,
        note="prefill_causal_4k with fp32 inputs and outputs"),
}


def _nan_tail(cache: torch.Tensor, lens: torch.Tensor) -> None:
    for b in range(cache.shape[0]):
        cache[b, :, int(lens[b]):, :] = float("nan")


def decode_inputs(B: int, H: int, K: int, d: int, dtype: str, seed: int = 0,
                  L: int | None = None, lens=None, ragged: tuple | None = None,
                  q_scale: float = 1.0, s_max: int | None = None,
                  nan_tail: bool = True) -> dict:
    """Draw one decode batch (CPU tensors).

    Exactly one of ``L`` (every sequence at L), ``lens`` (explicit list) or
    ``ragged`` ((lo, hi) inclusive, drawn first) gives the cached lengths.
    ``s_max`` defaults to max(lens) + 1 so that one append always fits.
    """
    dt = _DT[dtype]
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    if ragged is not None:
        seq = torch.randint(int(ragged[0]), int(ragged[1]) + 1, (B,), generator=g)
    elif lens is not None:
        seq = torch.as_tensor(list(lens), dtype=torch.int64)
    else:
        seq = torch.full((B,), int(L), dtype=torch.int64)
    if seq.numel() != B:
        raise ValueError("lens must have B entries")
    smax = int(seq.max().item()) + 1 if s_max is None else int(s_max)
    if int(seq.max().item()) > smax:
        raise ValueError("s_max smaller than a length")
    q = (torch.randn((B, H, d), generator=g) * float(q_scale)).to(dt)
    kc = torch.empty((B, K, smax, d), dtype=dt)
    vc = torch.empty((B, K, smax, d), dtype=dt)
    for b in range(B):
        kc[b] = torch.randn((K, smax, d), generator=g).to(dt)
    for b in range(B):
        vc[b] = torch.randn((K, smax, d), generator=g).to(dt)
    k_new = torch.randn((B, K, d), generator=g).to(dt)
    v_new = torch.randn((B, K, d), generator=g).to(dt)
    if nan_tail:
        _nan_tail(kc, seq)
        _nan_tail(vc, seq)
    return {"q": q, "k_cache": kc, "v_cache": vc, "k_new": k_new, "v_new": v_new,
            "seq_lens": seq.to(torch.int32), "S_max": smax, "seed": int(seed)}


def prefill_inputs(B: int, H: int, K: int, S: int, d: int, dtype: str, seed: int = 0,
                   s_max: int | None = None) -> dict:
    """Draw one causal-prefill batch: q [B,H,S,d], k/v [B,K,S_max,d] (CPU).

    Rows [S, S_max) of k and v, if any, are NaN and must never be read."""
    dt = _DT[dtype]
    smax = S if s_max is None else int(s_max)
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn((B, H, S, d), generator=g).to(dt)
    k = torch.full((B, K, smax, d), float("nan"), dtype=dt)
    v = torch.full((B, K, smax, d), float("nan"), dtype=dt)
    k[:, :, :S] = torch.randn((B, K, S, d), generator=g).to(dt)
    v[:, :, :S] = torch.randn((B, K, S, d), generator=g).to(dt)
    return {"q": q, "k": k, "v": v, "S_max": smax, "seed": int(seed)}


def attention_inputs(B: int, H: int, K: int, S_q: int, d: int, dtype: str, seed: int = 0,
                     kv_lens=None, s_max: int | None = None, rows_new: int = 0) -> dict:
    """Draw queries [B, H, S_q, d] and K/V caches [B, K, S_max, d] holding
    kv_lens[b] rows each (rows past them NaN), for chunked prefill and
    cross-attention; with rows_new > 0 also k_new, v_new [B, K, rows_new, d]
    (a chunk to append).  Draw order: q, then k rows, v rows (sequence by
    sequence), then k_new, v_new."""
    dt = _DT[dtype]
    lens = [int(x) for x in kv_lens]
    if len(lens) != B:
        raise ValueError("kv_lens must have B entries")
    smax = max(lens) + rows_new if s_max is None else int(s_max)
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    q = torch.randn((B, H, S_q, d), generator=g).to(dt)
    k = torch.full((B, K, smax, d), float("nan"), dtype=dt)
    v = torch.full((B, K, smax, d), float("nan"), dtype=dt)
    for b, L in enumerate(lens):
        k[b, :, :L] = torch.randn((K, L, d), generator=g).to(dt)
    for b, L in enumerate(lens):
        v[b, :, :L] = torch.randn((K, L, d), generator=g).to(dt)
    out = {"q": q, "k": k, "v": v, "kv_lens": torch.tensor(lens, dtype=torch.int32), "S_max": smax,
           "seed": int(seed)}
    if rows_new:
        out["k_new"] = torch.randn((B, K, rows_new, d), generator=g).to(dt)
        out["v_new"] = torch.randn((B, K, rows_new, d), generator=g).to(dt)
    return out


def projection_inputs(B: int, T: int, d_model: int, K: int, d: int, seed: int = 0) -> dict:
    """Hidden states x [B, T, d_model] ~ N(0, 1) and a merged K/V projection
    W_KV [K, 2d, d_model] ~ N(0, 1/d_model) (so projected rows are O(1)),
    both bf16.  Draw order: x, then W_KV."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    x = torch.randn((B, T, d_model), generator=g).to(torch.bfloat16)
    w = (torch.randn((K, 2 * d, d_model), generator=g) / d_model ** 0.5).to(torch.bfloat16)
    return {"x": x, "w_kv": w, "seed": int(seed)}


def meanpool_inputs(outer: int, H: int, inner: int, dtype: str, seed: int = 0) -> torch.Tensor:
    """Draw a [outer, H, inner] weight-like tensor (CPU)."""
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    return torch.randn((outer, H, inner), generator=g).to(_DT[dtype])


def paged_layout(inp: dict, block_size: int, seed: int = 0, spare_blocks: int = 0,
                 shuffle: bool = True) -> dict:
    """Re-lay a decode batch's contiguous caches as paged pools.

    Sequence b owns max_blocks = ceil(S_max / block_size) logical blocks; the
    physical id of its block i is perm[b * max_blocks + i], with perm a
    ``torch.randperm`` of num_blocks = B * max_blocks + spare_blocks drawn
    from a generator seeded with ``seed`` (identity when ``shuffle`` is
    False).  Pools are [num_blocks, K, block_size, d]: block perm[..] holds
    the block's positions of every KV head.  Positions past S_max and the
    spare blocks are NaN.  Adds k_pool, v_pool, block_table (int32 [B,
    max_blocks]), block_size to a copy of ``inp``."""
    kc, vc = inp["k_cache"], inp["v_cache"]
    B, K, smax, d = kc.shape
    bs = int(block_size)
    mb = -(-smax // bs)
    nb = B * mb + int(spare_blocks)
    if shuffle:
        perm = torch.randperm(nb, generator=torch.Generator(device="cpu").manual_seed(int(seed)))
    else:
        perm = torch.arange(nb)
    out = dict(inp)
    for name, cache in (("k_pool", kc), ("v_pool", vc)):
        padded = torch.full((B, K, mb * bs, d), float("nan"), dtype=cache.dtype)
        padded[:, :, :smax] = cache
        pool = torch.full((nb, K, bs, d), float("nan"), dtype=cache.dtype)
        pool[perm[:B * mb]] = padded.view(B, K, mb, bs, d).permute(0, 2, 1, 3, 4).reshape(B * mb, K, bs, d)
        out[name] = pool
    out["block_table"] = perm[:B * mb].reshape(B, mb).to(torch.int32).contiguous()
    out["block_size"] = bs
    return out


def workload_inputs(w: Workload, seed: int = 0, s_max: int | None = None) -> dict:
    """Inputs of a named workload."""
    if w.kind == "prefill":
        return prefill_inputs(w.B, w.H, w.K, w.L, w.d, w.dtype, seed=seed, s_max=s_max)
    if w.kind == "chunk":
        # the cache before the chunk, plus the chunk's rows to append
        T = w.extra["chunk"]
        return attention_inputs(w.B, w.H, w.K, T, w.d, w.dtype, seed=seed, kv_lens=[w.L - T] * w.B,
                                s_max=s_max or w.L, rows_new=T)
    if w.kind == "cross":
        return attention_inputs(w.B, w.H, w.K, w.extra["S_q"], w.d, w.dtype, seed=seed,
                                kv_lens=[w.L] * w.B, s_max=s_max)
    if w.ragged is not None:
        return decode_inputs(w.B, w.H, w.K, w.d, w.dtype, seed=seed, ragged=w.ragged,
                             q_scale=w.q_scale, s_max=s_max)
    return decode_inputs(w.B, w.H, w.K, w.d, w.dtype, seed=seed, L=w.L,
                         q_scale=w.q_scale, s_max=s_max)
