"""Seeded random shape sweep of every attention entry point against the fp64
oracle: group sizes, head dimensions, ragged lengths, block sizes and query
counts drawn from a fixed generator, so a reader can re-run any failing case
from its printed parameters."""
import numpy as np
import pytest
import torch

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd.inputs import attention_inputs, decode_inputs, paged_layout
from gpu_util import DEV, TOL, bf16_bound, f64, note, report, scale_of
from oracle import (cross_attention_ref, decode_int8_ref, decode_paged_ref, decode_ref, prefill_chunk_ref,
                    quantize_int8_ref)

pytestmark = pytest.mark.gpu

N_CASES = 12


SMALL_GROUPS = [1, 2, 3, 4, 5, 8, 16]
LARGE_GROUPS = [17, 24, 33, 48, 64, 71, 100, 128]   # several 16-head blocks per group


def _cases(seed, groups=SMALL_GROUPS):
    r = np.random.default_rng(seed)
    out = []
    for _ in range(N_CASES):
        K = int(r.choice([1, 2, 4, 8]))
        G = int(r.choice(groups))
        B = int(r.integers(1, 5))
        d = int(r.choice([64, 128]))
        lens = [int(x) for x in r.integers(0, 1500, B)]
        if r.random() < 0.3:
            lens[0] = 0
        out.append((B, G * K, K, d, lens))
    return out


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode_contiguous_paged_int8(case):
    _check_decode(case, *_cases(2024)[case])


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode_large_groups(case):
    _check_decode(case, *_cases(2026, LARGE_GROUPS)[case])


def _check_decode(case, B, H, K, d, lens):
    note(f"random decode B={B} H={H} K={K} d={d} lens={lens}")
    s_max = (max(lens) + 4) // 4 * 4
    inp = decode_inputs(B, H, K, d, "bf16", seed=500 + case, lens=lens, s_max=s_max, nan_tail=False)
    msl = max(max(lens), 1)
    sc = scale_of(d)
    q = inp["q"].to(DEV)
    sl = inp["seq_lens"].to(DEV)
    ws = torch.empty(max(gqa.gqa_decode_workspace_bytes(B, H, K, msl, d), 16), dtype=torch.uint8, device=DEV)
    # contiguous
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    gqa.gqa_decode(q, inp["k_cache"].to(DEV), inp["v_cache"].to(DEV), sl, out, ws, msl, scale=sc)
    torch.cuda.synchronize()
    ref = decode_ref(f64(inp["q"]), inp["k_cache"].float().numpy(), inp["v_cache"].float().numpy(), lens, sc)
    vmax = float(inp["v_cache"].float().abs().max())
    r1 = report("contiguous", f64(out), ref)
    assert r1["finite"] and r1["max_abs"] <= min(TOL["bf16"], bf16_bound(ref, vmax))
    # paged, block size 16 or 32, shuffled
    bs = 16 if case % 2 else 32
    pg = paged_layout(inp, bs, seed=600 + case, spare_blocks=2)
    pws = torch.empty(max(gqa.gqa_decode_paged_workspace_bytes(B, H, K, msl, d, bs), 16), dtype=torch.uint8,
                      device=DEV)
    pout = torch.empty_like(out)
    gqa.gqa_decode_paged(q, pg["k_pool"].to(DEV), pg["v_pool"].to(DEV), pg["block_table"].to(DEV), sl, pout, pws,
                         msl, scale=sc)
    torch.cuda.synchronize()
    pref = decode_paged_ref(f64(inp["q"]), pg["k_pool"].float().numpy(), pg["v_pool"].float().numpy(),
                            pg["block_table"].numpy(), np.array(lens), sc)
    r2 = report("paged", f64(pout), pref)
    assert r2["finite"] and r2["max_abs"] <= min(TOL["bf16"], bf16_bound(pref, vmax))
    # int8: quantised by the oracle and by the GPU (bit-exact), then decoded
    kc8, ks8 = quantize_int8_ref(inp["k_cache"].float().numpy())
    vc8, vs8 = quantize_int8_ref(inp["v_cache"].float().numpy())
    gk = torch.empty(inp["k_cache"].shape, dtype=torch.int8, device=DEV)
    gks = torch.empty(inp["k_cache"].shape[:3], dtype=torch.float32, device=DEV)
    gqa.gqa_kv_quantize_int8(inp["k_cache"].to(DEV), gk, gks)
    gv = torch.empty_like(gk)
    gvs = torch.empty_like(gks)
    gqa.gqa_kv_quantize_int8(inp["v_cache"].to(DEV), gv, gvs)
    iout = torch.empty_like(out)
    gqa.gqa_decode_int8(q, gk, gv, gks, gvs, sl, iout, ws, msl, scale=sc)
    torch.cuda.synchronize()
    assert np.array_equal(gk.cpu().numpy(), kc8) and np.array_equal(gvs.cpu().numpy(), vs8)
    iref = decode_int8_ref(f64(inp["q"]), kc8, vc8, ks8, vs8, np.array(lens), sc)
    vmax8 = float(np.abs(vc8.astype(np.float64) * vs8[..., None]).max())
    r3 = report("int8", f64(iout), iref)
    assert r3["finite"] and r3["max_abs"] <= min(TOL["bf16"], bf16_bound(iref, vmax8))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_chunk_and_cross(case):
    B, H, K, d, lens = _cases(2025)[case]
    r = np.random.default_rng(700 + case)
    S_q = int(r.integers(1, 200))
    kv = [max(L, S_q) for L in lens]          # a chunk lives inside its cache
    note(f"random chunk/cross B={B} H={H} K={K} d={d} S_q={S_q} kv={kv}")
    inp = attention_inputs(B, H, K, S_q, d, "bf16", seed=800 + case, kv_lens=kv, s_max=max(kv) + 2)
    q, k, v, kl = (inp[n].to(DEV) for n in ("q", "k", "v", "kv_lens"))
    sc = scale_of(d)
    vmax = max(float(inp["v"][b, :, :L].float().abs().max()) for b, L in enumerate(kv))
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    gqa.gqa_prefill_chunk(q, k, v, kl, out, scale=sc)
    torch.cuda.synchronize()
    ref = prefill_chunk_ref(f64(inp["q"]), inp["k"].float().numpy(), inp["v"].float().numpy(), np.array(kv), sc)
    r1 = report("chunk", f64(out), ref)
    assert r1["finite"] and r1["max_abs"] <= min(TOL["bf16"], bf16_bound(ref, vmax, weights_in_denominator=True))
    # cross-attention over the (possibly empty) original lengths
    kl2 = torch.tensor(lens, dtype=torch.int32)
    out2 = torch.empty_like(out)
    gqa.gqa_cross_attention(q, k, v, kl2.to(DEV), out2, scale=sc)
    torch.cuda.synchronize()
    ref2 = cross_attention_ref(f64(inp["q"]), inp["k"].float().numpy(), inp["v"].float().numpy(), kl2.numpy(), sc)
    r2 = report("cross", f64(out2), ref2)
    assert r2["finite"] and r2["max_abs"] <= min(TOL["bf16"], bf16_bound(ref2, vmax, weights_in_denominator=True))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode_f32(case):
    """The fp32 decode pass (matrix cores in fp32) over the same seeded group
    sizes, small and large, at the fp32 gate."""
    groups = SMALL_GROUPS if case % 2 == 0 else LARGE_GROUPS
    B, H, K, d, lens = _cases(2027 + case % 2, groups)[case]
    note(f"random f32 decode B={B} H={H} K={K} d={d} lens={lens}")
    s_max = max(lens) + 1
    inp = decode_inputs(B, H, K, d, "f32", seed=900 + case, lens=lens, s_max=s_max)
    msl = max(max(lens), 1)
    ws = torch.empty(max(gqa.gqa_decode_workspace_bytes(B, H, K, msl, d), 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    gqa.gqa_decode(inp["q"].to(DEV), inp["k_cache"].to(DEV), inp["v_cache"].to(DEV), inp["seq_lens"].to(DEV), out,
                   ws, msl, scale=scale_of(d))
    torch.cuda.synchronize()
    ref = decode_ref(f64(inp["q"]), inp["k_cache"].double().numpy(), inp["v_cache"].double().numpy(), lens,
                     scale_of(d))
    r = report("f32 decode", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["f32"]


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_chunk_and_cross_f32(case):
    """The fp32 prefill family (matrix cores in fp32): a chunk over a cache and
    cross-attention on seeded shapes, at the fp32 gate."""
    B, H, K, d, lens = _cases(2028)[case]
    r = np.random.default_rng(1000 + case)
    S_q = int(r.integers(1, 200))
    kv = [max(L, S_q) for L in lens]
    note(f"random f32 chunk/cross B={B} H={H} K={K} d={d} S_q={S_q} kv={kv}")
    inp = attention_inputs(B, H, K, S_q, d, "f32", seed=1100 + case, kv_lens=kv, s_max=max(kv) + 2)
    q, k, v, kl = (inp[n].to(DEV) for n in ("q", "k", "v", "kv_lens"))
    sc = scale_of(d)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    gqa.gqa_prefill_chunk(q, k, v, kl, out, scale=sc)
    torch.cuda.synchronize()
    ref = prefill_chunk_ref(f64(inp["q"]), inp["k"].double().numpy(), inp["v"].double().numpy(), np.array(kv), sc)
    r1 = report("f32 chunk", f64(out), ref)
    assert r1["finite"] and r1["max_abs"] <= TOL["f32"]
    kl2 = torch.tensor(lens, dtype=torch.int32)
    out2 = torch.empty_like(out)
    gqa.gqa_cross_attention(q, k, v, kl2.to(DEV), out2, scale=sc)
    torch.cuda.synchronize()
    ref2 = cross_attention_ref(f64(inp["q"]), inp["k"].double().numpy(), inp["v"].double().numpy(), kl2.numpy(),
                               sc)
    r2 = report("f32 cross", f64(out2), ref2)
    assert r2["finite"] and r2["max_abs"] <= TOL["f32"]
