"""GPU parity of chunked prefill over a cache (gqa_prefill_chunk), non-causal
cross-attention (gqa_cross_attention) and the multi-row append
(gqa_kv_append_rows) against the fp64 CPU oracle."""
import numpy as np
import pytest
import torch

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd.inputs import WORKLOADS, attention_inputs, prefill_inputs, workload_inputs
from gpu_util import oracle_by_kv_head, DEV, TOL, bf16_bound, f64, guarded, guards_intact, note, report, scale_of
from oracle import cross_attention_ref, kv_append_rows_ref, prefill_causal_ref, prefill_chunk_ref

pytestmark = pytest.mark.gpu


def _vmax(v, lens):
    return max(float(v[b, :, :L].float().abs().max()) if L else 0.0 for b, L in enumerate(lens))


def _chunk_gpu(inp, out_dtype=torch.bfloat16):
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    out = torch.empty(q.shape, dtype=out_dtype, device=DEV)
    gqa.gqa_prefill_chunk(q, k, v, inp["kv_lens"].to(DEV), out, scale=scale_of(q.shape[-1]))
    torch.cuda.synchronize()
    return out


CHUNK_CASES = [
    # B, H, K, d, S_q, lens (cache rows including the chunk)
    (2, 16, 4, 128, 16, [16, 300]),          # a chunk that is the whole sequence; an offset one
    (3, 32, 8, 128, 100, [100, 101, 1000]),  # ragged tail of the chunk, offsets 0/1/900
    (1, 8, 1, 64, 1, [77]),                  # a chunk of one query (= decode), G = 8
    (2, 12, 4, 128, 257, [257, 640]),        # G = 3, several query blocks
    (1, 16, 1, 128, 33, [200]),              # G = 16: two head chunks
    (2, 4, 4, 64, 65, [65, 129]),            # K = H (MHA)
]


@pytest.mark.parametrize("B,H,K,d,S_q,lens", CHUNK_CASES)
def test_chunk_shapes(B, H, K, d, S_q, lens):
    note(f"chunk B={B} H={H} K={K} d={d} S_q={S_q} lens={lens}")
    inp = attention_inputs(B, H, K, S_q, d, "bf16", seed=101, kv_lens=lens, s_max=max(lens) + 5)
    out = _chunk_gpu(inp)
    ref = prefill_chunk_ref(f64(inp["q"]), inp["k"].float().numpy(), inp["v"].float().numpy(),
                            inp["kv_lens"].numpy(), scale_of(d))
    r = report("chunk", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]
    assert r["max_abs"] <= bf16_bound(ref, _vmax(inp["v"], lens), weights_in_denominator=True)


def test_chunk_equals_prefill_causal_bitwise():
    """L_b = S: the chunk entry point is the causal prefill, bit for bit."""
    inp = prefill_inputs(2, 16, 4, 200, 128, "bf16", seed=102, s_max=210)
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    a = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    b = torch.empty_like(a)
    gqa.gqa_prefill_causal(q, k, v, a, scale=scale_of(128))
    gqa.gqa_prefill_chunk(q, k, v, torch.full((2,), 200, dtype=torch.int32, device=DEV), b, scale=scale_of(128))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_chunked_prefill_pipeline():
    """A 300-token prompt in chunks of 128, 128, 44: append each chunk's rows,
    attend with the chunk's queries; the rows equal causal prefill of the
    whole prompt (the oracle), and the cache equals the whole prompt's K/V."""
    B, H, K, d, S = 2, 16, 4, 128, 300
    full = prefill_inputs(B, H, K, S, d, "bf16", seed=103)
    kc = torch.full((B, K, 320, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    vc = torch.full_like(kc, float("nan"))
    sl = torch.zeros((B,), dtype=torch.int32, device=DEV)
    outs = []
    for c0, c1 in ((0, 128), (128, 256), (256, 300)):
        note(f"chunk [{c0}, {c1})")
        gqa.gqa_kv_append_rows(full["k"][:, :, c0:c1].contiguous().to(DEV), full["v"][:, :, c0:c1].contiguous().to(DEV),
                               kc, vc, sl)
        q = full["q"][:, :, c0:c1].contiguous().to(DEV)
        o = torch.empty(q.shape, dtype=torch.float32, device=DEV)
        gqa.gqa_prefill_chunk(q, kc, vc, sl, o, scale=scale_of(d))
        outs.append(o)
    torch.cuda.synchronize()
    assert sl.cpu().tolist() == [S, S]
    assert torch.equal(kc[:, :, :S].cpu(), full["k"][:, :, :S]) and torch.equal(vc[:, :, :S].cpu(), full["v"][:, :, :S])
    got = f64(torch.cat(outs, dim=2))
    ref = prefill_causal_ref(f64(full["q"]), full["k"].float().numpy(), full["v"].float().numpy(), scale_of(d))
    r = report("chunked pipeline", got, ref)
    assert r["finite"] and r["max_abs"] <= bf16_bound(ref, _vmax(full["v"], [S, S]), weights_in_denominator=True)


CROSS_CASES = [
    # B, H, K, d, S_q, kv_lens
    (4, 32, 8, 128, 77, [0, 1, 64, 1000]),   # empty, one row, a whole tile, ragged
    (2, 16, 4, 128, 1, [63, 65]),            # one query
    (2, 8, 1, 64, 300, [129, 500]),          # MQA, d = 64
    (1, 16, 1, 128, 40, [333]),              # G = 16
    (2, 6, 2, 128, 130, [200, 17]),          # G = 3
]


@pytest.mark.parametrize("B,H,K,d,S_q,lens", CROSS_CASES)
def test_cross_shapes(B, H, K, d, S_q, lens):
    note(f"cross B={B} H={H} K={K} d={d} S_q={S_q} lens={lens}")
    inp = attention_inputs(B, H, K, S_q, d, "bf16", seed=104, kv_lens=lens, s_max=max(lens) + 3)
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    gqa.gqa_cross_attention(q, k, v, inp["kv_lens"].to(DEV), out, scale=scale_of(d))
    torch.cuda.synchronize()
    ref = cross_attention_ref(f64(inp["q"]), inp["k"].float().numpy(), inp["v"].float().numpy(),
                              inp["kv_lens"].numpy(), scale_of(d))
    r = report("cross", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]
    assert r["max_abs"] <= bf16_bound(ref, _vmax(inp["v"], lens), weights_in_denominator=True)
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.count_nonzero(out[b]).item() == 0


def test_cross_fp32_out_and_guards():
    inp = attention_inputs(2, 16, 4, 50, 128, "bf16", seed=105, kv_lens=[90, 33])
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    out, buf, g = guarded(tuple(q.shape), torch.float32)
    gqa.gqa_cross_attention(q, k, v, inp["kv_lens"].to(DEV), out, scale=scale_of(128))
    torch.cuda.synchronize()
    assert guards_intact(buf, g, torch.float32)
    ref = cross_attention_ref(f64(inp["q"]), inp["k"].float().numpy(), inp["v"].float().numpy(),
                              inp["kv_lens"].numpy(), scale_of(128))
    assert report("cross f32", f64(out), ref)["max_abs"] <= TOL["bf16"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_append_rows_bit_exact(dtype):
    B, K, S, d, T = 3, 8, 40, 128, 7
    g = torch.Generator().manual_seed(106)
    kc = torch.randn((B, K, S, d), generator=g).to(dtype)
    vc = torch.randn((B, K, S, d), generator=g).to(dtype)
    kn = torch.randn((B, K, T, d), generator=g).to(dtype)
    vn = torch.randn((B, K, T, d), generator=g).to(dtype)
    sl = torch.tensor([0, 33, 34], dtype=torch.int32)   # the last has no room for 7 rows
    it = torch.int16 if dtype == torch.bfloat16 else torch.int32
    k2, v2, s2 = kv_append_rows_ref(kn.view(it).numpy(), vn.view(it).numpy(), kc.view(it).numpy(),
                                    vc.view(it).numpy(), sl.numpy())
    dk, dv, ds = kc.to(DEV), vc.to(DEV), sl.to(DEV)
    gqa.gqa_kv_append_rows(kn.to(DEV), vn.to(DEV), dk, dv, ds)
    torch.cuda.synchronize()
    assert ds.cpu().tolist() == list(s2) == [7, 40, 34]
    assert np.array_equal(dk.cpu().view(it).numpy(), k2) and np.array_equal(dv.cpu().view(it).numpy(), v2)


def test_chunk_full_workload():
    """2048-token chunk over a 6144-row cache (B=2, H=64, K=8): append the
    chunk, attend; every row of every head against the oracle."""
    w = WORKLOADS["prefill_chunk_8k"]
    inp = workload_inputs(w, seed=0)
    kc, vc, sl = inp["k"].to(DEV), inp["v"].to(DEV), inp["kv_lens"].to(DEV)
    note("chunk workload: GPU")
    gqa.gqa_kv_append_rows(inp["k_new"].to(DEV), inp["v_new"].to(DEV), kc, vc, sl)
    q = inp["q"].to(DEV)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    gqa.gqa_prefill_chunk(q, kc, vc, sl, out, scale=scale_of(w.d))
    torch.cuda.synchronize()
    assert sl.cpu().tolist() == [w.L] * w.B
    note("chunk workload: oracle, every row (per sequence and KV head, threaded)")
    k_all, v_all = kc.cpu(), vc.cpu()
    scale = scale_of(w.d)
    want = oracle_by_kv_head(lambda q_, k_, v_, l_: prefill_chunk_ref(q_, k_, v_, l_, scale), f64(inp["q"]),
                             k_all.float().numpy(), v_all.float().numpy(), np.array([w.L] * w.B))
    r = report("chunk 8k every row", f64(out), want)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]
    assert r["max_abs"] <= bf16_bound(want, _vmax(v_all, [w.L] * w.B), weights_in_denominator=True)


def test_cross_full_workload():
    """1024 queries over 4096 encoder rows (B=4, H=32, K=8), every row."""
    w = WORKLOADS["cross_attention_4k"]
    inp = workload_inputs(w, seed=0)
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    note("cross workload: GPU")
    gqa.gqa_cross_attention(q, k, v, inp["kv_lens"].to(DEV), out, scale=scale_of(w.d))
    torch.cuda.synchronize()
    note("cross workload: oracle, every row (per sequence and KV head, threaded)")
    scale = scale_of(w.d)
    ref = oracle_by_kv_head(lambda q_, k_, v_, l_: cross_attention_ref(q_, k_, v_, l_, scale), f64(inp["q"]),
                            inp["k"].float().numpy(), inp["v"].float().numpy(), inp["kv_lens"].numpy())
    r = report("cross 4k every row", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]
    assert r["max_abs"] <= bf16_bound(ref, _vmax(inp["v"], [w.L] * w.B), weights_in_denominator=True)
