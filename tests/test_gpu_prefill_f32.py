"""GPU parity of the fp32 prefill family (fp32 inputs and outputs, the
matrix cores in fp32) against the fp64 oracle at the fp32 gate (max-abs
1e-5): causal prefill, a chunk over a cache, cross-attention."""
import numpy as np
import pytest
import torch

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd.inputs import attention_inputs, prefill_inputs
from gpu_util import DEV, TOL, f64, guarded, guards_intact, note, report, scale_of
from oracle import cross_attention_ref, prefill_causal_ref, prefill_chunk_ref

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, K, S, d, S_max
    (1, 8, 2, 100, 128, 128),    # G = 4, S not a multiple of 16, NaN rows past S
    (2, 16, 4, 70, 64, 80),      # d = 64
    (1, 4, 4, 33, 128, 40),      # K = H (MHA)
    (1, 8, 1, 45, 64, 45),       # K = 1 (MQA), G = 8: two head chunks
    (1, 6, 2, 17, 128, 17),      # G = 3: an idle head row block
    (2, 8, 8, 1, 64, 1),         # one position
    (1, 71, 1, 20, 64, 24),      # G = 71: eighteen head chunks, the last holding 3 heads
    (1, 16, 2, 300, 128, 320),   # G = 8: ten 32-key tiles, nineteen query blocks
    (2, 32, 8, 257, 64, 260),    # G = 4: 32-position query blocks, a ragged last tile
]


@pytest.mark.parametrize("B,H,K,S,d,S_max", CASES)
def test_prefill_f32_shapes(B, H, K, S, d, S_max):
    note(f"prefill f32 B={B} H={H} K={K} S={S} d={d} S_max={S_max}")
    inp = prefill_inputs(B, H, K, S, d, "f32", seed=21, s_max=S_max)
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    out, buf, g = guarded(tuple(q.shape), torch.float32)
    gqa.gqa_prefill_causal(q, k, v, out, scale=scale_of(d))
    torch.cuda.synchronize()
    assert guards_intact(buf, g, torch.float32)
    ref = prefill_causal_ref(f64(inp["q"]), inp["k"].double().numpy(), inp["v"].double().numpy(), scale_of(d))
    r = report("prefill f32", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["f32"]


def test_prefill_f32_row0_is_v0():
    inp = prefill_inputs(1, 8, 2, 40, 128, "f32", seed=22)
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    out = torch.empty(q.shape, dtype=torch.float32, device=DEV)
    gqa.gqa_prefill_causal(q, k, v, out, scale=scale_of(128))
    torch.cuda.synchronize()
    for h in range(8):
        # one key: softmax weight exactly 1, so row 0 is V_0 (fp32 exact)
        assert torch.equal(out[0, h, 0].cpu(), inp["v"][0, h // 4, 0])


@pytest.mark.parametrize("B,H,K,S,L,d", [(2, 8, 2, 20, 90, 128), (1, 16, 4, 33, 33, 64), (1, 4, 1, 5, 200, 128)])
def test_chunk_f32(B, H, K, S, L, d):
    """Chunk of S queries over a cache of L rows (the chunk included)."""
    note(f"chunk f32 B={B} H={H} K={K} S={S} L={L} d={d}")
    inp = prefill_inputs(B, H, K, L, d, "f32", seed=23)
    qc = inp["q"][:, :, L - S:].contiguous()
    lens = torch.full((B,), L, dtype=torch.int32)
    out = torch.empty(qc.shape, dtype=torch.float32, device=DEV)
    gqa.gqa_prefill_chunk(qc.to(DEV), inp["k"].to(DEV), inp["v"].to(DEV), lens.to(DEV), out, scale=scale_of(d))
    torch.cuda.synchronize()
    ref = prefill_chunk_ref(f64(qc), inp["k"].double().numpy(), inp["v"].double().numpy(), lens.numpy(),
                            scale_of(d))
    r = report("chunk f32", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["f32"]


@pytest.mark.parametrize("B,H,K,S_q,lens,d", [(2, 8, 2, 30, [77, 0], 128), (1, 12, 3, 7, [300], 64)])
def test_cross_f32(B, H, K, S_q, lens, d):
    note(f"cross f32 B={B} H={H} K={K} S_q={S_q} lens={lens} d={d}")
    inp = attention_inputs(B, H, K, S_q, d, "f32", seed=24, kv_lens=lens)
    out = torch.empty(inp["q"].shape, dtype=torch.float32, device=DEV)
    gqa.gqa_cross_attention(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV), inp["kv_lens"].to(DEV), out,
                            scale=scale_of(d))
    torch.cuda.synchronize()
    ref = cross_attention_ref(f64(inp["q"]), inp["k"].double().numpy(), inp["v"].double().numpy(),
                              inp["kv_lens"].numpy(), scale_of(d))
    r = report("cross f32", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["f32"]
    for b, L in enumerate(lens):
        if L == 0:  # no visible row: zeros
            assert np.all(f64(out)[b] == 0.0)
