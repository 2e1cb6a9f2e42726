"""GPU parity of the causal prefill (gqa_prefill_causal) against the oracle."""
import numpy as np
import pytest
import torch

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd.inputs import WORKLOADS, decode_inputs, prefill_inputs, workload_inputs
from gpu_util import oracle_by_kv_head, DEV, TOL, bf16_bound, f64, guarded, guards_intact, note, report, run_decode, scale_of
from oracle import prefill_causal_ref

pytestmark = pytest.mark.gpu


def _run(inp, out_dtype=torch.bfloat16):
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    out = torch.empty(q.shape, dtype=out_dtype, device=DEV)
    gqa.gqa_prefill_causal(q, k, v, out, scale=scale_of(q.shape[-1]))
    torch.cuda.synchronize()
    return out


def _vmax(inp, S):
    return float(inp["v"][:, :, :S].float().abs().max())


CASES = [
    # B, H, K, S, d, S_max
    (1, 8, 2, 100, 128, 128),    # ragged S, NaN rows beyond S
    (2, 16, 4, 300, 128, 300),   # G = 4
    (1, 8, 1, 77, 64, 80),       # G = 8, d = 64
    (1, 12, 4, 64, 128, 64),     # G = 3
    (1, 16, 1, 130, 128, 130),   # G = 16: two head chunks
    (2, 4, 4, 33, 64, 40),       # K = H (MHA)
    (1, 8, 8, 1, 128, 1),        # one position
    (1, 10, 5, 150, 128, 150),   # G = 2: four 16-position blocks per workgroup
    (2, 10, 2, 90, 64, 96),      # G = 5: three idle row tiles
    (1, 4, 4, 300, 128, 300),    # G = 1 (MHA): eight blocks per workgroup, S not a multiple of 128
    (1, 71, 1, 90, 64, 96),      # G = 71 (MQA): nine head chunks, the last holding 7 heads
    (1, 48, 2, 70, 128, 70),     # G = 24: three head chunks
]


@pytest.mark.parametrize("B,H,K,S,d,S_max", CASES)
def test_prefill_shapes(B, H, K, S, d, S_max):
    note(f"prefill B={B} H={H} K={K} S={S} d={d} S_max={S_max}")
    inp = prefill_inputs(B, H, K, S, d, "bf16", seed=7, s_max=S_max)
    out = _run(inp)
    ref = prefill_causal_ref(f64(inp["q"]), inp["k"].float().numpy(), inp["v"].float().numpy(), scale_of(d))
    r = report("prefill", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]
    assert r["max_abs"] <= bf16_bound(ref, _vmax(inp, S), weights_in_denominator=True)


def test_prefill_fp32_out_and_guards():
    inp = prefill_inputs(1, 8, 2, 90, 128, "bf16", seed=8)
    q, k, v = inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV)
    out, buf, g = guarded(tuple(q.shape), torch.float32)
    gqa.gqa_prefill_causal(q, k, v, out, scale=scale_of(128))
    torch.cuda.synchronize()
    assert guards_intact(buf, g, torch.float32)
    ref = prefill_causal_ref(f64(inp["q"]), inp["k"].float().numpy(), inp["v"].float().numpy(), scale_of(128))
    r = report("prefill f32 out", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]


def test_prefill_row0_is_v0():
    inp = prefill_inputs(1, 8, 2, 40, 128, "bf16", seed=12)
    out = _run(inp, torch.float32)
    for h in range(8):
        # one key: softmax weight exactly 1, so the row is V_0 (bf16 exact in fp32)
        assert torch.equal(out[0, h, 0].cpu(), inp["v"][0, h // 4, 0].float())


def test_decode_after_append_matches_prefill_row():
    """Incremental decode over an appended cache equals the last causal row."""
    B, H, K, S, d = 2, 16, 4, 200, 128
    inp = prefill_inputs(B, H, K, S, d, "bf16", seed=13)
    pre = f64(_run(inp, torch.float32))
    i = S - 1
    dec_in = {"q": inp["q"][:, :, i].contiguous(),
              "k_cache": inp["k"].clone(), "v_cache": inp["v"].clone(),
              "seq_lens": torch.full((B,), i, dtype=torch.int32),
              "k_new": inp["k"][:, :, i].contiguous(), "v_new": inp["v"][:, :, i].contiguous()}
    dec, _ = run_decode(dec_in, out_dtype=torch.float32, append=True, max_seq_len=S)
    ref = prefill_causal_ref(f64(inp["q"]), inp["k"].float().numpy(), inp["v"].float().numpy(),
                             scale_of(d), rows=[i])[:, :, 0]
    report("decode row", f64(dec), ref)
    report("prefill row", pre[:, :, i], ref)
    assert np.abs(f64(dec) - ref).max() <= TOL["bf16"]
    assert np.abs(pre[:, :, i] - f64(dec)).max() <= 2 * TOL["bf16"]


def test_prefill_full_workload_every_row():
    """The 4096-token causal prefill (B=2, H=64, K=8, d=128) in the launch the
    benchmark times, every output row of every head against the fp64 oracle."""
    w = WORKLOADS["prefill_causal_4k"]
    note("prefill full workload: inputs")
    inp = workload_inputs(w, seed=0)
    note("prefill full workload: GPU")
    out = f64(_run(inp))
    note("prefill full workload: oracle, every row (per sequence and KV head, threaded)")
    scale = scale_of(w.d)
    ref = oracle_by_kv_head(lambda q, k, v: prefill_causal_ref(q, k, v, scale), f64(inp["q"]),
                            inp["k"].float().numpy(), inp["v"].float().numpy())
    r = report("prefill 4k every row", out, ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]
    assert r["max_abs"] <= bf16_bound(ref, _vmax(inp, w.L), weights_in_denominator=True)
