"""GPU parity of the fused step gqa_decode_append (append + decode in two launches)."""
import numpy as np
import pytest
import torch

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd.inputs import WORKLOADS, decode_inputs, workload_inputs
from gpu_util import DEV, TOL, bf16_bound, f64, note, report, scale_of
from oracle import decode_ref, kv_append_ref

pytestmark = pytest.mark.gpu

_INT = {torch.bfloat16: torch.int16, torch.float32: torch.int32}


def _fused(inp, max_seq_len, out_dtype=None):
    q, kc, vc = inp["q"].to(DEV), inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    sl = inp["seq_lens"].to(DEV)
    B, H, d = q.shape
    K = kc.shape[1]
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, H, K, max_seq_len, d), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, H, d), dtype=out_dtype or q.dtype, device=DEV)
    gqa.gqa_decode_append(q, inp["k_new"].to(DEV), inp["v_new"].to(DEV), kc, vc, sl, out, ws,
                          max_seq_len, scale=scale_of(d))
    torch.cuda.synchronize()
    return out, kc, vc, sl


def _unfused(inp, max_seq_len, out_dtype=None):
    q, kc, vc = inp["q"].to(DEV), inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    sl = inp["seq_lens"].to(DEV)
    B, H, d = q.shape
    K = kc.shape[1]
    gqa.gqa_kv_append(inp["k_new"].to(DEV), inp["v_new"].to(DEV), kc, vc, sl)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, H, K, max_seq_len, d), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, H, d), dtype=out_dtype or q.dtype, device=DEV)
    gqa.gqa_decode(q, kc, vc, sl, out, ws, max_seq_len, scale=scale_of(d))
    torch.cuda.synchronize()
    return out, kc, vc, sl


# B = 130 (three 64-lane chunks of the length scans, the new lengths
# published for all of them), ragged, one empty and one full cache
RAGGED_130 = [0, 310, 1] + [int(x) for x in np.random.RandomState(9).randint(0, 301, 127)]

CASES = [
    # B, H, K, d, lens, S_max, dtype
    (4, 32, 8, 128, [0, 1, 700, 4095], 4096, "bf16"),   # empty, one row, middle, last free row
    (3, 16, 4, 64, [31, 32, 33], 40, "bf16"),
    (2, 64, 8, 128, [511, 2048], 2049, "bf16"),
    (2, 56, 8, 128, [300, 300], 300, "bf16"),           # full caches: no append
    (2, 71, 1, 64, [100, 257], 300, "bf16"),
    (2, 48, 1, 128, [0, 999], 1000, "bf16"),            # G = 48; the last free row
    (1, 128, 2, 64, [333], 400, "bf16"),                # G = 64
    (2, 40, 1, 128, [500, 500], 500, "bf16"),           # G = 40, full caches: no append
    (3, 12, 4, 128, [0, 63, 200], 256, "f32"),
    (2, 16, 16, 64, [64, 64], 64, "f32"),               # full caches, fp32
    (130, 8, 2, 64, RAGGED_130, 310, "bf16"),
]


@pytest.mark.parametrize("B,H,K,d,lens,S_max,dtype", CASES)
def test_fused_step_vs_oracle_and_unfused(B, H, K, d, lens, S_max, dtype):
    note(f"fused step B={B} H={H} K={K} d={d} lens={lens} S_max={S_max} {dtype}")
    inp = decode_inputs(B, H, K, d, dtype, seed=17, lens=lens, s_max=S_max)
    msl = min(max(lens) + 1, S_max)
    out, kc, vc, sl = _fused(inp, msl)
    out2, kc2, vc2, sl2 = _unfused(inp, msl)
    # caches and lengths: bit-identical to the oracle's append and to the unfused path
    it = _INT[inp["k_cache"].dtype]
    k_ref, v_ref, s_ref = kv_append_ref(inp["k_new"].view(it).numpy(), inp["v_new"].view(it).numpy(),
                                        inp["k_cache"].view(it).numpy(), inp["v_cache"].view(it).numpy(),
                                        inp["seq_lens"].numpy())
    assert np.array_equal(sl.cpu().numpy(), s_ref)
    assert np.array_equal(kc.cpu().view(it).numpy(), k_ref) and np.array_equal(vc.cpu().view(it).numpy(), v_ref)
    # same plan, same arithmetic: the fused output equals the unfused one bit for bit
    assert torch.equal(out, out2) and torch.equal(sl, sl2)
    # oracle decode over the oracle-appended caches (bit-identical to kc, vc)
    ref = decode_ref(f64(inp["q"]), kc.cpu().float().numpy(), vc.cpu().float().numpy(), s_ref, scale_of(d))
    r = report("fused", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL[dtype]
    if dtype == "bf16":
        vmax = float(vc.cpu().float().nan_to_num(0.0).abs().max())
        assert r["max_abs"] <= bf16_bound(ref, vmax)


def test_fused_step_full_workload():
    w = WORKLOADS["decode_llama3_8b"]
    inp = workload_inputs(w, seed=0)
    note("fused step on the Llama-3-8B layer")
    out, kc, vc, sl = _fused(inp, w.L + 1)
    assert sl.cpu().tolist() == [w.L + 1] * w.B
    ref = np.zeros(tuple(out.shape))
    for b in range(w.B):
        k2, v2, s2 = kv_append_ref(inp["k_new"][b:b + 1].float().numpy(), inp["v_new"][b:b + 1].float().numpy(),
                                   inp["k_cache"][b:b + 1].float().numpy(), inp["v_cache"][b:b + 1].float().numpy(),
                                   inp["seq_lens"][b:b + 1].numpy())
        ref[b] = decode_ref(f64(inp["q"][b:b + 1]), k2, v2, s2, scale_of(w.d))[0]
        assert torch.equal(kc[b, :, w.L].cpu(), inp["k_new"][b]) and torch.equal(vc[b, :, w.L].cpu(), inp["v_new"][b])
    r = report("fused llama3_8b", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]


def test_fused_step_mqa_workload():
    """The multi-query workload (71 query heads on one KV head, d = 64, 32768
    cached rows) in the launch configuration the benchmark times: the fused
    append + decode through the one-workgroup-per-group pass; every appended
    row checked, sampled sequences against the oracle."""
    w = WORKLOADS["decode_mqa_71h"]
    inp = workload_inputs(w, seed=0)
    note("fused step on the 71-head multi-query layer")
    out, kc, vc, sl = _fused(inp, w.L + 1)
    assert sl.cpu().tolist() == [w.L + 1] * w.B
    assert torch.equal(kc[:, :, w.L].cpu(), inp["k_new"]) and torch.equal(vc[:, :, w.L].cpu(), inp["v_new"])
    for b in (0, 13, w.B - 1):
        k2, v2, s2 = kv_append_ref(inp["k_new"][b:b + 1].float().numpy(), inp["v_new"][b:b + 1].float().numpy(),
                                   inp["k_cache"][b:b + 1].float().numpy(), inp["v_cache"][b:b + 1].float().numpy(),
                                   inp["seq_lens"][b:b + 1].numpy())
        ref = decode_ref(f64(inp["q"][b:b + 1]), k2, v2, s2, scale_of(w.d))
        r = report(f"fused mqa b={b}", f64(out[b:b + 1]), ref)
        assert r["finite"] and r["max_abs"] <= TOL["bf16"]
        assert r["max_abs"] <= bf16_bound(ref, float(np.abs(v2[0, :, :w.L + 1]).max()))


@pytest.mark.parametrize("H,K,d", [(16, 4, 128), (48, 1, 128), (71, 1, 64)])
def test_many_fused_steps_until_a_cache_fills(H, K, d):
    """40 consecutive fused decode steps on a ragged batch whose shortest
    cache fills up on the way: after every step the lengths match the
    oracle's appends, the output matches the oracle's decode, and at the end
    the caches are bit-identical to the oracle's (full caches stop growing).
    G = 48 and 71 take the one-workgroup-per-group pass, whose first wave
    writes the new rows into the cache before the group's copies start."""
    B, S_max = 3, 64
    note(f"40 fused steps H={H} K={K} d={d}")
    lens = [40, 0, 30]
    inp = decode_inputs(B, H, K, d, "bf16", seed=121, lens=lens, s_max=S_max)
    g = torch.Generator().manual_seed(122)
    it = torch.int16
    kc, vc, sl = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV), inp["seq_lens"].to(DEV)
    k_ref, v_ref = inp["k_cache"].view(it).numpy(), inp["v_cache"].view(it).numpy()
    s_ref = inp["seq_lens"].numpy()
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, H, K, S_max, d), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, H, d), dtype=torch.float32, device=DEV)
    for step in range(40):
        q = torch.randn((B, H, d), generator=g).to(torch.bfloat16)
        kn = torch.randn((B, K, d), generator=g).to(torch.bfloat16)
        vn = torch.randn((B, K, d), generator=g).to(torch.bfloat16)
        gqa.gqa_decode_append(q.to(DEV), kn.to(DEV), vn.to(DEV), kc, vc, sl, out, ws, S_max, scale=scale_of(d))
        k_ref, v_ref, s_ref = kv_append_ref(kn.view(it).numpy(), vn.view(it).numpy(), k_ref, v_ref, s_ref)
        torch.cuda.synchronize()
        assert sl.cpu().tolist() == list(s_ref), f"step {step}"
        kf = torch.from_numpy(k_ref.copy()).view(torch.bfloat16).float().numpy()
        vf = torch.from_numpy(v_ref.copy()).view(torch.bfloat16).float().numpy()
        ref = decode_ref(f64(q), kf, vf, s_ref, scale_of(d))
        vmax = max(float(np.abs(vf[b, :, :L]).max()) if L else 0.0 for b, L in enumerate(s_ref))
        err = float(np.abs(f64(out) - ref).max())
        assert np.isfinite(err) and err <= bf16_bound(ref, vmax), f"step {step}: {err}"
    assert list(s_ref) == [S_max, 40, S_max]
    assert np.array_equal(kc.cpu().view(it).numpy(), k_ref) and np.array_equal(vc.cpu().view(it).numpy(), v_ref)
