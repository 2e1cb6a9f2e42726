"""GPU parity of the fused K/V projection + append (gqa_kv_project_append)
against the fp64 CPU oracle.  Bound per element: the fp32 sum of d_model
exact bf16 products errs by at most d_model * 2^-24 * sum |x w|, and the
bf16 rounding of the result by u = 2^-8 of its magnitude."""
import numpy as np
import pytest
import torch

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd.inputs import WORKLOADS, projection_inputs
from gpu_util import BF16_U, DEV, TOL, note, report
from oracle import kv_project_append_ref, kv_project_ref

pytestmark = pytest.mark.gpu


def _bound(x, w, dm):
    xa = np.abs(x.float().numpy())
    wa = np.abs(w.float().numpy())
    ka, va = kv_project_ref(xa, wa)
    return ka, va


CASES = [
    # B, T, d_model, K, d, S_max, lens
    (3, 1, 4096, 8, 128, 20, [0, 7, 19]),     # decode: one token; the last cache is full
    (2, 5, 512, 4, 64, 16, [3, 12]),          # five tokens; the second has no room
    (1, 40, 1024, 2, 128, 64, [10]),          # 40 tokens: three token tiles, ragged
    (2, 1, 256, 1, 128, 8, [1, 2]),           # one KV head, small d_model
    (2, 3, 896, 2, 64, 9, [0, 4]),            # d_model = 28 k-steps: uneven split over the waves
    (1, 2, 32, 2, 128, 4, [1]),               # one k-step: most waves idle
    (1, 300, 512, 2, 128, 400, [50]),         # 300 tokens: 9600 row words, separate length update
]


@pytest.mark.parametrize("B,T,dm,K,d,S_max,lens", CASES)
def test_project_append(B, T, dm, K, d, S_max, lens):
    note(f"project B={B} T={T} dm={dm} K={K} d={d} lens={lens}")
    inp = projection_inputs(B, T, dm, K, d, seed=111)
    kc = torch.full((B, K, S_max, d), float("nan"), dtype=torch.bfloat16)
    vc = torch.full((B, K, S_max, d), float("nan"), dtype=torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32)
    dk, dv, ds = kc.to(DEV), vc.to(DEV), sl.to(DEV)
    ws = torch.empty(gqa.gqa_kv_project_workspace_bytes(B, T, dm, K, d), dtype=torch.uint8, device=DEV)
    gqa.gqa_kv_project_append(inp["x"].to(DEV), inp["w_kv"].to(DEV), dk, dv, ds, ws)
    torch.cuda.synchronize()
    k2, v2, s2 = kv_project_append_ref(inp["x"].float().numpy(), inp["w_kv"].float().numpy(),
                                       kc.float().numpy(), vc.float().numpy(), sl.numpy())
    assert ds.cpu().tolist() == list(s2)
    ka, va = _bound(inp["x"], inp["w_kv"], dm)
    gk, gv = dk.cpu().float().numpy(), dv.cpu().float().numpy()
    for b, L in enumerate(lens):
        if L + T > S_max:   # no room: untouched (all NaN)
            assert np.isnan(gk[b]).all() and np.isnan(gv[b]).all()
            continue
        assert np.isnan(gk[b, :, :L]).all() and np.isnan(gk[b, :, L + T:]).all()
        for got, ref, acc in ((gk[b, :, L:L + T], k2[b, :, L:L + T], ka[b]), (gv[b, :, L:L + T], v2[b, :, L:L + T], va[b])):
            e1 = dm * 2.0 ** -24 * acc
            bound = BF16_U * (np.abs(ref) + e1) + e1 + 1e-30
            err = np.abs(got - ref)
            assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3f}"
            report("project", got, ref)


def test_project_full_workload():
    """Llama-3-8B layer: 16 decode tokens, d_model 4096, W_KV [8, 256, 4096],
    appended at position 8192 of an 8193-row cache."""
    w = WORKLOADS["kv_project_llama3_8b"]
    dm, T = w.extra["d_model"], w.extra["T"]
    inp = projection_inputs(w.B, T, dm, w.K, w.d, seed=0)
    S_max = w.L + 1
    dk = torch.zeros((w.B, w.K, S_max, w.d), dtype=torch.bfloat16, device=DEV)
    dv = torch.zeros_like(dk)
    ds = torch.full((w.B,), w.L, dtype=torch.int32, device=DEV)
    ws = torch.empty(gqa.gqa_kv_project_workspace_bytes(w.B, T, dm, w.K, w.d), dtype=torch.uint8, device=DEV)
    gqa.gqa_kv_project_append(inp["x"].to(DEV), inp["w_kv"].to(DEV), dk, dv, ds, ws)
    torch.cuda.synchronize()
    assert ds.cpu().tolist() == [w.L + 1] * w.B
    kr, vr = kv_project_ref(inp["x"].float().numpy(), inp["w_kv"].float().numpy())
    ka, va = _bound(inp["x"], inp["w_kv"], dm)
    for got, ref, acc in ((dk[:, :, w.L:w.L + 1].cpu().float().numpy(), kr, ka),
                          (dv[:, :, w.L:w.L + 1].cpu().float().numpy(), vr, va)):
        e1 = dm * 2.0 ** -24 * acc
        assert np.all(np.abs(got - ref) <= BF16_U * (np.abs(ref) + e1) + e1)
        r = report("project llama3_8b", got, ref)
        assert r["max_abs"] <= TOL["bf16"]
    assert torch.count_nonzero(dk[:, :, :w.L]).item() == 0


@pytest.mark.parametrize("B,T,dm,K,d", [(16, 1, 4096, 8, 128), (3, 7, 1024, 4, 64), (1, 33, 2048, 2, 128)])
def test_project_rows(B, T, dm, K, d):
    """gqa_kv_project: rows [B, K, T, d] against the oracle, element bound."""
    inp = projection_inputs(B, T, dm, K, d, seed=113)
    ko = torch.empty((B, K, T, d), dtype=torch.bfloat16, device=DEV)
    vo = torch.empty_like(ko)
    gqa.gqa_kv_project(inp["x"].to(DEV), inp["w_kv"].to(DEV), ko, vo)
    torch.cuda.synchronize()
    kr, vr = kv_project_ref(inp["x"].float().numpy(), inp["w_kv"].float().numpy())
    ka, va = _bound(inp["x"], inp["w_kv"], dm)
    for got, ref, acc in ((ko.cpu().float().numpy(), kr, ka), (vo.cpu().float().numpy(), vr, va)):
        e1 = dm * 2.0 ** -24 * acc
        assert np.all(np.abs(got - ref) <= BF16_U * (np.abs(ref) + e1) + e1)
        report("project rows", got, ref)


def test_project_then_fused_decode_step():
    """A decode step from hidden states: gqa_kv_project gives k_new, v_new and
    gqa_decode_append appends them inside the attention pass; the caches
    equal the projected rows and the output matches the oracle's decode over
    the oracle-appended caches (the projected rows as the GPU rounded them)."""
    from grouped_query_kv_amd.inputs import decode_inputs
    from gpu_util import bf16_bound, f64, scale_of
    from oracle import decode_ref, kv_append_ref
    B, H, K, d, dm = 4, 32, 8, 128, 1024
    inp = decode_inputs(B, H, K, d, "bf16", seed=114, lens=[100, 1, 777, 0])
    pj = projection_inputs(B, 1, dm, K, d, seed=115)
    kn = torch.empty((B, K, 1, d), dtype=torch.bfloat16, device=DEV)
    vn = torch.empty_like(kn)
    gqa.gqa_kv_project(pj["x"].to(DEV), pj["w_kv"].to(DEV), kn, vn)
    kc, vc, sl = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV), inp["seq_lens"].to(DEV)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, H, K, 778, d), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    gqa.gqa_decode_append(inp["q"].to(DEV), kn[:, :, 0].contiguous(), vn[:, :, 0].contiguous(), kc, vc, sl, out, ws,
                          778, scale=scale_of(d))
    torch.cuda.synchronize()
    kr, vr = kv_project_ref(pj["x"].float().numpy(), pj["w_kv"].float().numpy())
    ka, va = _bound(pj["x"], pj["w_kv"], dm)
    for got, ref, acc in ((kn.cpu().float().numpy(), kr, ka), (vn.cpu().float().numpy(), vr, va)):
        e1 = dm * 2.0 ** -24 * acc
        assert np.all(np.abs(got - ref) <= BF16_U * (np.abs(ref) + e1) + e1)
    k2, v2, s2 = kv_append_ref(kn[:, :, 0].cpu().float().numpy(), vn[:, :, 0].cpu().float().numpy(),
                               inp["k_cache"].float().numpy(), inp["v_cache"].float().numpy(), inp["seq_lens"].numpy())
    assert sl.cpu().tolist() == list(s2)
    ref = decode_ref(f64(inp["q"]), k2, v2, s2, scale_of(d))
    r = report("project + fused decode", f64(out), ref)
    vmax = max(float(np.nan_to_num(np.abs(v2[b, :, :L])).max()) for b, L in enumerate(s2))
    assert r["finite"] and r["max_abs"] <= bf16_bound(ref, vmax)
