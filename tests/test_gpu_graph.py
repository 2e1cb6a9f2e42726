"""A fused decode step (gqa_decode_append with a caller workspace: no
allocation, no memset, two kernel launches) captured in a HIP graph through
torch.cuda.graph and replayed: after every replay -- with the program's own
eager work and synchronisations between replays -- the output, the caches and
the lengths equal those of the same step run eagerly, bit for bit; the last
step is also checked against the oracle."""
import numpy as np
import pytest
import torch

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd.inputs import decode_inputs
from gpu_util import DEV, TOL, bf16_bound, f64, note, report, scale_of
from oracle import decode_ref

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("H,K,d", [(32, 8, 128), (71, 1, 64)])
def test_graph_replayed_decode_step_equals_eager(H, K, d):
    B, S_max, steps = 4, 512, 4
    lens = [0, 100, 300, 509]
    note(f"graph-captured decode step H={H} K={K} d={d}")
    inp = decode_inputs(B, H, K, d, "bf16", seed=31, lens=lens, s_max=S_max)
    gen = torch.Generator().manual_seed(32)
    qs = [torch.randn((B, H, d), generator=gen).to(torch.bfloat16) for _ in range(steps)]
    kns = [torch.randn((B, K, d), generator=gen).to(torch.bfloat16) for _ in range(steps)]
    vns = [torch.randn((B, K, d), generator=gen).to(torch.bfloat16) for _ in range(steps)]
    sc = scale_of(d)

    # eager state and graph state, separate copies of the same caches
    ek, ev, esl = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV), inp["seq_lens"].to(DEV)
    gk, gv, gsl = ek.clone(), ev.clone(), esl.clone()
    ws_e = torch.empty(gqa.gqa_decode_workspace_bytes(B, H, K, S_max, d), dtype=torch.uint8, device=DEV)
    ws_g = torch.empty_like(ws_e)
    out_e = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    out_g = torch.empty_like(out_e)
    q_g = torch.zeros((B, H, d), dtype=torch.bfloat16, device=DEV)
    kn_g = torch.zeros((B, K, d), dtype=torch.bfloat16, device=DEV)
    vn_g = torch.zeros((B, K, d), dtype=torch.bfloat16, device=DEV)

    # one eager call on scratch copies first, so every kernel is loaded
    # before the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        sk, sv, ssl = gk.clone(), gv.clone(), gsl.clone()
        gqa.gqa_decode_append(q_g, kn_g, vn_g, sk, sv, ssl, out_g, ws_g, S_max, scale=sc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del sk, sv, ssl

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gqa.gqa_decode_append(q_g, kn_g, vn_g, gk, gv, gsl, out_g, ws_g, S_max, scale=sc)
    torch.cuda.synchronize()
    assert torch.equal(gsl, esl)  # capture records, it does not run

    for i in range(steps):
        q_g.copy_(qs[i].to(DEV))
        kn_g.copy_(kns[i].to(DEV))
        vn_g.copy_(vns[i].to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        gqa.gqa_decode_append(qs[i].to(DEV), kns[i].to(DEV), vns[i].to(DEV), ek, ev, esl, out_e, ws_e, S_max,
                              scale=sc)
        torch.cuda.synchronize()
        assert torch.equal(gsl, esl), f"replay {i}: lengths"
        assert torch.equal(out_g, out_e), f"replay {i}: output"
        # bit patterns (rows past the lengths hold NaN, which never compares equal)
        assert torch.equal(gk.view(torch.int16), ek.view(torch.int16)), f"replay {i}: K cache"
        assert torch.equal(gv.view(torch.int16), ev.view(torch.int16)), f"replay {i}: V cache"

    # the state after the last replay against the oracle
    L = gsl.cpu().numpy()
    assert list(L) == [min(n + steps, S_max) for n in lens]  # the last cache fills on the way
    kf, vf = gk.cpu().float().numpy(), gv.cpu().float().numpy()
    ref = decode_ref(f64(qs[-1]), kf, vf, L, sc)
    vmax = max(float(np.abs(vf[b, :, :n]).max()) for b, n in enumerate(L))
    r = report("graph replay", f64(out_g), ref)
    assert r["finite"] and r["max_abs"] <= min(TOL["bf16"], bf16_bound(ref, vmax))
