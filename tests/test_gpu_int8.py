"""GPU parity of the int8 KV-cache path (gqa_kv_quantize_int8,
gqa_kv_append_int8, gqa_decode_int8) against the fp64 CPU oracle.  Codes and
scales are integer / fp32 decisions taken in fp32 on both sides and must
match bit for bit; the decode output is held to the bf16 bound."""
import numpy as np
import pytest
import torch

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd.inputs import WORKLOADS, decode_inputs, workload_inputs
from gpu_util import DEV, TOL, bf16_bound, f64, guarded, guards_intact, note, report, scale_of
from oracle import decode_int8_ref, dequantize_int8_ref, kv_append_int8_ref, quantize_int8_ref

pytestmark = pytest.mark.gpu


def _round4(n):
    return (n + 3) // 4 * 4


def _quantize_gpu(x):
    xd = x.to(DEV)
    codes = torch.empty(x.shape, dtype=torch.int8, device=DEV)
    scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=DEV)
    gqa.gqa_kv_quantize_int8(xd, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu(), scales.cpu()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_quantize_bit_exact(dtype, d):
    g = torch.Generator().manual_seed(71)
    rows = 1000 + 7  # not a multiple of the rows per workgroup
    x = torch.randn((rows, d), generator=g) * torch.exp(torch.randn((rows, 1), generator=g) * 3)
    x[5] = 0.0                                    # zero row
    x[6, :] = 0.0
    x[6, 3] = -1e-30                              # tiny amax
    x[7] = torch.arange(d) - d / 2                # exact ties after scaling
    x[8, 0] = 127.0
    x[8, 1:] = torch.tensor([2.5, -2.5, 3.5, 0.5, -0.5, 1.5, 126.5] * (d // 7 + 1))[: d - 1]
    x = x.to(dtype)
    note(f"quantize rows={rows} d={d} {dtype}")
    codes, scales = _quantize_gpu(x)
    c_ref, s_ref = quantize_int8_ref(x.float().numpy())
    assert np.array_equal(codes.numpy(), c_ref)
    assert np.array_equal(scales.numpy().view(np.uint32), s_ref.view(np.uint32))
    c1, s1 = _quantize_gpu(x[:1])                 # a single row
    assert np.array_equal(c1.numpy(), c_ref[:1]) and np.array_equal(s1.numpy(), s_ref[:1])


def _int8_case(B, H, K, d, lens, seed, s_max=None):
    """bf16 workload caches quantised on both sides; rows past L_b poisoned."""
    s_max = _round4(s_max or (max(lens) + 1))
    inp = decode_inputs(B, H, K, d, "bf16", seed=seed, lens=lens, s_max=s_max, nan_tail=False)
    kc, ks = _quantize_gpu(inp["k_cache"])
    vc, vs = _quantize_gpu(inp["v_cache"])
    kc_r, ks_r = quantize_int8_ref(inp["k_cache"].float().numpy())
    vc_r, vs_r = quantize_int8_ref(inp["v_cache"].float().numpy())
    assert np.array_equal(kc.numpy(), kc_r) and np.array_equal(vc.numpy(), vc_r)
    assert np.array_equal(ks.numpy(), ks_r) and np.array_equal(vs.numpy(), vs_r)
    for b, L in enumerate(lens):  # never-read rows: junk codes, NaN scales
        for t in (kc, vc):
            t[b, :, L:] = 127
        for t in (ks, vs):
            t[b, :, L:] = float("nan")
    return inp, kc, vc, ks, vs


def _run(inp, kc, vc, ks, vs, msl, out_dtype=torch.bfloat16, sl=None):
    B, H, d = inp["q"].shape
    K = kc.shape[1]
    ws = torch.empty(max(gqa.gqa_decode_workspace_bytes(B, H, K, msl, d), 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, H, d), dtype=out_dtype, device=DEV)
    gqa.gqa_decode_int8(inp["q"].to(DEV), kc.to(DEV), vc.to(DEV), ks.to(DEV), vs.to(DEV),
                        (inp["seq_lens"] if sl is None else sl).to(DEV), out, ws, msl, scale=scale_of(d))
    torch.cuda.synchronize()
    return out


def _vmax(vc, vs, lens):
    v = dequantize_int8_ref(vc.numpy(), vs.numpy())
    return max(float(np.abs(v[b, :, :L]).max()) if L else 0.0 for b, L in enumerate(lens))


RAGGED_130 = [0, 300, 1] + [int(x) for x in np.random.RandomState(6).randint(0, 301, 127)]

# a large ragged batch (>= 256 sequence-head units), lengths 0..600
RAGGED_40 = [0, 1, 600] + [int(x) for x in np.random.RandomState(5).randint(0, 601, 37)]

CASES = [
    # B, H, K, d, lens
    (3, 32, 8, 128, [1, 33, 1000]),
    (4, 64, 8, 128, [0, 16, 17, 3000]),
    (2, 16, 4, 64, [31, 2100]),
    (2, 56, 8, 128, [300, 5]),         # G = 7
    (2, 8, 8, 128, [2, 97]),           # K = H (MHA)
    (2, 32, 1, 128, [129, 4100]),      # K = 1 (MQA), G = 32
    (1, 71, 1, 64, [257]),             # G = 71: five head blocks
    (1, 144, 1, 64, [300]),            # G = 144: nine head blocks (one wave per block)
    (40, 16, 8, 64, RAGGED_40),        # 320 units: one-dimensional grid, partition slowest
    (130, 8, 2, 64, RAGGED_130),       # B = 130: three 64-lane chunks of the length scans
    (2, 64, 1, 128, [900, 33]),        # d = 128, G = 64: four waves
    (1, 100, 1, 128, [700]),           # d = 128, G = 100: seven waves, the last with four heads
    (1, 128, 1, 128, [1500]),          # d = 128, G = 128: eight waves
]


@pytest.mark.parametrize("B,H,K,d,lens", CASES)
def test_int8_decode_shapes(B, H, K, d, lens):
    note(f"int8 decode B={B} H={H} K={K} d={d} lens={lens}")
    inp, kc, vc, ks, vs = _int8_case(B, H, K, d, lens, seed=81)
    out = _run(inp, kc, vc, ks, vs, max(lens))
    ref = decode_int8_ref(f64(inp["q"]), kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(),
                          inp["seq_lens"].numpy(), scale_of(d))
    r = report("int8", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]
    assert r["max_abs"] <= bf16_bound(ref, _vmax(vc, vs, lens))
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.count_nonzero(out[b]).item() == 0


@pytest.mark.parametrize("qmul", [2.0 ** 17, 2.0 ** -20])
def test_int8_decode_query_range(qmul):
    """Queries 2^17 times and 2^-20 times the workload's: scores spread so far
    that the softmax is one-hot, and so little that the weights are nearly
    uniform."""
    B, H, K, d, lens = 2, 32, 8, 128, [257, 40]
    note(f"int8 decode query range x{qmul}")
    inp, kc, vc, ks, vs = _int8_case(B, H, K, d, lens, seed=83)
    inp["q"] = (inp["q"].float() * qmul).to(torch.bfloat16)
    out = _run(inp, kc, vc, ks, vs, max(lens))
    ref = decode_int8_ref(f64(inp["q"]), kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(),
                          inp["seq_lens"].numpy(), scale_of(d))
    r = report(f"int8 q x{qmul}", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]
    assert r["max_abs"] <= bf16_bound(ref, _vmax(vc, vs, lens))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_int8_out_dtype_and_guards(out_dtype):
    B, H, K, d, lens = 2, 32, 8, 128, [500, 77]
    inp, kc, vc, ks, vs = _int8_case(B, H, K, d, lens, seed=82)
    out, buf, guard = guarded((B, H, d), out_dtype)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, H, K, 500, d), dtype=torch.uint8, device=DEV)
    gqa.gqa_decode_int8(inp["q"].to(DEV), kc.to(DEV), vc.to(DEV), ks.to(DEV), vs.to(DEV),
                        inp["seq_lens"].to(DEV), out, ws, 500, scale=scale_of(d))
    torch.cuda.synchronize()
    assert guards_intact(buf, guard, out_dtype)
    ref = decode_int8_ref(f64(inp["q"]), kc.numpy(), vc.numpy(), ks.numpy(), vs.numpy(),
                          inp["seq_lens"].numpy(), scale_of(d))
    r = report(f"int8 {out_dtype}", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= bf16_bound(ref, _vmax(vc, vs, lens))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_int8_append_bit_exact(dtype):
    B, K, d, S = 4, 8, 128, 12
    g = torch.Generator().manual_seed(91)
    kc = torch.randint(-127, 128, (B, K, S, d), generator=g, dtype=torch.int8)
    vc = torch.randint(-127, 128, (B, K, S, d), generator=g, dtype=torch.int8)
    ks = torch.rand((B, K, S), generator=g)
    vs = torch.rand((B, K, S), generator=g)
    kn = (torch.randn((B, K, d), generator=g) * 3).to(dtype)
    vn = (torch.randn((B, K, d), generator=g) * 0.1).to(dtype)
    kn[1, 2] = 0.0                                 # a zero row
    sl = torch.tensor([0, 5, 11, S], dtype=torch.int32)  # last one full
    ref = kv_append_int8_ref(kn.float().numpy(), vn.float().numpy(), kc.numpy(), vc.numpy(), ks.numpy(),
                             vs.numpy(), sl.numpy())
    dev = [t.to(DEV) for t in (kc, vc, ks, vs, sl)]
    note(f"int8 append {dtype}")
    gqa.gqa_kv_append_int8(kn.to(DEV), vn.to(DEV), *dev)
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in dev]
    assert got[4].tolist() == list(ref[4]) == [1, 6, 12, S]
    for a, b in zip(got[:2], ref[:2]):
        assert np.array_equal(a, b)
    for a, b in zip(got[2:4], ref[2:4]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_int8_full_workload():
    """Llama-3-8B layer: bf16 cache quantised on the GPU (codes and scales
    bit-exact against the oracle), then one decode step with the quantising
    append fused in -- the call the benchmark times."""
    w = WORKLOADS["decode_int8_llama3_8b"]
    note("int8 full workload: inputs")
    inp = workload_inputs(w, seed=0, s_max=_round4(w.L + 1))
    B, H, d = inp["q"].shape
    K, S = w.K, inp["k_cache"].shape[2]
    kc = torch.empty((B, K, S, d), dtype=torch.int8, device=DEV)
    vc = torch.empty_like(kc)
    ks = torch.empty((B, K, S), dtype=torch.float32, device=DEV)
    vs = torch.empty_like(ks)
    kb, vb = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV)
    # rows past L are NaN in the workload's bf16 cache: quantise rows [0, L)
    # of each sequence through a contiguous staging buffer
    L = w.L
    kc.zero_(), vc.zero_(), ks.zero_(), vs.zero_()
    for b in range(B):
        for src, codes, sc in ((kb, kc, ks), (vb, vc, vs)):
            c_tmp = torch.empty((K, L, d), dtype=torch.int8, device=DEV)
            s_tmp = torch.empty((K, L), dtype=torch.float32, device=DEV)
            gqa.gqa_kv_quantize_int8(src[b, :, :L].contiguous(), c_tmp, s_tmp)
            codes[b, :, :L] = c_tmp
            sc[b, :, :L] = s_tmp
    sl = inp["seq_lens"].to(DEV)
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, H, K, L + 1, d), dtype=torch.uint8, device=DEV)
    note("int8 full workload: GPU step (quantising append fused into the decode, as benchmarked)")
    gqa.gqa_decode_append_int8(inp["q"].to(DEV), inp["k_new"].to(DEV), inp["v_new"].to(DEV), kc, vc, ks, vs, sl,
                               out, ws, L + 1, scale=scale_of(d))
    torch.cuda.synchronize()
    assert sl.cpu().tolist() == [L + 1] * B
    note("int8 full workload: oracle")
    ref = np.zeros((B, H, d))
    vmax = 0.0
    for b in range(B):
        c = {}
        for nm in ("k", "v"):
            codes, sc = quantize_int8_ref(inp[f"{nm}_cache"][b:b + 1, :, :L].float().numpy())
            c[nm] = (np.concatenate([codes, np.zeros((1, K, S - L, d), np.int8)], axis=2),
                     np.concatenate([sc, np.zeros((1, K, S - L), np.float32)], axis=2))
        out_c = kv_append_int8_ref(inp["k_new"][b:b + 1].float().numpy(), inp["v_new"][b:b + 1].float().numpy(),
                                   c["k"][0], c["v"][0], c["k"][1], c["v"][1], np.array([L]))
        kc_r, vc_r, ks_r, vs_r, s_r = out_c
        assert np.array_equal(kc[b:b + 1, :, :L + 1].cpu().numpy(), kc_r[:, :, :L + 1])
        assert np.array_equal(vs[b:b + 1, :, :L + 1].cpu().numpy(), vs_r[:, :, :L + 1])
        ref[b] = decode_int8_ref(f64(inp["q"][b:b + 1]), kc_r, vc_r, ks_r, vs_r, s_r, scale_of(d))[0]
        vmax = max(vmax, float(np.abs(dequantize_int8_ref(vc_r[:, :, :L + 1], vs_r[:, :, :L + 1])).max()))
    r = report("int8 llama3_8b", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]
    assert r["max_abs"] <= bf16_bound(ref, vmax)


FUSED_CASES = [
    # B, H, K, d, lens, s_max, steps
    (3, 32, 8, 128, [1, 33, 1000], None, 1),
    (4, 64, 8, 128, [0, 16, 17, 3000], None, 1),
    (2, 16, 4, 64, [31, 2100], None, 1),
    (2, 32, 1, 128, [129, 4100], None, 1),        # G = 32: two head blocks
    (1, 71, 1, 64, [257], None, 1),               # G = 71: five head blocks
    (4, 32, 8, 128, [64, 3, 4, 95], None, 1),     # new row at chunk / scale-group edges
    (3, 32, 8, 128, [12, 5, 12], 12, 1),          # full caches: no append
    (2, 32, 8, 128, [60, 3], 64, 8),              # eight steps; the first cache fills up
    (40, 16, 8, 64, RAGGED_40, None, 2),          # 320 units: one-dimensional grid
    (3, 96, 2, 128, [95, 0, 60], 104, 10),        # G = 48 (one workgroup per group): ten steps,
                                                  # the first cache fills up, new rows at group edges
    (2, 71, 1, 64, [31, 32], None, 3),            # G = 71, d = 64: chunk edges, three steps
]


@pytest.mark.parametrize("B,H,K,d,lens,s_max,steps", FUSED_CASES)
def test_int8_fused_append_matches_unfused(B, H, K, d, lens, s_max, steps):
    """gqa_decode_append_int8 == gqa_kv_append_int8 + gqa_decode_int8: the
    same codes, scales and lengths and the same output bits, step after step;
    and the output within the bf16 bound of the oracle on the grown cache."""
    note(f"int8 fused append B={B} H={H} K={K} d={d} lens={lens} s_max={s_max} steps={steps}")
    inp, kc, vc, ks, vs = _int8_case(B, H, K, d, lens, seed=83, s_max=s_max)
    S = kc.shape[2]
    msl = min(max(lens) + steps, S)
    fused = [t.to(DEV) for t in (kc, vc, ks, vs, inp["seq_lens"])]
    split = [t.clone() for t in fused]
    ref = [t.numpy().copy() for t in (kc, vc, ks, vs, inp["seq_lens"])]
    nbytes = gqa.gqa_decode_workspace_bytes(B, H, K, msl, d)
    ws_f = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ws_s = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    g = torch.Generator().manual_seed(84)
    for step in range(steps):
        q = torch.randn((B, H, d), generator=g).to(torch.bfloat16)
        kn = (torch.randn((B, K, d), generator=g) * 2).to(torch.bfloat16)
        vn = torch.randn((B, K, d), generator=g).to(torch.bfloat16)
        out_f = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
        out_s = torch.empty_like(out_f)
        qd, knd, vnd = q.to(DEV), kn.to(DEV), vn.to(DEV)
        gqa.gqa_decode_append_int8(qd, knd, vnd, *fused, out_f, ws_f, msl, scale=scale_of(d))
        gqa.gqa_kv_append_int8(knd, vnd, *split)
        gqa.gqa_decode_int8(qd, *split[:4], split[4], out_s, ws_s, msl, scale=scale_of(d))
        torch.cuda.synchronize()
        ref = list(kv_append_int8_ref(kn.float().numpy(), vn.float().numpy(), *ref))
        got = [t.cpu().numpy() for t in fused]
        assert got[4].tolist() == split[4].cpu().tolist() == list(ref[4])
        for a, s2, r in zip(got[:2], split[:2], ref[:2]):
            assert np.array_equal(a, s2.cpu().numpy()) and np.array_equal(a, r)
        for a, s2, r in zip(got[2:4], split[2:4], ref[2:4]):
            u = a.view(np.uint32)
            assert np.array_equal(u, s2.cpu().numpy().view(np.uint32)) and np.array_equal(u, r.view(np.uint32))
        assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
        o_ref = decode_int8_ref(f64(q), ref[0], ref[1], ref[2], ref[3], ref[4], scale_of(d))
        r = report(f"int8 fused step {step}", f64(out_f), o_ref)
        assert r["finite"] and r["max_abs"] <= bf16_bound(o_ref, _vmax(torch.from_numpy(ref[1]),
                                                                       torch.from_numpy(ref[3]), ref[4]))
