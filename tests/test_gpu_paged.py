"""GPU parity of the paged-cache path (gqa_decode_paged, gqa_kv_append_paged)
against the fp64 CPU oracle."""
import numpy as np
import pytest
import torch

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd.inputs import WORKLOADS, decode_inputs, paged_layout, workload_inputs
from gpu_util import DEV, TOL, bf16_bound, f64, guarded, guards_intact, note, report, scale_of
from oracle import decode_paged_ref, kv_append_paged_ref

pytestmark = pytest.mark.gpu

_INT = {torch.bfloat16: torch.int16, torch.float32: torch.int32}


def _np(t):
    return t.float().numpy()


def _vmax(pool):
    return float(pool.float().nan_to_num(0.0).abs().max())


def _run(p, msl, out_dtype=torch.bfloat16):
    q = p["q"].to(DEV)
    kp, vp = p["k_pool"].to(DEV), p["v_pool"].to(DEV)
    bt, sl = p["block_table"].to(DEV), p["seq_lens"].to(DEV)
    B, H, d = q.shape
    K = kp.shape[1]
    ws = torch.empty(max(gqa.gqa_decode_paged_workspace_bytes(B, H, K, msl, d, p["block_size"]), 16),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((B, H, d), dtype=out_dtype, device=DEV)
    gqa.gqa_decode_paged(q, kp, vp, bt, sl, out, ws, msl, scale=scale_of(d))
    torch.cuda.synchronize()
    return out


def _ref(p):
    return decode_paged_ref(f64(p["q"]), _np(p["k_pool"]), _np(p["v_pool"]), p["block_table"].numpy(),
                            p["seq_lens"].numpy(), scale_of(p["q"].shape[-1]))


CASES = [
    # B, H, K, d, lens, block_size
    (3, 32, 8, 128, [1, 33, 1000], 16),
    (4, 64, 8, 128, [0, 16, 17, 3000], 16),   # empty, block edge, several partitions
    (2, 16, 4, 64, [31, 2100], 32),
    (2, 56, 8, 128, [300, 5], 64),            # G = 7
    (2, 8, 8, 128, [2, 97], 16),              # K = H (MHA)
    (2, 32, 1, 128, [129, 4100], 48),         # K = 1 (MQA), G = 32, block_size 48
    (1, 71, 1, 64, [257], 16),                # G = 71: five head blocks
    (2, 48, 1, 128, [777, 31], 32),           # G = 48: three head blocks
    (1, 128, 2, 64, [1500], 16),              # G = 64: four head blocks
    # partitions capped at 62 blocks of 16 rows (992 positions)
    (40, 8, 8, 64, [8000 + 37 * i for i in range(40)], 16),
    # B = 130: three 64-lane chunks of the length scans, ragged, an empty sequence
    (130, 8, 2, 64, [0, 300, 1] + [int(x) for x in np.random.RandomState(4).randint(0, 301, 127)], 16),
]


@pytest.mark.parametrize("B,H,K,d,lens,bs", CASES)
def test_paged_decode_shapes(B, H, K, d, lens, bs):
    note(f"paged decode B={B} H={H} K={K} d={d} max_len={max(lens)} bs={bs}")
    inp = decode_inputs(B, H, K, d, "bf16", seed=21, lens=lens)
    p = paged_layout(inp, bs, seed=22, spare_blocks=5)
    out = _run(p, max(lens))
    ref = _ref(p)
    r = report("paged", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]
    assert r["max_abs"] <= bf16_bound(ref, _vmax(p["v_pool"]))
    for b, L in enumerate(lens):
        if L == 0:
            assert torch.count_nonzero(out[b]).item() == 0


def test_paged_shared_prefix_blocks_and_guards():
    """Two sequences share their first blocks (a common prompt); the output is
    written exactly in place, fp32 or bf16."""
    B, H, K, d, bs = 3, 32, 8, 128, 16
    inp = decode_inputs(B, H, K, d, "bf16", seed=31, lens=[700, 700, 650])
    p = paged_layout(inp, bs, seed=32, spare_blocks=2)
    bt = p["block_table"].clone()
    bt[1, :20] = bt[0, :20]      # sequence 1 reads sequence 0's first 320 rows
    bt[2, 5] = bt[2, 4]          # a block listed twice in one table
    p["block_table"] = bt
    p["q"][1] = p["q"][0]
    for out_dtype in (torch.float32, torch.bfloat16):
        q = p["q"].to(DEV)
        kp, vp = p["k_pool"].to(DEV), p["v_pool"].to(DEV)
        bt_d, sl = bt.to(DEV), p["seq_lens"].to(DEV)
        out, buf, guard = guarded((B, H, d), out_dtype)
        ws = torch.empty(gqa.gqa_decode_paged_workspace_bytes(B, H, K, 700, d, bs), dtype=torch.uint8, device=DEV)
        gqa.gqa_decode_paged(q, kp, vp, bt_d, sl, out, ws, 700, scale=scale_of(d))
        torch.cuda.synchronize()
        assert guards_intact(buf, guard, out_dtype)
        ref = _ref(p)
        r = report(f"shared {out_dtype}", f64(out), ref)
        assert r["finite"] and r["max_abs"] <= TOL["bf16"]
        assert r["max_abs"] <= bf16_bound(ref, _vmax(p["v_pool"]))


def test_paged_matches_contiguous_decode():
    """The same cache, paged or contiguous, gives the same attention (both
    within the bf16 bound of the oracle and of each other)."""
    B, H, K, d = 2, 32, 8, 128
    inp = decode_inputs(B, H, K, d, "bf16", seed=41, lens=[5000, 1234])
    p = paged_layout(inp, 16, seed=42)
    out_p = _run(p, 5000)
    q, kc, vc, sl = (inp[n].to(DEV) for n in ("q", "k_cache", "v_cache", "seq_lens"))
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, H, K, 5000, d), dtype=torch.uint8, device=DEV)
    out_c = torch.empty_like(out_p)
    gqa.gqa_decode(q, kc, vc, sl, out_c, ws, 5000, scale=scale_of(d))
    torch.cuda.synchronize()
    ref = _ref(p)
    b = bf16_bound(ref, _vmax(p["v_pool"]))
    assert report("paged", f64(out_p), ref)["max_abs"] <= b
    assert report("contiguous", f64(out_c), ref)["max_abs"] <= b


def test_paged_wide_groups_at_the_block_cap():
    """Groups of 48 query heads (three 16-head blocks sharing each K/V chunk)
    over long ragged sequences, where the paged partitions reach their cap
    of 62 blocks of 16 rows (the contiguous decode of the same cache splits
    it into longer partitions): sampled sequences of both match the oracle."""
    B, H, K, d = 64, 96, 2, 64
    lens = [7900 + 3 * i for i in range(B)]
    note(f"paged wide groups at the block cap B={B} H={H} K={K} d={d}")
    inp = decode_inputs(B, H, K, d, "bf16", seed=47, lens=lens)
    p = paged_layout(inp, 16, seed=48)
    msl = max(lens)
    out_p = _run(p, msl)
    q, kc, vc, sl = (inp[n].to(DEV) for n in ("q", "k_cache", "v_cache", "seq_lens"))
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, H, K, msl, d), dtype=torch.uint8, device=DEV)
    out_c = torch.empty_like(out_p)
    gqa.gqa_decode(q, kc, vc, sl, out_c, ws, msl, scale=scale_of(d))
    torch.cuda.synchronize()
    for b in (0, 37, B - 1):
        sub = paged_layout({"k_cache": inp["k_cache"][b:b + 1], "v_cache": inp["v_cache"][b:b + 1]}, 16,
                           shuffle=False)
        ref = decode_paged_ref(f64(inp["q"][b:b + 1]), _np(sub["k_pool"]), _np(sub["v_pool"]),
                               sub["block_table"].numpy(), np.array([lens[b]]), scale_of(d))
        bound = bf16_bound(ref, _vmax(sub["v_pool"]))
        for name, out in (("paged", out_p), ("contiguous", out_c)):
            r = report(f"wide {name} b={b}", f64(out[b:b + 1]), ref)
            assert r["finite"] and r["max_abs"] <= TOL["bf16"] and r["max_abs"] <= bound


@pytest.mark.parametrize("dtype,bs", [("bf16", 16), ("f32", 32)])
def test_paged_append_bit_exact(dtype, bs):
    """Append through the table: bit-identical pools and lengths to the
    oracle; a full table and an invalid block id leave their sequence alone."""
    B, K, d = 4, 8, 128
    lens = [0, 15, 40, 47]
    inp = decode_inputs(B, 8, K, d, dtype, seed=51, lens=lens, s_max=48)
    p = paged_layout(inp, bs, seed=52, spare_blocks=1)
    bt = p["block_table"].clone()
    bt[2, 40 // bs] = -5                      # invalid id: sequence 2 untouched
    cap = p["block_table"].shape[1] * bs
    lens_in = torch.tensor([0, 15, 40, cap], dtype=torch.int32)  # sequence 3: table full
    it = _INT[p["k_pool"].dtype]
    k_ref, v_ref, s_ref = kv_append_paged_ref(
        inp["k_new"].view(it).numpy(), inp["v_new"].view(it).numpy(), p["k_pool"].view(it).numpy(),
        p["v_pool"].view(it).numpy(), bt.numpy(), lens_in.numpy())
    kp, vp = p["k_pool"].to(DEV), p["v_pool"].to(DEV)
    sl = lens_in.to(DEV)
    note(f"paged append {dtype} bs={bs}")
    gqa.gqa_kv_append_paged(inp["k_new"].to(DEV), inp["v_new"].to(DEV), kp, vp, bt.to(DEV), sl)
    torch.cuda.synchronize()
    assert sl.cpu().tolist() == list(s_ref) == [1, 16, 40, cap]
    assert np.array_equal(kp.cpu().view(it).numpy(), k_ref)
    assert np.array_equal(vp.cpu().view(it).numpy(), v_ref)


def test_paged_append_then_decode():
    """One paged decode step: append the new token, then attend over it."""
    B, H, K, d, bs = 3, 32, 8, 128, 16
    inp = decode_inputs(B, H, K, d, "bf16", seed=61, lens=[15, 16, 1999])
    p = paged_layout(inp, bs, seed=62, spare_blocks=3)
    kp, vp, bt, sl = (p[n].to(DEV) for n in ("k_pool", "v_pool", "block_table", "seq_lens"))
    gqa.gqa_kv_append_paged(inp["k_new"].to(DEV), inp["v_new"].to(DEV), kp, vp, bt, sl)
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(gqa.gqa_decode_paged_workspace_bytes(B, H, K, 2000, d, bs), dtype=torch.uint8, device=DEV)
    gqa.gqa_decode_paged(inp["q"].to(DEV), kp, vp, bt, sl, out, ws, 2000, scale=scale_of(d))
    torch.cuda.synchronize()
    it = torch.int16
    k2, v2, s2 = kv_append_paged_ref(inp["k_new"].view(it).numpy(), inp["v_new"].view(it).numpy(),
                                     p["k_pool"].view(it).numpy(), p["v_pool"].view(it).numpy(),
                                     p["block_table"].numpy(), p["seq_lens"].numpy())
    assert sl.cpu().tolist() == list(s2)
    k2 = torch.from_numpy(k2).view(torch.bfloat16)
    v2 = torch.from_numpy(v2).view(torch.bfloat16)
    ref = decode_paged_ref(f64(inp["q"]), _np(k2), _np(v2), p["block_table"].numpy(), s2, scale_of(d))
    r = report("append+decode", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= bf16_bound(ref, _vmax(v2))


def test_paged_full_workload():
    """The Llama-3-8B layer over 16-row blocks in shuffled order, in the
    launch configuration the benchmark times (the fused append + decode)."""
    w = WORKLOADS["decode_paged_llama3_8b"]
    note("paged full workload: inputs")
    inp = workload_inputs(w, seed=0)
    p = paged_layout(inp, w.extra["block_size"], seed=1)
    kp, vp, bt, sl = (p[n].to(DEV) for n in ("k_pool", "v_pool", "block_table", "seq_lens"))
    B, H, d = inp["q"].shape
    out = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(gqa.gqa_decode_paged_workspace_bytes(B, H, w.K, w.L + 1, d, p["block_size"]),
                     dtype=torch.uint8, device=DEV)
    note("paged full workload: GPU (append fused into the paged decode, as benchmarked)")
    gqa.gqa_decode_append_paged(inp["q"].to(DEV), inp["k_new"].to(DEV), inp["v_new"].to(DEV), kp, vp, bt, sl, out,
                                ws, w.L + 1, scale=scale_of(d))
    torch.cuda.synchronize()
    assert sl.cpu().tolist() == [w.L + 1] * B
    note("paged full workload: oracle")
    ref = np.zeros((B, H, d))
    bs = p["block_size"]
    for b in range(B):  # per sequence: the appended cache is the contiguous one plus the new row
        kc = inp["k_cache"][b:b + 1].clone()
        vc = inp["v_cache"][b:b + 1].clone()
        kc[0, :, w.L] = inp["k_new"][b]
        vc[0, :, w.L] = inp["v_new"][b]
        # the pool row the append wrote, read back through the table
        blk = int(p["block_table"][b, w.L // bs])
        assert torch.equal(kp[blk, :, w.L % bs].cpu(), inp["k_new"][b])
        assert torch.equal(vp[blk, :, w.L % bs].cpu(), inp["v_new"][b])
        sub = paged_layout({"k_cache": kc, "v_cache": vc}, bs, shuffle=False)
        ref[b] = decode_paged_ref(f64(inp["q"][b:b + 1]), _np(sub["k_pool"]), _np(sub["v_pool"]),
                                  sub["block_table"].numpy(), np.array([w.L + 1]), scale_of(d))[0]
    r = report("paged llama3_8b", f64(out), ref)
    assert r["finite"] and r["max_abs"] <= TOL["bf16"]
    assert r["max_abs"] <= bf16_bound(ref, _vmax(p["v_pool"]))


FUSED_CASES = [
    # B, H, K, d, lens, block_size, s_max, steps
    (3, 32, 8, 128, [1, 33, 1000], 16, None, 1),
    (4, 64, 8, 128, [0, 16, 17, 3000], 16, None, 1),
    (2, 16, 4, 64, [31, 2100], 32, None, 1),
    (2, 32, 1, 128, [129, 4100], 48, None, 1),       # G = 32: two head blocks
    (1, 71, 1, 64, [257], 16, None, 1),              # G = 71: five head blocks
    (2, 48, 1, 128, [777, 31], 32, None, 2),         # G = 48: three head blocks, two steps
    (1, 128, 2, 64, [1500], 16, None, 3),            # G = 64: four head blocks, three steps
    (40, 8, 8, 64, [8000 + 37 * i for i in range(40)], 16, None, 1),  # 62-block partitions, 320 units
    (2, 32, 8, 128, [60, 3], 16, 64, 8),             # eight steps; the first table fills up
]


def _fused_vs_unfused(inp, p, bt, lens_in, steps, seed):
    """Run `steps` decode steps through gqa_decode_append_paged and through
    gqa_kv_append_paged + gqa_decode_paged on copies of the same pools: the
    pools, lengths and output bits must agree every step, and the output
    must be within the bf16 bound of the oracle on the grown cache."""
    B, H, d = inp["q"].shape
    K, bs = p["k_pool"].shape[1], p["block_size"]
    cap = bt.shape[1] * bs
    msl = min(max(lens_in) + steps, cap)
    fused = [p["k_pool"].to(DEV), p["v_pool"].to(DEV), torch.tensor(lens_in, dtype=torch.int32, device=DEV)]
    split = [t.clone() for t in fused]
    ref = [p["k_pool"].view(torch.int16).numpy().copy(), p["v_pool"].view(torch.int16).numpy().copy(),
           np.array(lens_in, dtype=np.int32)]
    btd = bt.to(DEV)
    nbytes = gqa.gqa_decode_paged_workspace_bytes(B, H, K, msl, d, bs)
    ws_f = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ws_s = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    g = torch.Generator().manual_seed(seed)
    for step in range(steps):
        q = torch.randn((B, H, d), generator=g).to(torch.bfloat16)
        kn = torch.randn((B, K, d), generator=g).to(torch.bfloat16)
        vn = torch.randn((B, K, d), generator=g).to(torch.bfloat16)
        qd, knd, vnd = q.to(DEV), kn.to(DEV), vn.to(DEV)
        out_f = torch.empty((B, H, d), dtype=torch.bfloat16, device=DEV)
        out_s = torch.empty_like(out_f)
        gqa.gqa_decode_append_paged(qd, knd, vnd, fused[0], fused[1], btd, fused[2], out_f, ws_f, msl,
                                    scale=scale_of(d))
        gqa.gqa_kv_append_paged(knd, vnd, split[0], split[1], btd, split[2])
        gqa.gqa_decode_paged(qd, split[0], split[1], btd, split[2], out_s, ws_s, msl, scale=scale_of(d))
        torch.cuda.synchronize()
        ref = list(kv_append_paged_ref(kn.view(torch.int16).numpy(), vn.view(torch.int16).numpy(), ref[0], ref[1],
                                       bt.numpy(), ref[2]))
        assert fused[2].cpu().tolist() == split[2].cpu().tolist() == list(ref[2])
        for i in range(2):
            a = fused[i].cpu().view(torch.int16).numpy()
            assert np.array_equal(a, split[i].cpu().view(torch.int16).numpy()) and np.array_equal(a, ref[i])
        assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
        kf = torch.from_numpy(ref[0]).view(torch.bfloat16)
        vf = torch.from_numpy(ref[1]).view(torch.bfloat16)
        o_ref = decode_paged_ref(f64(q), _np(kf), _np(vf), bt.numpy(), ref[2], scale_of(d))
        r = report(f"paged fused step {step}", f64(out_f), o_ref)
        assert r["finite"] and r["max_abs"] <= bf16_bound(o_ref, _vmax(vf))


@pytest.mark.parametrize("B,H,K,d,lens,bs,s_max,steps", FUSED_CASES)
def test_paged_fused_append_matches_unfused(B, H, K, d, lens, bs, s_max, steps):
    note(f"paged fused append B={B} H={H} K={K} d={d} max_len={max(lens)} bs={bs} steps={steps}")
    inp = decode_inputs(B, H, K, d, "bf16", seed=71, lens=lens, s_max=s_max or max(lens) + steps)
    p = paged_layout(inp, bs, seed=72, spare_blocks=2)
    _fused_vs_unfused(inp, p, p["block_table"], lens, steps, seed=73)


@pytest.mark.parametrize("H,K", [(32, 8), (96, 2)])   # G = 4; G = 48 (the wide pass)
def test_paged_fused_append_full_table_and_invalid_id(H, K):
    """A full table and an invalid block id at the append position: that
    sequence is attended as it is and keeps its length, as in the
    standalone append."""
    B, d, bs = 4, 128, 16
    lens = [0, 15, 32, 48]
    inp = decode_inputs(B, H, K, d, "bf16", seed=74, lens=lens, s_max=48)
    p = paged_layout(inp, bs, seed=75, spare_blocks=1)
    assert p["block_table"].shape[1] * bs == 48  # sequence 3: table full
    bt = p["block_table"].clone()
    bt[2, 32 // bs] = -5                         # invalid id where sequence 2 would append
    note("paged fused append: full table + invalid id")
    _fused_vs_unfused(inp, p, bt, lens, 2, seed=76)
