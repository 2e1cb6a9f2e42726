"""GPU parity of gqa_kv_append (bit exact) and gqa_meanpool_convert."""
import numpy as np
import pytest
import torch

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd.inputs import decode_inputs, meanpool_inputs
from gpu_util import DEV, f64, guarded, guards_intact, note
from oracle import kv_append_ref, meanpool_convert_ref

pytestmark = pytest.mark.gpu

_INT = {torch.bfloat16: torch.int16, torch.float32: torch.int32}


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_append_bit_exact_with_guards(dtype, d):
    B, K, S_max = 5, 8, 40
    # lengths: empty, middle, last free row, full cache (no write, no increment), middle
    lens = [0, 17, S_max - 1, S_max, 3]
    inp = decode_inputs(B, 8, K, d, dtype, seed=21, lens=lens, s_max=S_max)
    tdt = inp["k_cache"].dtype
    kc, kbuf, g = guarded(tuple(inp["k_cache"].shape), tdt)
    vc, vbuf, _ = guarded(tuple(inp["v_cache"].shape), tdt)
    sl, sbuf, gs = guarded((B,), torch.int32)
    kc.copy_(inp["k_cache"].to(DEV))
    vc.copy_(inp["v_cache"].to(DEV))
    sl.copy_(inp["seq_lens"].to(DEV))
    note(f"append {dtype} d={d}")
    gqa.gqa_kv_append(inp["k_new"].to(DEV), inp["v_new"].to(DEV), kc, vc, sl)
    torch.cuda.synchronize()
    it = _INT[tdt]
    k_ref, v_ref, s_ref = kv_append_ref(inp["k_new"].view(it).numpy(), inp["v_new"].view(it).numpy(),
                                        inp["k_cache"].view(it).numpy(), inp["v_cache"].view(it).numpy(),
                                        inp["seq_lens"].numpy())
    assert np.array_equal(sl.cpu().numpy(), s_ref)
    assert np.array_equal(kc.cpu().view(it).numpy(), k_ref)
    assert np.array_equal(vc.cpu().view(it).numpy(), v_ref)
    assert guards_intact(kbuf, g, tdt) and guards_intact(vbuf, g, tdt) and guards_intact(sbuf, gs, torch.int32)


def test_append_twice_then_lengths():
    inp = decode_inputs(2, 8, 2, 128, "bf16", seed=3, lens=[4, 9], s_max=12)
    kc, vc, sl = inp["k_cache"].to(DEV), inp["v_cache"].to(DEV), inp["seq_lens"].to(DEV)
    kn, vn = inp["k_new"].to(DEV), inp["v_new"].to(DEV)
    gqa.gqa_kv_append(kn, vn, kc, vc, sl)
    gqa.gqa_kv_append(vn, kn, kc, vc, sl)
    torch.cuda.synchronize()
    assert sl.cpu().tolist() == [6, 11]
    assert torch.equal(kc[:, :, 4][0].cpu(), inp["k_new"][0]) and torch.equal(kc[0, :, 5].cpu(), inp["v_new"][0])
    assert torch.equal(vc[1, :, 10].cpu(), inp["k_new"][1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("outer,H,K,inner", [(3, 8, 2, 64), (2, 64, 8, 4096), (5, 7, 1, 12), (4, 6, 3, 5), (2, 16, 16, 32)])
def test_meanpool_vs_oracle(dtype, outer, H, K, inner):
    src = meanpool_inputs(outer, H, inner, dtype, seed=31)
    dst = torch.empty((outer, K, inner), dtype=src.dtype, device=DEV)
    note(f"meanpool {dtype} {outer}x{H}->{K}x{inner}")
    gqa.gqa_meanpool_convert(src.to(DEV), dst)
    torch.cuda.synchronize()
    ref = meanpool_convert_ref(f64(src), K)
    got = f64(dst)
    scale = float(np.abs(f64(src)).max())
    if dtype == "bf16":
        # one rounding of the fp32 mean to bf16 (relative u = 2^-8) plus the fp32 sum
        bound = np.abs(ref) * 2.0 ** -8 + 1e-6 * scale
    else:
        bound = np.full(ref.shape, 1e-6 * scale)
    assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_meanpool_identical_heads_exact(dtype):
    """A group of identical heads pools to that head exactly (bf16 bit exact:
    every fp32 partial sum r*x is exact and the quotient rounds back to x)."""
    outer, K, G, inner = 3, 8, 8, 256
    base = meanpool_inputs(outer, K, inner, dtype, seed=41)
    src = base.repeat_interleave(G, dim=1).contiguous()
    dst = torch.empty((outer, K, inner), dtype=src.dtype, device=DEV)
    gqa.gqa_meanpool_convert(src.to(DEV), dst)
    torch.cuda.synchronize()
    if dtype == "bf16":
        assert torch.equal(dst.cpu(), base)
    else:
        # fp32 partial sums may round: within one ulp of the shared head
        assert torch.allclose(dst.cpu(), base, rtol=2.0 ** -22, atol=0)


def test_meanpool_g1_identity():
    src = meanpool_inputs(4, 8, 128, "bf16", seed=2)
    dst = torch.empty_like(src, device=DEV)
    gqa.gqa_meanpool_convert(src.to(DEV), dst)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), src)


def _fp32_rule(src: torch.Tensor, K: int) -> torch.Tensor:
    """The conversion's stated rounding rule on the host: fp32 sum over the
    group's heads in head order, one IEEE fp32 division by G, then rounding
    to the element type."""
    x = src.float().numpy()
    outer, H, inner = x.shape
    G = H // K
    xs = x.reshape(outer, K, G, inner)
    s = np.zeros((outer, K, inner), dtype=np.float32)
    for r in range(G):
        s = s + xs[:, :, r]
    return torch.from_numpy(s / np.float32(G)).to(src.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("outer,H,K,inner", [(2, 64, 8, 4104), (1, 71, 1, 1024), (3, 24, 2, 8), (4, 6, 3, 5)])
def test_meanpool_rounding_rule_bit_exact(dtype, outer, H, K, inner):
    """Bit for bit the stated rule, on shapes covering more than one block of
    eight heads with a ragged tail (G = 71), tiny rows and the unvectorised
    path (inner not a multiple of the 16-byte word)."""
    src = meanpool_inputs(outer, H, inner, dtype, seed=32)
    dst = torch.empty((outer, K, inner), dtype=src.dtype, device=DEV)
    note(f"meanpool rule {dtype} {outer}x{H}->{K}x{inner}")
    gqa.gqa_meanpool_convert(src.to(DEV), dst)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), _fp32_rule(src, K))


def test_meanpool_full_workload():
    """The T5-XXL-shaped projection weight the benchmark converts: against
    the oracle (bound as above) and bit for bit against the stated rule."""
    from grouped_query_kv_amd.inputs import WORKLOADS
    w = WORKLOADS["meanpool_t5xxl"]
    inner = w.d * w.extra["d_model"]
    src = meanpool_inputs(1, w.H, inner, w.dtype, seed=0)
    dst = torch.empty((1, w.K, inner), dtype=src.dtype, device=DEV)
    note("meanpool full workload")
    gqa.gqa_meanpool_convert(src.to(DEV), dst)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), _fp32_rule(src, w.K))
    ref = meanpool_convert_ref(f64(src), w.K)
    got = f64(dst)
    bound = np.abs(ref) * 2.0 ** -8 + 1e-6 * float(np.abs(f64(src)).max())
    assert np.all(np.abs(got - ref) <= bound)
