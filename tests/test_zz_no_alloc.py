"""The allocation-free decode step gqa_decode_append_noalloc (partials in the
library's static device scratch) against gqa_decode_append with a caller
workspace: same kernels and plan, so outputs, caches and lengths must agree
bit for bit; both within the oracle tolerance.  Two calls in a row, the
second smaller than the first (the scratch keeps the first call's contents),
then an fp32 call."""
import numpy as np
import pytest
import torch

import grouped_query_kv_amd as gqa
from grouped_query_kv_amd.inputs import decode_inputs
from gpu_util import DEV, TOL, bf16_bound, f64, note, report, scale_of
from oracle import decode_ref, kv_append_ref

pytestmark = pytest.mark.gpu

_INT = {torch.bfloat16: torch.int16, torch.float32: torch.int32}


def _on_gpu(inp):
    return {k: inp[k].to(DEV) for k in ("q", "k_new", "v_new", "k_cache", "v_cache", "seq_lens")}


def _step_pair(B, H, K, d, lens, S_max, dtype, seed):
    note(f"no-alloc step B={B} H={H} K={K} d={d} lens={lens} S_max={S_max} {dtype} seed={seed}")
    inp = decode_inputs(B, H, K, d, dtype, seed=seed, lens=lens, s_max=S_max)
    msl = min(max(lens) + 1, S_max)
    scale = scale_of(d)
    a, b = _on_gpu(inp), _on_gpu(inp)
    out_a = torch.empty((B, H, d), dtype=a["q"].dtype, device=DEV)
    out_b = torch.full((B, H, d), float("nan"), dtype=b["q"].dtype, device=DEV)
    ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, H, K, msl, d), dtype=torch.uint8, device=DEV)
    gqa.gqa_decode_append(a["q"], a["k_new"], a["v_new"], a["k_cache"], a["v_cache"], a["seq_lens"], out_a,
                          ws, msl, scale=scale)
    gqa.gqa_decode_append_noalloc(b["q"], b["k_new"], b["v_new"], b["k_cache"], b["v_cache"], b["seq_lens"],
                                  out_b, msl, scale=scale)
    torch.cuda.synchronize()
    # same kernels, same plan: bit-identical results, caches and lengths
    assert torch.equal(out_a, out_b)
    assert torch.equal(a["seq_lens"], b["seq_lens"])
    it = _INT[a["k_cache"].dtype]
    assert torch.equal(a["k_cache"].view(it), b["k_cache"].view(it))
    assert torch.equal(a["v_cache"].view(it), b["v_cache"].view(it))
    # and both equal the oracle's append, and its decode within tolerance
    k_ref, v_ref, s_ref = kv_append_ref(inp["k_new"].view(it).numpy(), inp["v_new"].view(it).numpy(),
                                        inp["k_cache"].view(it).numpy(), inp["v_cache"].view(it).numpy(),
                                        inp["seq_lens"].numpy())
    assert np.array_equal(b["seq_lens"].cpu().numpy(), s_ref)
    assert np.array_equal(b["k_cache"].cpu().view(it).numpy(), k_ref)
    kc, vc = b["k_cache"].cpu().float().numpy(), b["v_cache"].cpu().float().numpy()
    ref = decode_ref(f64(inp["q"]), kc, vc, s_ref, scale)
    r = report("no-alloc", f64(out_b), ref)
    assert r["finite"] and r["max_abs"] <= TOL[dtype]
    if dtype == "bf16":
        vmax = float(np.abs(np.nan_to_num(vc)).max())
        assert r["max_abs"] <= bf16_bound(ref, vmax)


def test_noalloc_matches_workspace_entry_point_twice_then_smaller():
    # first call: a ragged batch with many partitions, including an empty
    # sequence and a full cache (no append for it)
    _step_pair(4, 32, 8, 128, [2000, 0, 4095, 4096], 4096, "bf16", seed=31)
    # second call, smaller: fewer sequences, heads and positions; the scratch
    # still holds the first call's partials
    _step_pair(2, 8, 2, 64, [17, 5], 64, "bf16", seed=32)
    # fp32 caches, multi-query group
    _step_pair(2, 20, 1, 64, [300, 41], 320, "f32", seed=33)

