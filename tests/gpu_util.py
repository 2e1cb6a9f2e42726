"""Helpers for the GPU parity tests (the HIP path vs the CPU oracle)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import grouped_query_kv_amd as gqa

DEV = torch.device("cuda:0")

# Tolerances on the max-abs error against the fp64 oracle (the pass/fail
# gates of the method's statement): fp32 inputs 1e-5, bf16 inputs 2e-2.
TOL = {"f32": 1e-5, "bf16": 2e-2}


def note(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a CPU/GPU float tensor (bf16 and fp32 embed exactly)."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def guarded(shape, dtype, guard_elems=64, fill=None):
    """A contiguous tensor of `shape` inside a larger buffer with sentinel
    guard bands; returns (view, buffer, guard)."""
    n = int(np.prod(shape))
    buf = torch.empty(n + 2 * guard_elems, dtype=dtype, device=DEV)
    if dtype == torch.int32:
        buf.fill_(-777)
    else:
        buf.fill_(float("nan") if fill is None else fill)
    view = buf[guard_elems:guard_elems + n].view(*shape)
    return view, buf, guard_elems


def guards_intact(buf: torch.Tensor, guard: int, dtype) -> bool:
    head = buf[:guard].to("cpu")
    tail = buf[-guard:].to("cpu")
    if dtype == torch.int32:
        return bool((head == -777).all() and (tail == -777).all())
    return bool(torch.isnan(head).all() and torch.isnan(tail).all())


BF16_U = 2.0 ** -8  # unit roundoff of bf16 (8-bit significand, round to nearest even)


def bf16_bound(ref: np.ndarray, v_absmax: float, weights_in_denominator: bool = False) -> float:
    """Arithmetic error bound of a bf16 attention output.  Each softmax weight
    is rounded to bf16 once (relative error <= u = 2^-8) before multiplying V,
    which moves the weighted sum by at most u * max|v|; the output is rounded
    once more (u |out|).  When the denominator also sums the rounded weights
    (prefill) the quotient can move by up to twice the weight error.  fp32
    accumulation error is orders smaller."""
    w = 2 * BF16_U if weights_in_denominator else BF16_U
    return w * v_absmax + BF16_U * float(np.abs(ref).max()) + 1e-6


def report(name: str, got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    r = {"max_abs": float(err.max()) if err.size else 0.0,
         "rms_ref": rms,
         "max_abs_over_rms": float(err.max() / rms) if rms > 0 else 0.0,
         "finite": bool(np.all(np.isfinite(got)))}
    note(f"  [{name}] max_abs={r['max_abs']:.3e} rms(ref)={rms:.3e} "
         f"max_abs/rms={r['max_abs_over_rms']:.3e}")
    return r


def run_decode(inp: dict, out_dtype=None, max_seq_len=None, append=False):
    """Copy a decode batch to the GPU, optionally append, run gqa_decode.
    Returns (out_gpu_tensor, device_tensors)."""
    q = inp["q"].to(DEV)
    kc = inp["k_cache"].to(DEV)
    vc = inp["v_cache"].to(DEV)
    sl = inp["seq_lens"].to(DEV)
    dev = {"q": q, "k_cache": kc, "v_cache": vc, "seq_lens": sl}
    if append:
        kn = inp["k_new"].to(DEV)
        vn = inp["v_new"].to(DEV)
        gqa.gqa_kv_append(kn, vn, kc, vc, sl)
    B, H, d = q.shape
    K = kc.shape[1]
    msl = int(inp["seq_lens"].max().item()) + (1 if append else 0) if max_seq_len is None else max_seq_len
    msl = min(msl, kc.shape[2])
    ws = torch.empty(max(gqa.gqa_decode_workspace_bytes(B, H, K, msl, d), 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, H, d), dtype=out_dtype or q.dtype, device=DEV)
    gqa.gqa_decode(q, kc, vc, sl, out, ws, msl, scale=scale_of(d))
    torch.cuda.synchronize()
    return out, dev


def scale_of(d: int) -> float:
    """fp32 value of 1/sqrt(d), passed identically to the GPU and the oracle."""
    return float(np.float32(1.0 / math.sqrt(d)))


def oracle_by_kv_head(fn, q, k, v, *args, workers: int | None = None) -> np.ndarray:
    """Evaluate an oracle attention function ``fn(q, k, v, *args)`` (q [B, H,
    S_q, d], k/v [B, K, S_kv, d], any extra per-sequence arrays in ``args``
    indexed by b) one (sequence, KV head) slice at a time, the slices spread
    over host threads (NumPy releases the GIL inside its kernels; BLAS runs
    single-threaded per slice).  The slices are independent, so the result
    is exactly what one call over the whole batch returns."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    B, H, Sq, d = q.shape
    K = k.shape[1]
    G = H // K
    out = np.zeros((B, H, Sq, d))
    if workers is None:
        try:
            workers = len(os.sched_getaffinity(0))
        except AttributeError:
            workers = os.cpu_count() or 1
        workers = max(1, min(16, workers))

    def one(bk):
        b, kh = bk
        sl = [a[b:b + 1] for a in args]
        out[b:b + 1, kh * G:(kh + 1) * G] = fn(q[b:b + 1, kh * G:(kh + 1) * G], k[b:b + 1, kh:kh + 1],
                                              v[b:b + 1, kh:kh + 1], *sl)

    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(one, [(b, kh) for b in range(B) for kh in range(K)]))
    return out
