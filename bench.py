"""Benchmark of the GQA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

With --workload prefill_causal_4k it times the causal prefill instead (one
step = one prefill of the whole batch; value in TFLOP/s of unmasked work);
prefill_chunk_8k times a chunked-prefill step (append a 2048-row chunk, then
its queries attend over the 8192-row cache) and cross_attention_4k a
non-causal cross-attention step.

A step is one pass of the whole decode hot path over one batch: append the
new token's K/V rows of every sequence and attend over the cache including
them (gqa_decode_append: the append fused into the partition pass, then the
combine pass -- the same work as gqa_kv_append followed by gqa_decode).  A
paged workload (decode_paged_llama3_8b) runs gqa_decode_append_paged (the
append through the block table fused into the paged decode) over 16-row
blocks in shuffled physical order; an int8
workload (decode_int8_llama3_8b) runs gqa_decode_append_int8 (the
quantising append fused into the int8 partition pass) over the cache
quantised once before timing (bytes counted as stored: d codes + one fp32
scale per row).  decode_mqa_71h is a multi-query layer (71 query heads on
one KV head, d=64, 32768 cached tokens), whose groups of more than 16 heads
take the one-workgroup-per-group partition pass.  The default workload is
the Llama-3-8B-shaped layer: B=16 sequences at 8192 cached tokens, 32 query
heads over 8 KV heads, d=128, bf16 (synthetic N(0,1) data).

The caches are kept in several copies that the steps rotate through, so no
step finds the previous step's cache lines in the 256 MB Infinity Cache; each
step appends one more token, so the context grows by one per visit of a copy
and the algorithmic bytes are counted from the actual lengths.

Prints one JSON line.  `value` is the KV-cache read rate of the whole step
(algorithmic KV bytes / step time); tokens/s (B tokens per step) and the
fraction of the 8 TB/s HBM peak are reported beside it.  `roofline` covers
the dominant kernel (the decode partition pass), timed live with HIP events
recorded on its stream around each launch.  `cpu_baseline` is the fp64 CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 matrix-core peak
F32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix-core peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_llama3_8b")
    ap.add_argument("--copies", type=int, default=4, help="cache copies rotated over the steps")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-baseline time budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations timed beside the headline decode workload")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="timed steps per additional configuration (warm-up: min(--warmup, 5))")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))


def sources_code_sha256(paths) -> str:
    """SHA-256 of the code in the given source files (repository-relative),
    with C/C++ comments removed and whitespace runs collapsed (the library's
    build-id hash), so that an edit of comments alone leaves it unchanged."""
    from grouped_query_kv_amd.build import code_sha256

    return code_sha256(paths)


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch recorded from rocprofv3 counters for `kernel` on
    `workload` (profiles/traffic.json), or None when nothing was recorded for
    that pair or the code of the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)["workloads"][workload]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("kernel") != kernel:
        return None
    if sources_code_sha256(rec["sources"]) != rec["sources_code_sha256"]:
        return None
    return int(rec["read_bytes"] + rec["write_bytes"])


def kv_bytes(lens, K, d, elem, row_extra=0):
    """K and V bytes of the cached rows: 2 * K * L_b rows of d elements
    (plus `row_extra` bytes per row, the fp32 scale of an int8 row)."""
    return int(sum(2 * K * int(L) * (d * elem + row_extra) for L in lens))


def host_cores():
    """The host cores this process may use (at most 16: the share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline_decode(inp, w, budget_s):
    """Time the fp64 oracle (unchanged) on whole sequences of the workload,
    on the host's cores (BLAS threads), until about `budget_s` seconds have
    been spent."""
    from threadpoolctl import threadpool_limits

    from grouped_query_kv_amd.inputs import paged_layout
    from oracle import (decode_int8_ref, decode_paged_ref, decode_ref, kv_append_int8_ref,
                        kv_append_paged_ref, kv_append_ref, quantize_int8_ref)

    paged = "block_size" in w.extra
    int8 = w.extra.get("kv_dtype") == "int8"
    elem, row_extra = (1, 4) if int8 else ((4, 0) if w.dtype == "f32" else (2, 0))
    d = w.d
    scale = float(np.float32(1.0 / math.sqrt(d)))
    done_bytes, done_seqs, t_used = 0, 0, 0.0
    cores = host_cores()
    with threadpool_limits(limits=cores):
        b = 0
        while t_used < budget_s:
            sl = inp["seq_lens"][b:b + 1].numpy()
            q = inp["q"][b:b + 1].double().numpy()
            kc = inp["k_cache"][b:b + 1].float().numpy()
            vc = inp["v_cache"][b:b + 1].float().numpy()
            kn = inp["k_new"][b:b + 1].float().numpy()
            vn = inp["v_new"][b:b + 1].float().numpy()
            if int8:
                L = int(sl[0])
                kq, ksq = quantize_int8_ref(inp["k_cache"][b:b + 1, :, :L].float().numpy())
                vq, vsq = quantize_int8_ref(inp["v_cache"][b:b + 1, :, :L].float().numpy())
                pad = lambda a: np.concatenate([a, np.zeros(a.shape[:2] + (1,) + a.shape[3:], a.dtype)], axis=2)
                kq, vq, ksq, vsq = pad(kq), pad(vq), pad(ksq), pad(vsq)
                t0 = time.perf_counter()
                kq, vq, ksq, vsq, sl = kv_append_int8_ref(kn, vn, kq, vq, ksq, vsq, sl)
                decode_int8_ref(q, kq, vq, ksq, vsq, sl, scale)
                t_used += time.perf_counter() - t0
            elif paged:
                pg = paged_layout({"k_cache": inp["k_cache"][b:b + 1], "v_cache": inp["v_cache"][b:b + 1]},
                                  w.extra["block_size"], seed=b)
                kp, vp = pg["k_pool"].float().numpy(), pg["v_pool"].float().numpy()
                bt = pg["block_table"].numpy()
                t0 = time.perf_counter()
                if w.append:
                    kp, vp, sl = kv_append_paged_ref(kn, vn, kp, vp, bt, sl)
                decode_paged_ref(q, kp, vp, bt, sl, scale)
                t_used += time.perf_counter() - t0
            else:
                t0 = time.perf_counter()
                if w.append:
                    kc, vc, sl = kv_append_ref(kn, vn, kc, vc, sl)
                decode_ref(q, kc, vc, sl, scale)
                t_used += time.perf_counter() - t0
            done_bytes += kv_bytes(sl, w.K, d, elem, row_extra)
            done_seqs += 1
            b = (b + 1) % w.B
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "tokens_per_s": done_seqs / t_used,
            "sample": f"{done_seqs} whole sequences of the workload ({'paged ' if paged else 'int8 ' if int8 else ''}append + decode over "
                      f"{int(inp['seq_lens'][0]) + (1 if w.append else 0)} positions, all {w.H} heads), "
                      f"{t_used:.1f} s of fp64 NumPy on {cores} BLAS threads"}


def bench_decode(args, w, sub=False):
    import grouped_query_kv_amd as gqa
    from grouped_query_kv_amd.inputs import paged_layout, workload_inputs

    dev = torch.device("cuda:0")
    R = max(1, args.copies)
    visits = math.ceil((args.warmup + args.steps) / R)
    base_len = int(w.L) if w.ragged is None else w.ragged[1]
    s_max = (base_len + visits + 2 + 3) // 4 * 4
    t_gen = time.perf_counter()
    inp = workload_inputs(w, seed=args.seed, s_max=s_max)
    t_gen = time.perf_counter() - t_gen
    B, H, K, d = w.B, w.H, w.K, w.d
    q = inp["q"].to(dev)
    kn, vn = inp["k_new"].to(dev), inp["v_new"].to(dev)
    paged = "block_size" in w.extra
    int8 = w.extra.get("kv_dtype") == "int8"
    # groups of more than 16 query heads take the one-workgroup-per-group bf16 pass
    wide = w.dtype == "bf16" and not int8 and (H // K + 15) // 16 > 1
    elem, row_extra = (1, 4) if int8 else ((4, 0) if w.dtype == "f32" else (2, 0))
    copies = []
    if int8:
        # the workload's bf16 caches quantised once on the GPU (set-up, untimed)
        kb, vb = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
        kc0 = torch.empty(kb.shape, dtype=torch.int8, device=dev)
        vc0 = torch.empty(vb.shape, dtype=torch.int8, device=dev)
        ks0 = torch.empty(kb.shape[:3], dtype=torch.float32, device=dev)
        vs0 = torch.empty(vb.shape[:3], dtype=torch.float32, device=dev)
        gqa.gqa_kv_quantize_int8(kb, kc0, ks0)
        gqa.gqa_kv_quantize_int8(vb, vc0, vs0)
        del kb, vb
    elif paged:
        pg = paged_layout(inp, w.extra["block_size"], seed=args.seed + 1)
        kc0, vc0 = pg["k_pool"].to(dev), pg["v_pool"].to(dev)
        bt = pg["block_table"].to(dev)
    else:
        kc0, vc0 = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
    for r in range(R):
        copies.append({"k": kc0 if r == 0 else kc0.clone(), "v": vc0 if r == 0 else vc0.clone(),
                       "sl": inp["seq_lens"].to(dev).clone()})
        if int8:
            copies[-1]["ks"] = ks0 if r == 0 else ks0.clone()
            copies[-1]["vs"] = vs0 if r == 0 else vs0.clone()
    host_lens = [inp["seq_lens"].clone() for _ in range(R)]
    max_len = int(inp["seq_lens"].max()) + visits + 1
    if paged:
        bs = w.extra["block_size"]
        ws = torch.empty(gqa.gqa_decode_paged_workspace_bytes(B, H, K, max_len, d, bs),
                         dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(gqa.gqa_decode_workspace_bytes(B, H, K, max_len, d), dtype=torch.uint8, device=dev)
    # fp32 caches produce fp32 outputs (the library's fp32 path), bf16 ones bf16
    out = torch.empty((B, H, d), dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        c = copies[i % R]
        if ev is not None:
            gqa.gqa_set_timing_events(ev[0], ev[1])
        if int8:
            # quantising append fused into the int8 partition pass (two launches)
            gqa.gqa_decode_append_int8(q, kn, vn, c["k"], c["v"], c["ks"], c["vs"], c["sl"], out, ws,
                                       max_len, scale=scale, stream=stream)
            host_lens[i % R] += 1
        elif paged:
            if w.append:
                # append through the block table fused into the paged decode (two launches)
                gqa.gqa_decode_append_paged(q, kn, vn, c["k"], c["v"], bt, c["sl"], out, ws, max_len,
                                            scale=scale, stream=stream)
                host_lens[i % R] += 1
            else:
                gqa.gqa_decode_paged(q, c["k"], c["v"], bt, c["sl"], out, ws, max_len, scale=scale,
                                     stream=stream)
        elif w.append:
            # append + decode as one fused call (two kernel launches)
            gqa.gqa_decode_append(q, kn, vn, c["k"], c["v"], c["sl"], out, ws, max_len,
                                  scale=scale, stream=stream)
            host_lens[i % R] += 1
        else:
            gqa.gqa_decode(q, c["k"], c["v"], c["sl"], out, ws, max_len, scale=scale, stream=stream)
        if ev is not None:
            gqa.gqa_set_timing_events(None, None)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # algorithmic KV bytes of each timed step (lengths after that step's append)
    step_bytes = []
    sim = [h.clone() for h in host_lens]
    for i in range(args.warmup, args.warmup + args.steps):
        if w.append:
            sim[i % R] += 1
        step_bytes.append(kv_bytes(sim[i % R].tolist(), K, d, elem, row_extra))
    # the partition pass is bracketed by timing events in every EVERY-th timed
    # step (recording events costs a couple of microseconds of gap per step)
    EVERY = 4
    sampled = list(range(0, args.steps, EVERY))
    events = {j: (gqa.HipEvent(), gqa.HipEvent()) for j in sampled}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j, i in enumerate(range(args.warmup, args.warmup + args.steps)):
        step(i, events.get(j))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = [events[j][0].elapsed_ms(events[j][1]) for j in sampled]
    total_bytes = sum(step_bytes)
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = total_bytes / elapsed / 1e9
    kern_avg_ms = float(np.mean(kern_ms))
    achieved = float(np.mean([step_bytes[j] for j in sampled])) / (kern_avg_ms * 1e-3) / 1e9
    p10, p50, p90 = (float(x) for x in np.percentile(kern_ms, [10, 50, 90]))
    # warm figure: the same cache copy every step (it partly stays in the
    # 256 MB Infinity Cache); never the headline
    warm_ms = None
    if not (paged or int8 or sub):
        wev = (gqa.HipEvent(), gqa.HipEvent())
        c0 = copies[0]
        for _ in range(6):
            gqa.gqa_decode(q, c0["k"], c0["v"], c0["sl"], out, ws, max_len, scale=scale, stream=stream)
        wts = []
        for _ in range(10):
            gqa.gqa_set_timing_events(*wev)
            gqa.gqa_decode(q, c0["k"], c0["v"], c0["sl"], out, ws, max_len, scale=scale, stream=stream)
            gqa.gqa_set_timing_events(None, None)
            wts.append(wev[0].elapsed_ms(wev[1]))
        warm_ms = float(np.median(wts))
    copy_gbs = None if sub else copy_ceiling(dev)
    res = {
        "metric": "GQA decode KV-read GB/s (% of HBM peak) + attention tokens/s, 1\u00d7MI355X",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "K": K, "d": d,
                   "context": (int(w.L) if w.ragged is None else list(w.ragged)),
                   "append_per_step": bool(w.append), "cache_copies": R,
                   **({"block_size": w.extra["block_size"], "block_order": "shuffled"} if paged else {}),
                   **({"kv_dtype": "int8", "kv_row_bytes": d + 4} if int8 else {}),
                   "seed": args.seed, "parallelism": "single GPU"},
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": int(total_bytes / args.steps),
        "roofline": {"kernel": ("int8 decode partition pass" + (" with fused append" if w.append else "") +
                                " (decode_split_int8_kernel)" if int8 else
                                "paged decode partition pass" + (" with fused append" if w.append else "") +
                                " (decode_split_bf16_kernel, paged)" if paged else
                                "fp32 decode partition pass (decode_split_f32_kernel)" if w.dtype == "f32" else
                                "decode partition pass" + (" with fused append" if w.append else "") +
                                (" (decode_wide_bf16_kernel)" if wide else " (decode_split_bf16_kernel)")),
                     "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic("decode_split_int8_kernel" if int8 else
                                                 "decode_split_f32_kernel" if w.dtype == "f32" else
                                                 "decode_wide_bf16_kernel" if wide else
                                                 "decode_split_bf16_kernel" + ("_paged" if paged else ""), w.name),
                     "avg_kernel_us": round(kern_avg_ms * 1e3, 3), "timed_launches": len(sampled),
                     "kernel_us_p10_p50_p90": [round(p10 * 1e3, 2), round(p50 * 1e3, 2), round(p90 * 1e3, 2)],
                     **({"copy_ceiling_GBps": round(copy_gbs, 1)} if copy_gbs is not None else {}),
                     **({"warm_kernel_us": round(warm_ms * 1e3, 2)} if warm_ms is not None else {})},
        "input_gen_s": round(t_gen, 1),
    }
    return res, inp


def copy_ceiling(dev, nbytes=1 << 30):
    """Device-to-device copy rate of a 1 GiB buffer (read + write bytes / time):
    a measured ceiling for streaming kernels, beside the 8 TB/s spec."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def visible_pairs(w):
    """(query, key) pairs that carry weight, per (sequence, head)."""
    if w.kind == "prefill":
        return w.L * (w.L + 1) // 2
    if w.kind == "chunk":
        T = w.extra["chunk"]
        return T * (w.L - T) + T * (T + 1) // 2
    return w.extra["S_q"] * w.L                       # cross-attention: no mask


def cpu_baseline_prefill(inp, w, budget_s):
    """Time the fp64 oracle (unchanged) on whole (sequence, head) slices of
    the workload, on the host's cores, until about `budget_s` seconds."""
    from threadpoolctl import threadpool_limits

    from oracle import cross_attention_ref, prefill_causal_ref, prefill_chunk_ref

    scale = float(np.float32(1.0 / math.sqrt(w.d)))
    G = w.H // w.K
    done, t_used, heads = 0.0, 0.0, 0
    cores = host_cores()
    with threadpool_limits(limits=cores):
        while t_used < budget_s and heads < w.B * w.H:
            b, h = divmod(heads, w.H)
            q = inp["q"][b:b + 1, h:h + 1].double().numpy()
            kv = slice(h // G, h // G + 1)
            if w.kind == "chunk":   # the cache after the chunk's append
                T = w.extra["chunk"]
                L0 = w.L - T
                k = torch.cat([inp["k"][b:b + 1, kv, :L0], inp["k_new"][b:b + 1, kv]], dim=2).float().numpy()
                v = torch.cat([inp["v"][b:b + 1, kv, :L0], inp["v_new"][b:b + 1, kv]], dim=2).float().numpy()
            else:
                k = inp["k"][b:b + 1, kv].float().numpy()
                v = inp["v"][b:b + 1, kv].float().numpy()
            t0 = time.perf_counter()
            if w.kind == "prefill":
                prefill_causal_ref(q, k, v, scale)
            elif w.kind == "chunk":
                prefill_chunk_ref(q, k, v, np.array([w.L]), scale)
            else:
                cross_attention_ref(q, k, v, np.array([w.L]), scale)
            t_used += time.perf_counter() - t0
            done += 4.0 * w.d * visible_pairs(w)
            heads += 1
    return {"value": done / t_used / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} whole (sequence, head) slices of the workload, "
                      f"{t_used:.1f} s of fp64 NumPy on {cores} BLAS threads"}


PREFILL_METRIC = {
    "prefill": "GQA causal prefill TFLOP/s (fraction of bf16 MFMA peak), 1\u00d7MI355X",
    "chunk": "GQA chunked prefill over a KV cache TFLOP/s (fraction of bf16 MFMA peak), 1\u00d7MI355X",
    "cross": "GQA cross-attention TFLOP/s (fraction of bf16 MFMA peak), 1\u00d7MI355X",
}


def bench_prefill(args, w):
    """Prefill-family step: causal prefill; chunked prefill (append the
    chunk's rows, then its queries attend over the cache); cross-attention."""
    import grouped_query_kv_amd as gqa
    from grouped_query_kv_amd.inputs import workload_inputs

    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    inp = workload_inputs(w, seed=args.seed)
    t_gen = time.perf_counter() - t_gen
    q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
    out = torch.empty_like(q)
    scale = float(np.float32(1.0 / math.sqrt(w.d)))
    stream = torch.cuda.current_stream()
    if w.kind != "prefill":
        lens0 = inp["kv_lens"].to(dev)
        lens = lens0.clone()
    if w.kind == "chunk":
        kn, vn = inp["k_new"].to(dev), inp["v_new"].to(dev)

    def step(ev=None):
        if w.kind == "chunk":
            lens.copy_(lens0)          # every step appends the same chunk to the same cache
            gqa.gqa_kv_append_rows(kn, vn, k, v, lens, stream=stream)
        if ev is not None:
            gqa.gqa_set_timing_events(*ev)
        if w.kind == "prefill":
            gqa.gqa_prefill_causal(q, k, v, out, scale=scale, stream=stream)
        elif w.kind == "chunk":
            gqa.gqa_prefill_chunk(q, k, v, lens, out, scale=scale, stream=stream)
        else:
            gqa.gqa_cross_attention(q, k, v, lens, out, scale=scale, stream=stream)
        if ev is not None:
            gqa.gqa_set_timing_events(None, None)

    for _ in range(args.warmup):
        step()
    events = [(gqa.HipEvent(), gqa.HipEvent()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in events:
        step(ev)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_ms = float(np.mean([a.elapsed_ms(b) for a, b in events]))
    flops = 4.0 * w.B * w.H * w.d * visible_pairs(w)   # two products, visible pairs only
    ms_per_step = elapsed * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    S_q = {"prefill": w.L, "chunk": w.extra.get("chunk"), "cross": w.extra.get("S_q")}[w.kind]
    cfg = {"workload": w.name, "B": w.B, "H": w.H, "K": w.K, "d": w.d, "S_q": S_q, "kv_len": w.L,
           "seed": args.seed, "parallelism": "single GPU"}
    # a contraction takes the matrix-core peak of its own type
    f32 = w.dtype == "f32"
    peak = F32_MFMA_PEAK_TFLOPS if f32 else BF16_MFMA_PEAK_TFLOPS
    res = {
        "metric": PREFILL_METRIC[w.kind].replace("bf16 MFMA", "fp32 MFMA") if f32 else PREFILL_METRIC[w.kind],
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": cfg,
        "tokens_per_s": round(w.B * S_q / (ms_per_step * 1e-3), 1),
        "roofline": {"kernel": f"{w.kind} attention ({'prefill_f32_kernel' if f32 else 'prefill_kernel'})",
                     "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": (recorded_traffic("prefill_causal_kernel", w.name)
                                 if w.kind == "prefill" and not f32 else None),
                     "avg_kernel_us": round(kern_ms * 1e3, 3)},
        "input_gen_s": round(t_gen, 1),
    }
    return res, inp


def bench_project(args, w):
    """Fused K/V projection + append of one decode token per sequence: HBM
    bound on reading W_KV once per step."""
    import grouped_query_kv_amd as gqa
    from grouped_query_kv_amd.inputs import projection_inputs

    dev = torch.device("cuda:0")
    dm, T = w.extra["d_model"], w.extra["T"]
    t_gen = time.perf_counter()
    inp = projection_inputs(w.B, T, dm, w.K, w.d, seed=args.seed)
    t_gen = time.perf_counter() - t_gen
    x = inp["x"].to(dev)
    # one W_KV per layer of a 32-layer model (537 MB in all, beyond the 256 MB
    # Infinity Cache), visited in turn, so every step reads its W_KV from HBM
    layers = 32
    wkvs = [inp["w_kv"].to(dev) for _ in range(layers)]
    S_max = w.L + T
    kc = torch.zeros((w.B, w.K, S_max, w.d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    lens0 = torch.full((w.B,), w.L, dtype=torch.int32, device=dev)
    lens = lens0.clone()
    ws = torch.empty(gqa.gqa_kv_project_workspace_bytes(w.B, T, dm, w.K, w.d), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        lens.copy_(lens0)              # every step writes the same position
        if ev is not None:
            gqa.gqa_set_timing_events(*ev)
        gqa.gqa_kv_project_append(x, wkvs[i % layers], kc, vc, lens, ws, stream=stream)
        if ev is not None:
            gqa.gqa_set_timing_events(None, None)

    for i in range(args.warmup):
        step(i)
    events = [(gqa.HipEvent(), gqa.HipEvent()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, ev in enumerate(events):
        step(args.warmup + i, ev)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_ms = float(np.mean([a.elapsed_ms(b) for a, b in events]))
    byts = wkvs[0].numel() * 2 + x.numel() * 2 + 2 * w.B * T * w.K * w.d * 2   # W_KV + x read, K/V rows written
    ms_per_step = elapsed * 1e3 / args.steps
    res = {
        "metric": "GQA fused K/V projection + append GB/s (W_KV streamed once per step), 1\u00d7MI355X",
        "value": round(byts / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": T, "d_model": dm, "K": w.K, "d": w.d,
                   "w_kv_copies": layers, "seed": args.seed, "parallelism": "single GPU"},
        "tokens_per_s": round(w.B * T / (ms_per_step * 1e-3), 1),
        "roofline": {"kernel": "K/V projection (kv_project_kernel)",
                     "bound": "hbm",
                     "achieved": round(byts / (kern_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(byts / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_kernel_us": round(kern_ms * 1e3, 3)},
        "input_gen_s": round(t_gen, 1),
    }
    return res, inp


def cpu_baseline_project(inp, w, budget_s):
    """The oracle's projection of whole steps (all tokens, all heads), on the
    host's cores, repeated for about `budget_s` seconds."""
    from threadpoolctl import threadpool_limits

    from oracle import kv_project_ref

    x = inp["x"].float().numpy()
    wk = inp["w_kv"].float().numpy()
    byts = wk.size * 2 + x.size * 2 + 2 * x.shape[0] * x.shape[1] * wk.shape[0] * (wk.shape[1] // 2) * 2
    steps, t_used = 0, 0.0
    cores = host_cores()
    with threadpool_limits(limits=cores):
        while t_used < budget_s:
            t0 = time.perf_counter()
            kv_project_ref(x, wk)
            t_used += time.perf_counter() - t0
            steps += 1
    return {"value": steps * byts / t_used / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{steps} whole projection steps, {t_used:.1f} s of fp64 NumPy on {cores} BLAS threads"}


def bench_meanpool(args, w):
    """Mean-pool conversion of one projection weight per step ([outer, H,
    inner] -> [outer, K, inner]); the weights of a 24-layer checkpoint's K and
    V projections (48 matrices, 1.6 GB) are visited in turn, so every step
    reads its source from HBM."""
    import grouped_query_kv_amd as gqa
    from grouped_query_kv_amd.inputs import meanpool_inputs

    dev = torch.device("cuda:0")
    inner = w.d * w.extra["d_model"]
    t_gen = time.perf_counter()
    src0 = meanpool_inputs(1, w.H, inner, w.dtype, seed=args.seed)
    t_gen = time.perf_counter() - t_gen
    n = w.extra["matrices"]
    srcs = [src0.to(dev)]
    srcs += [srcs[0].clone() for _ in range(n - 1)]
    dsts = [torch.empty((1, w.K, inner), dtype=src0.dtype, device=dev) for _ in range(n)]
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if ev is not None:
            gqa.gqa_set_timing_events(*ev)
        gqa.gqa_meanpool_convert(srcs[i % n], dsts[i % n], stream=stream)
        if ev is not None:
            gqa.gqa_set_timing_events(None, None)

    for i in range(args.warmup):
        step(i)
    events = [(gqa.HipEvent(), gqa.HipEvent()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, ev in enumerate(events):
        step(args.warmup + i, ev)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern = [a.elapsed_ms(b) for a, b in events]
    kern_ms = float(np.mean(kern))
    eb = src0.element_size()
    byts = (w.H + w.K) * inner * eb          # every source element read once, every output written once
    ms_per_step = elapsed * 1e3 / args.steps
    res = {
        "metric": "GQA mean-pool conversion GB/s (bytes read + written), 1\u00d7MI355X",
        "value": round(byts / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "outer": 1, "H": w.H, "K": w.K, "inner": inner, "matrices": n,
                   "seed": args.seed, "parallelism": "single GPU"},
        "roofline": {"kernel": "mean-pool conversion (meanpool_vec_kernel)", "bound": "hbm",
                     "achieved": round(byts / (kern_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(byts / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_kernel_us": round(kern_ms * 1e3, 3),
                     "kernel_us_p10_p50_p90": [round(float(x) * 1e3, 2) for x in np.percentile(kern, [10, 50, 90])]},
        "input_gen_s": round(t_gen, 1),
    }
    return res, src0


def cpu_baseline_meanpool(src, w, budget_s):
    """The oracle's conversion of whole matrices on the host, repeated for
    about `budget_s` seconds."""
    from oracle import meanpool_convert_ref

    x = src.double().numpy()
    byts = (w.H + w.K) * x.shape[2] * src.element_size()
    mats, t_used = 0, 0.0
    while t_used < budget_s:
        t0 = time.perf_counter()
        meanpool_convert_ref(x, w.K)
        t_used += time.perf_counter() - t0
        mats += 1
    return {"value": mats * byts / t_used / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{mats} whole matrices, {t_used:.1f} s of fp64 NumPy (element-wise: one thread)"}


HEADLINE = "decode_llama3_8b"
# The five configurations of the decode/prefill problem statement, by number;
# the headline line is configuration 2, the others are timed beside it.
CONFIGS = {1: "decode_tiny_f32", 2: "decode_llama3_8b", 3: "decode_70b_ragged", 4: "decode_long_131k",
           5: "prefill_causal_4k"}


def _compact(n, r):
    """The fields of one configuration's result kept in the sub-key."""
    rf = r["roofline"]
    c = {"config": n, "workload": r["config"]["workload"], "value": r["value"], "unit": r["unit"],
         "ms_per_step": r["ms_per_step"], "steps": r["steps"], "warmup": r["warmup"], "dtype": r["dtype"],
         "tokens_per_s": r.get("tokens_per_s"),
         "roofline": {k: rf[k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac", "traffic",
                                         "avg_kernel_us") if k in rf}}
    if "hbm_frac" in r:
        c["hbm_frac"] = r["hbm_frac"]
    if n == 1:
        c["note"] = ("0.5 MB of KV: held in the caches, latency-bound; the GB/s figures are no HBM claim "
                     "(the time per step is the result)")
    return c


def bench_other_configs(args):
    """Configurations 1, 3, 4 and 5, each timed on its own inputs (no CPU
    baseline), in the same run as the headline."""
    import copy

    from grouped_query_kv_amd.inputs import WORKLOADS

    out = {}
    for n, name in CONFIGS.items():
        if name == HEADLINE:
            continue
        w = WORKLOADS[name]
        sub = copy.copy(args)
        sub.steps, sub.warmup = max(1, args.config_steps), min(args.warmup, 5)
        if w.kind == "decode" and w.ragged is None and w.B * w.K * int(w.L) * w.d < (1 << 20):
            # a cache-resident decode of a few microseconds per step: enough
            # steps that one slow host-side launch does not set the mean
            sub.steps = max(sub.steps, 10 * args.config_steps)
        if w.kind == "prefill":
            # the matrix-core clock ramps over the first few hundred
            # microseconds of sustained work: warm it like the headline run
            sub.steps, sub.warmup = max(sub.steps, 50), max(sub.warmup, 20)
        print(f"bench: config {n} ({name}), {sub.steps} steps", file=sys.stderr, flush=True)
        if w.kind == "prefill":
            r, inp = bench_prefill(sub, w)
        else:
            r, inp = bench_decode(sub, w, sub=True)
        out[str(n)] = _compact(n, r)
        del inp, r
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    from grouped_query_kv_amd.inputs import WORKLOADS

    w = WORKLOADS[args.workload]
    if w.kind == "meanpool":
        res, inp = bench_meanpool(args, w)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_meanpool(inp, w, args.cpu_seconds)
    elif w.kind == "project":
        res, inp = bench_project(args, w)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_project(inp, w, args.cpu_seconds)
    elif w.kind in ("prefill", "chunk", "cross"):
        res, inp = bench_prefill(args, w)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_prefill(inp, w, args.cpu_seconds)
    else:
        res, inp = bench_decode(args, w)
        # the other configurations are timed before the CPU baseline, so that
        # no BLAS worker threads of the baseline compete with the launches
        if args.workload == HEADLINE and not args.no_configs:
            res["configs"] = bench_other_configs(args)
        if not args.no_cpu_baseline:
            res["cpu_baseline"] = cpu_baseline_decode(inp, w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
