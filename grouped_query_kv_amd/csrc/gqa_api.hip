// C ABI of libgqa: argument validation, split planning and kernel launches.
// The declarations and their contracts are in include/gqa.h.
#include <cmath>
#include <cstdarg>
#include <algorithm>
#include <cstdio>
#include <mutex>
#include <string>

#include "gqa.h"
#include "gqa_internal.h"

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_ev_begin = nullptr;
thread_local hipEvent_t g_ev_end = nullptr;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return GQA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == GQA_F32 ? 4 : (dtype == GQA_BF16 ? 2 : 0); }

int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return GQA_OK;
}

// Launch with optional timing events around the main kernel.
struct TimedRegion {
  hipStream_t s;
  explicit TimedRegion(hipStream_t st) : s(st) {
    if (g_ev_begin && g_ev_end) (void)hipEventRecord(g_ev_begin, s);
  }
  ~TimedRegion() {
    if (g_ev_begin && g_ev_end) (void)hipEventRecord(g_ev_end, s);
  }
};

}  // namespace


extern "C" {

int gqa_abi_version(void) { return 1; }

#ifndef GQA_BUILD_ID
#error "GQA_BUILD_ID (the code hash of the sources) must be defined by the build"
#endif
const char* gqa_build_id(void) { return GQA_BUILD_ID; }

const char* gqa_last_error(void) { return g_last_error.c_str(); }

int gqa_set_timing_events(void* begin_event, void* end_event) {
  if ((begin_event == nullptr) != (end_event == nullptr))
    return fail(GQA_ERR_INVALID, "gqa_set_timing_events: pass two events or two NULLs");
  g_ev_begin = static_cast<hipEvent_t>(begin_event);
  g_ev_end = static_cast<hipEvent_t>(end_event);
  return ok();
}

uint64_t gqa_kv_cache_bytes(int layers, int K, int d, int elem_bytes_, uint64_t tokens) {
  if (layers < 0 || K < 0 || d < 0 || elem_bytes_ < 0) return 0;
  return 2ull * (uint64_t)layers * (uint64_t)K * (uint64_t)d * (uint64_t)elem_bytes_ * tokens;
}

int gqa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  int32_t* seq_lens, int B, int K, int S_max, int d, int dtype, void* stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !seq_lens)
    return fail(GQA_ERR_INVALID, "gqa_kv_append: null pointer");
  if (B < 1 || K < 1 || S_max < 1) return fail(GQA_ERR_INVALID, "gqa_kv_append: sizes must be >= 1");
  if (d != 64 && d != 128) return fail(GQA_ERR_UNSUPPORTED, "gqa_kv_append: d=%d (64 or 128)", d);
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(GQA_ERR_UNSUPPORTED, "gqa_kv_append: dtype %d", dtype);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return fail(GQA_ERR_INVALID, "gqa_kv_append: misaligned pointer");
  const int r = check_hip(gqa::launch_kv_append(k_new, v_new, k_cache, v_cache, seq_lens, B, K, S_max,
                                                d * eb, static_cast<hipStream_t>(stream)),
                          "gqa_kv_append launch");
  return r ? r : ok();
}

static int validate_heads(const char* fn, int B, int H, int K, int d) {
  if (B < 1 || H < 1 || K < 1) return fail(GQA_ERR_INVALID, "%s: B, H, K must be >= 1", fn);
  if (K > H || H % K != 0) return fail(GQA_ERR_INVALID, "%s: H=%d not a multiple of K=%d", fn, H, K);
  if (d != 64 && d != 128) return fail(GQA_ERR_UNSUPPORTED, "%s: d=%d (64 or 128)", fn, d);
  return GQA_OK;
}

// The flat split indexes positions with 32-bit integers.
static bool flat_fits(int B, int K, int max_seq_len) {
  return (long long)K * B * gqa::pad32(max_seq_len) < (1LL << 30);
}

size_t gqa_decode_workspace_bytes(int B, int H, int K, int max_seq_len, int d) {
  if (B < 1 || H < 1 || K < 1 || K > H || H % K || max_seq_len < 0 || (d != 64 && d != 128)) return 0;
  if (!flat_fits(B, K, max_seq_len)) return 0;
  return gqa::decode_workspace_bytes(B, H, K, max_seq_len, d);
}

// Shared body of gqa_decode and gqa_decode_append (k_new == nullptr: no append).
static int static_scratch(void** ptr);
static constexpr size_t kStaticScratchBytes = (size_t)64 << 20;

// workspace == nullptr with use_static: the partials go to the library's
// static scratch array of the current device (no allocation).
static int decode_impl(const char* fn, const void* q, const void* k_new, const void* v_new,
                       void* k_cache, void* v_cache, int32_t* seq_lens, void* out, void* workspace,
                       size_t workspace_bytes, int B, int H, int K, int S_max, int max_seq_len,
                       int d, float scale, int dtype, int out_dtype, void* stream,
                       bool use_static = false) {
  if (!q || !k_cache || !v_cache || !seq_lens || !out) return fail(GQA_ERR_INVALID, "%s: null pointer", fn);
  if (int r = validate_heads(fn, B, H, K, d)) return r;
  if (S_max < 1 || max_seq_len < 0 || max_seq_len > S_max)
    return fail(GQA_ERR_INVALID, "%s: need 0 <= max_seq_len <= S_max, S_max >= 1", fn);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(GQA_ERR_INVALID, "%s: scale must be finite and > 0", fn);
  if (dtype == GQA_F32) {
    if (out_dtype != GQA_F32) return fail(GQA_ERR_UNSUPPORTED, "%s: f32 input needs f32 output", fn);
  } else if (dtype == GQA_BF16) {
    if (out_dtype != GQA_BF16 && out_dtype != GQA_F32)
      return fail(GQA_ERR_UNSUPPORTED, "%s: out_dtype %d", fn, out_dtype);
  } else {
    return fail(GQA_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  }
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (k_new && (!aligned16(k_new) || !aligned16(v_new))) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return fail(GQA_ERR_INVALID, "%s: misaligned pointer", fn);
  if (!flat_fits(B, K, max_seq_len))
    return fail(GQA_ERR_UNSUPPORTED, "%s: B * K * max_seq_len too large (2^30 positions)", fn);
  const gqa::DecodePlan plan = gqa::plan_decode(B, H, K, max_seq_len, d,
                                                dtype == GQA_BF16 ? gqa::PassKind::kBf16 : gqa::PassKind::kF32);
  const size_t need = gqa::decode_workspace_bytes(B, H, K, max_seq_len, d);
  if (use_static) {
    if (need > kStaticScratchBytes)
      return fail(GQA_ERR_WORKSPACE,
                  "%s: these sizes need %zu bytes of scratch; the static scratch holds %zu "
                  "(use gqa_decode_append with a caller workspace)", fn, need, kStaticScratchBytes);
    if (int r = static_scratch(&workspace)) return r;
    workspace_bytes = kStaticScratchBytes;
  }
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(GQA_ERR_WORKSPACE, "%s: workspace needs %zu bytes (16-byte aligned), got %zu", fn,
                need, workspace ? workspace_bytes : (size_t)0);
  const gqa::DecodeWorkspace ws = gqa::carve_decode_workspace(workspace, plan, B, K, d);
  const float scale_log2 = scale * gqa::kLog2eHost;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int r;
  {
    TimedRegion timed(s);
    r = check_hip(dtype == GQA_BF16
                      ? gqa::launch_decode_split_bf16(q, k_cache, v_cache, seq_lens, ws, plan, B, H,
                                                      K, S_max, d, scale_log2, k_new, v_new,
                                                      nullptr, s)
                      : gqa::launch_decode_split_f32(q, k_cache, v_cache, seq_lens, ws, plan, B, H,
                                                     K, S_max, d, scale_log2, k_new, v_new, s),
                  "partition-pass launch");
  }
  if (r) return r;
  r = check_hip(gqa::launch_decode_combine(ws, seq_lens, out, plan, B, H, K, d,
                                           out_dtype == GQA_BF16, k_new != nullptr, s),
                "combine-pass launch");
  return r ? r : ok();
}

int gqa_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
               void* out, void* workspace, size_t workspace_bytes, int B, int H, int K, int S_max,
               int max_seq_len, int d, float scale, int dtype, int out_dtype, void* stream) {
  // read-only use of the caches and lengths (no append)
  return decode_impl("gqa_decode", q, nullptr, nullptr, const_cast<void*>(k_cache),
                     const_cast<void*>(v_cache), const_cast<int32_t*>(seq_lens), out, workspace,
                     workspace_bytes, B, H, K, S_max, max_seq_len, d, scale, dtype, out_dtype, stream);
}

int gqa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, int32_t* seq_lens, void* out, void* workspace,
                      size_t workspace_bytes, int B, int H, int K, int S_max, int max_seq_len, int d,
                      float scale, int dtype, int out_dtype, void* stream) {
  if (!k_new || !v_new) return fail(GQA_ERR_INVALID, "gqa_decode_append: null pointer");
  return decode_impl("gqa_decode_append", q, k_new, v_new, k_cache, v_cache, seq_lens, out,
                     workspace, workspace_bytes, B, H, K, S_max, max_seq_len, d, scale, dtype,
                     out_dtype, stream);
}

// ---- the allocation-free decode step ----
// The partials of gqa_decode_append_noalloc live in this file-scope device
// array (one copy per GPU, held until the process ends).  Its name is a
// host-side stand-in in host code: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept.  Nothing in it must start at zero: every partition that
// the combine pass reads is written by the partition pass of the same call.
// Calls that overlap on one GPU share the array and race.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int static_scratch(void** ptr) {
  int dev = -1;
  if (int r = check_hip(hipGetDevice(&dev), "hipGetDevice")) return r;
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GQA_ERR_UNSUPPORTED, "static scratch: device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (int r = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))
      return r;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u))
      return fail(GQA_ERR_HIP, "static scratch: bad device address %p", p);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return GQA_OK;
}

int gqa_decode_append_noalloc(const void* q, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, int32_t* seq_lens, void* out, int B, int H, int K,
                              int S_max, int max_seq_len, int d, float scale, int dtype,
                              int out_dtype, void* stream) {
  if (!k_new || !v_new) return fail(GQA_ERR_INVALID, "gqa_decode_append_noalloc: null pointer");
  return decode_impl("gqa_decode_append_noalloc", q, k_new, v_new, k_cache, v_cache, seq_lens, out,
                     nullptr, 0, B, H, K, S_max, max_seq_len, d, scale, dtype, out_dtype, stream,
                     /*use_static=*/true);
}

// Paged KV cache: the largest partition whose block ids fit one per lane.
static int paged_max_part_tokens(int block_size) { return 63 * block_size; }

static int validate_paged(const char* fn, int num_blocks, int block_size, int max_blocks) {
  if (num_blocks < 1 || max_blocks < 1) return fail(GQA_ERR_INVALID, "%s: num_blocks, max_blocks must be >= 1", fn);
  if (block_size < 16 || block_size % 16 != 0)
    return fail(GQA_ERR_UNSUPPORTED, "%s: block_size=%d (a multiple of 16)", fn, block_size);
  if ((long long)max_blocks * block_size > (1LL << 30))
    return fail(GQA_ERR_INVALID, "%s: table capacity too large", fn);
  return GQA_OK;
}

int gqa_kv_append_paged(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                        const int32_t* block_table, int32_t* seq_lens, int B, int K, int num_blocks,
                        int block_size, int max_blocks, int d, int dtype, void* stream) {
  const char* fn = "gqa_kv_append_paged";
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !seq_lens)
    return fail(GQA_ERR_INVALID, "%s: null pointer", fn);
  if (B < 1 || K < 1) return fail(GQA_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (int r = validate_paged(fn, num_blocks, block_size, max_blocks)) return r;
  if (d != 64 && d != 128) return fail(GQA_ERR_UNSUPPORTED, "%s: d=%d (64 or 128)", fn, d);
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(GQA_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) || (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return fail(GQA_ERR_INVALID, "%s: misaligned pointer", fn);
  const gqa::PagedArgs pg{block_table, block_size, max_blocks, num_blocks};
  const int r = check_hip(gqa::launch_kv_append_paged(k_new, v_new, k_pool, v_pool, pg, seq_lens, B, K,
                                                      d * eb, static_cast<hipStream_t>(stream)),
                          "gqa_kv_append_paged launch");
  return r ? r : ok();
}

size_t gqa_decode_paged_workspace_bytes(int B, int H, int K, int max_seq_len, int d, int block_size) {
  if (B < 1 || H < 1 || K < 1 || K > H || H % K || max_seq_len < 0 || (d != 64 && d != 128) ||
      block_size < 16 || block_size % 16)
    return 0;
  if (!flat_fits(B, K, max_seq_len)) return 0;
  return gqa::decode_workspace_bytes(B, H, K, max_seq_len, d, paged_max_part_tokens(block_size));
}

// Shared body of gqa_decode_paged and gqa_decode_append_paged (k_new == nullptr: no append).
static int decode_paged_impl(const char* fn, const void* q, const void* k_new, const void* v_new,
                             void* k_pool, void* v_pool, const int32_t* block_table,
                             int32_t* seq_lens, void* out, void* workspace, size_t workspace_bytes,
                             int B, int H, int K, int num_blocks, int block_size, int max_blocks,
                             int max_seq_len, int d, float scale, int dtype, int out_dtype,
                             void* stream) {
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !out)
    return fail(GQA_ERR_INVALID, "%s: null pointer", fn);
  if (int r = validate_heads(fn, B, H, K, d)) return r;
  if (int r = validate_paged(fn, num_blocks, block_size, max_blocks)) return r;
  if (max_seq_len < 0 || max_seq_len > max_blocks * block_size)
    return fail(GQA_ERR_INVALID, "%s: need 0 <= max_seq_len <= max_blocks * block_size", fn);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(GQA_ERR_INVALID, "%s: scale must be finite and > 0", fn);
  if (dtype != GQA_BF16) return fail(GQA_ERR_UNSUPPORTED, "%s: paged caches are bf16", fn);
  if (out_dtype != GQA_BF16 && out_dtype != GQA_F32)
    return fail(GQA_ERR_UNSUPPORTED, "%s: out_dtype %d", fn, out_dtype);
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) ||
      (k_new && (!aligned16(k_new) || !aligned16(v_new))) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u) || (reinterpret_cast<uintptr_t>(block_table) & 3u))
    return fail(GQA_ERR_INVALID, "%s: misaligned pointer", fn);
  if (!flat_fits(B, K, max_seq_len))
    return fail(GQA_ERR_UNSUPPORTED, "%s: B * K * max_seq_len too large (2^30 positions)", fn);
  const gqa::DecodePlan plan = gqa::plan_decode(B, H, K, max_seq_len, d, gqa::PassKind::kBf16,
                                                paged_max_part_tokens(block_size));
  const size_t need =
      gqa::decode_workspace_bytes(B, H, K, max_seq_len, d, paged_max_part_tokens(block_size));
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(GQA_ERR_WORKSPACE, "%s: workspace needs %zu bytes (16-byte aligned), got %zu", fn,
                need, workspace ? workspace_bytes : (size_t)0);
  const gqa::DecodeWorkspace ws = gqa::carve_decode_workspace(workspace, plan, B, K, d);
  const gqa::PagedArgs pg{block_table, block_size, max_blocks, num_blocks};
  hipStream_t s = static_cast<hipStream_t>(stream);
  int r;
  {
    TimedRegion timed(s);
    r = check_hip(gqa::launch_decode_split_bf16(q, k_pool, v_pool, seq_lens, ws, plan, B, H, K,
                                                max_blocks * block_size, d, scale * gqa::kLog2eHost,
                                                k_new, v_new, &pg, s),
                  "partition-pass launch");
  }
  if (r) return r;
  r = check_hip(gqa::launch_decode_combine(ws, seq_lens, out, plan, B, H, K, d,
                                           out_dtype == GQA_BF16, k_new != nullptr, s),
                "combine-pass launch");
  return r ? r : ok();
}

int gqa_decode_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                     const int32_t* seq_lens, void* out, void* workspace, size_t workspace_bytes,
                     int B, int H, int K, int num_blocks, int block_size, int max_blocks,
                     int max_seq_len, int d, float scale, int dtype, int out_dtype, void* stream) {
  // read-only use of the pools and lengths (no append)
  return decode_paged_impl("gqa_decode_paged", q, nullptr, nullptr, const_cast<void*>(k_pool),
                           const_cast<void*>(v_pool), block_table, const_cast<int32_t*>(seq_lens),
                           out, workspace, workspace_bytes, B, H, K, num_blocks, block_size,
                           max_blocks, max_seq_len, d, scale, dtype, out_dtype, stream);
}

int gqa_decode_append_paged(const void* q, const void* k_new, const void* v_new, void* k_pool,
                            void* v_pool, const int32_t* block_table, int32_t* seq_lens, void* out,
                            void* workspace, size_t workspace_bytes, int B, int H, int K,
                            int num_blocks, int block_size, int max_blocks, int max_seq_len, int d,
                            float scale, int dtype, int out_dtype, void* stream) {
  if (!k_new || !v_new) return fail(GQA_ERR_INVALID, "gqa_decode_append_paged: null pointer");
  return decode_paged_impl("gqa_decode_append_paged", q, k_new, v_new, k_pool, v_pool, block_table,
                           seq_lens, out, workspace, workspace_bytes, B, H, K, num_blocks,
                           block_size, max_blocks, max_seq_len, d, scale, dtype, out_dtype, stream);
}

int gqa_kv_quantize_int8(const void* src, void* codes, float* scales, int64_t rows, int d, int dtype,
                         void* stream) {
  const char* fn = "gqa_kv_quantize_int8";
  if (!src || !codes || !scales) return fail(GQA_ERR_INVALID, "%s: null pointer", fn);
  if (rows < 1) return fail(GQA_ERR_INVALID, "%s: rows must be >= 1", fn);
  if (d != 64 && d != 128) return fail(GQA_ERR_UNSUPPORTED, "%s: d=%d (64 or 128)", fn, d);
  if (dtype != GQA_F32 && dtype != GQA_BF16) return fail(GQA_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (!aligned16(src) || (reinterpret_cast<uintptr_t>(codes) & 7u) ||
      (reinterpret_cast<uintptr_t>(scales) & 3u))
    return fail(GQA_ERR_INVALID, "%s: misaligned pointer", fn);
  const int r = check_hip(gqa::launch_quantize_rows_int8(src, codes, scales, rows, d, dtype == GQA_BF16,
                                                         static_cast<hipStream_t>(stream)),
                          "quantize launch");
  return r ? r : ok();
}

int gqa_kv_append_int8(const void* k_new, const void* v_new, void* k_codes, void* v_codes,
                       float* k_scales, float* v_scales, int32_t* seq_lens, int B, int K, int S_max,
                       int d, int dtype, void* stream) {
  const char* fn = "gqa_kv_append_int8";
  if (!k_new || !v_new || !k_codes || !v_codes || !k_scales || !v_scales || !seq_lens)
    return fail(GQA_ERR_INVALID, "%s: null pointer", fn);
  if (B < 1 || K < 1 || S_max < 1) return fail(GQA_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (d != 64 && d != 128) return fail(GQA_ERR_UNSUPPORTED, "%s: d=%d (64 or 128)", fn, d);
  if (dtype != GQA_F32 && dtype != GQA_BF16) return fail(GQA_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_codes) || !aligned16(v_codes) ||
      (reinterpret_cast<uintptr_t>(k_scales) & 3u) || (reinterpret_cast<uintptr_t>(v_scales) & 3u) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return fail(GQA_ERR_INVALID, "%s: misaligned pointer", fn);
  const int r = check_hip(gqa::launch_kv_append_int8(k_new, v_new, k_codes, v_codes, k_scales, v_scales,
                                                     seq_lens, B, K, S_max, d, dtype == GQA_BF16,
                                                     static_cast<hipStream_t>(stream)),
                          "append launch");
  return r ? r : ok();
}

// Shared body of gqa_decode_int8 and gqa_decode_append_int8 (k_new == nullptr: no append).
static int decode_int8_impl(const char* fn, const void* q, const void* k_new, const void* v_new,
                            void* k_codes, void* v_codes, float* k_scales, float* v_scales,
                            int32_t* seq_lens, void* out, void* workspace, size_t workspace_bytes,
                            int B, int H, int K, int S_max, int max_seq_len, int d, float scale,
                            int q_dtype, int out_dtype, void* stream) {
  if (!q || !k_codes || !v_codes || !k_scales || !v_scales || !seq_lens || !out)
    return fail(GQA_ERR_INVALID, "%s: null pointer", fn);
  if (int r = validate_heads(fn, B, H, K, d)) return r;
  if (S_max < 4 || S_max % 4 != 0 || max_seq_len < 0 || max_seq_len > S_max)
    return fail(GQA_ERR_INVALID, "%s: need S_max a positive multiple of 4 and 0 <= max_seq_len <= S_max", fn);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(GQA_ERR_INVALID, "%s: scale must be finite and > 0", fn);
  if (q_dtype != GQA_BF16) return fail(GQA_ERR_UNSUPPORTED, "%s: queries must be bf16", fn);
  if (out_dtype != GQA_BF16 && out_dtype != GQA_F32)
    return fail(GQA_ERR_UNSUPPORTED, "%s: out_dtype %d", fn, out_dtype);
  if (!aligned16(q) || !aligned16(k_codes) || !aligned16(v_codes) || !aligned16(k_scales) ||
      !aligned16(v_scales) || !aligned16(out) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u) ||
      (k_new && (!aligned16(k_new) || !aligned16(v_new))))
    return fail(GQA_ERR_INVALID, "%s: misaligned pointer", fn);
  if (!flat_fits(B, K, max_seq_len))
    return fail(GQA_ERR_UNSUPPORTED, "%s: B * K * max_seq_len too large (2^30 positions)", fn);
  const gqa::DecodePlan plan = gqa::plan_decode(B, H, K, max_seq_len, d, gqa::PassKind::kInt8);
  const size_t need = gqa::decode_workspace_bytes(B, H, K, max_seq_len, d);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(GQA_ERR_WORKSPACE, "%s: workspace needs %zu bytes (16-byte aligned), got %zu", fn,
                need, workspace ? workspace_bytes : (size_t)0);
  const gqa::DecodeWorkspace ws = gqa::carve_decode_workspace(workspace, plan, B, K, d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int r;
  {
    TimedRegion timed(s);
    r = check_hip(gqa::launch_decode_split_int8(q, k_codes, v_codes, k_scales, v_scales, seq_lens, ws,
                                                plan, B, H, K, S_max, d, scale * gqa::kLog2eHost,
                                                k_new, v_new, s),
                  "partition-pass launch");
  }
  if (r) return r;
  r = check_hip(gqa::launch_decode_combine(ws, seq_lens, out, plan, B, H, K, d,
                                           out_dtype == GQA_BF16, k_new != nullptr, s),
                "combine-pass launch");
  return r ? r : ok();
}

int gqa_decode_int8(const void* q, const void* k_codes, const void* v_codes, const float* k_scales,
                    const float* v_scales, const int32_t* seq_lens, void* out, void* workspace,
                    size_t workspace_bytes, int B, int H, int K, int S_max, int max_seq_len, int d,
                    float scale, int q_dtype, int out_dtype, void* stream) {
  // read-only use of the cache and lengths (no append)
  return decode_int8_impl("gqa_decode_int8", q, nullptr, nullptr, const_cast<void*>(k_codes),
                          const_cast<void*>(v_codes), const_cast<float*>(k_scales),
                          const_cast<float*>(v_scales), const_cast<int32_t*>(seq_lens), out,
                          workspace, workspace_bytes, B, H, K, S_max, max_seq_len, d, scale,
                          q_dtype, out_dtype, stream);
}

int gqa_decode_append_int8(const void* q, const void* k_new, const void* v_new, void* k_codes,
                           void* v_codes, float* k_scales, float* v_scales, int32_t* seq_lens,
                           void* out, void* workspace, size_t workspace_bytes, int B, int H, int K,
                           int S_max, int max_seq_len, int d, float scale, int dtype, int out_dtype,
                           void* stream) {
  if (!k_new || !v_new) return fail(GQA_ERR_INVALID, "gqa_decode_append_int8: null pointer");
  return decode_int8_impl("gqa_decode_append_int8", q, k_new, v_new, k_codes, v_codes, k_scales,
                          v_scales, seq_lens, out, workspace, workspace_bytes, B, H, K, S_max,
                          max_seq_len, d, scale, dtype, out_dtype, stream);
}

// Shared validation and launch of the prefill family.
static int prefill_impl(const char* fn, const void* q, const void* k, const void* v, void* out,
                        const int32_t* kv_lens, int B, int H, int K, int S, int S_kv, int S_max,
                        int d, float scale, int dtype, int out_dtype, bool causal, void* stream) {
  if (!q || !k || !v || !out) return fail(GQA_ERR_INVALID, "%s: null pointer", fn);
  if (int r = validate_heads(fn, B, H, K, d)) return r;
  if (S < 1 || S_max < 1 || S_kv > S_max)
    return fail(GQA_ERR_INVALID, "%s: need S >= 1 and key lengths <= S_max", fn);
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(GQA_ERR_INVALID, "%s: scale must be finite and > 0", fn);
  if (dtype == GQA_F32) {
    if (out_dtype != GQA_F32) return fail(GQA_ERR_UNSUPPORTED, "%s: f32 input needs f32 output", fn);
  } else if (dtype == GQA_BF16) {
    if (out_dtype != GQA_BF16 && out_dtype != GQA_F32)
      return fail(GQA_ERR_UNSUPPORTED, "%s: out_dtype %d", fn, out_dtype);
  } else {
    return fail(GQA_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  }
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(kv_lens) & 3u))
    return fail(GQA_ERR_INVALID, "%s: misaligned pointer", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int r;
  {
    TimedRegion timed(s);
    r = check_hip(dtype == GQA_BF16
                      ? gqa::launch_prefill_bf16(q, k, v, out, kv_lens, B, H, K, S, S_kv, S_max, d,
                                                 scale * gqa::kLog2eHost, out_dtype == GQA_BF16, causal, s)
                      : gqa::launch_prefill_f32(q, k, v, out, kv_lens, B, H, K, S, S_kv, S_max, d,
                                                scale * gqa::kLog2eHost, causal, s),
                  "prefill launch");
  }
  return r ? r : ok();
}

int gqa_prefill_causal(const void* q, const void* k, const void* v, void* out, int B, int H, int K,
                       int S, int S_max, int d, float scale, int dtype, int out_dtype, void* stream) {
  if (S < 1 || S_max < S) return fail(GQA_ERR_INVALID, "gqa_prefill_causal: need 1 <= S <= S_max");
  return prefill_impl("gqa_prefill_causal", q, k, v, out, nullptr, B, H, K, S, S, S_max, d, scale,
                      dtype, out_dtype, true, stream);
}

int gqa_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens,
                      void* out, int B, int H, int K, int S, int S_max, int d, float scale, int dtype,
                      int out_dtype, void* stream) {
  if (!seq_lens) return fail(GQA_ERR_INVALID, "gqa_prefill_chunk: null pointer");
  if (S < 1 || S_max < S) return fail(GQA_ERR_INVALID, "gqa_prefill_chunk: need 1 <= S <= S_max");
  return prefill_impl("gqa_prefill_chunk", q, k_cache, v_cache, out, seq_lens, B, H, K, S, 0, S_max, d,
                      scale, dtype, out_dtype, true, stream);
}

int gqa_cross_attention(const void* q, const void* k, const void* v, const int32_t* kv_lens, void* out,
                        int B, int H, int K, int S_q, int S_max, int d, float scale, int dtype,
                        int out_dtype, void* stream) {
  if (!kv_lens) return fail(GQA_ERR_INVALID, "gqa_cross_attention: null pointer");
  return prefill_impl("gqa_cross_attention", q, k, v, out, kv_lens, B, H, K, S_q, 0, S_max, d, scale,
                      dtype, out_dtype, false, stream);
}

int gqa_kv_append_rows(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       int32_t* seq_lens, int B, int K, int T, int S_max, int d, int dtype, void* stream) {
  const char* fn = "gqa_kv_append_rows";
  if (!k_new || !v_new || !k_cache || !v_cache || !seq_lens) return fail(GQA_ERR_INVALID, "%s: null pointer", fn);
  if (B < 1 || K < 1 || T < 1 || S_max < 1) return fail(GQA_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (d != 64 && d != 128) return fail(GQA_ERR_UNSUPPORTED, "%s: d=%d (64 or 128)", fn, d);
  const int eb = elem_bytes(dtype);
  if (!eb) return fail(GQA_ERR_UNSUPPORTED, "%s: dtype %d", fn, dtype);
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return fail(GQA_ERR_INVALID, "%s: misaligned pointer", fn);
  const int r = check_hip(gqa::launch_kv_append_rows(k_new, v_new, k_cache, v_cache, seq_lens, B, K, T,
                                                     S_max, d * eb, static_cast<hipStream_t>(stream)),
                          "append launch");
  return r ? r : ok();
}

static int validate_project(const char* fn, int B, int T, int d_model, int K, int d, int dtype) {
  if (B < 1 || T < 1 || K < 1 || d_model < 1) return fail(GQA_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (d != 64 && d != 128) return fail(GQA_ERR_UNSUPPORTED, "%s: d=%d (64 or 128)", fn, d);
  if (d_model % 32 != 0) return fail(GQA_ERR_UNSUPPORTED, "%s: d_model=%d (a multiple of 32)", fn, d_model);
  if (dtype != GQA_BF16) return fail(GQA_ERR_UNSUPPORTED, "%s: bf16 only (matrix-core path)", fn);
  if ((long long)B * T > (1LL << 24) || (long long)B * T * K * d > (1LL << 30))
    return fail(GQA_ERR_INVALID, "%s: too many tokens", fn);
  return GQA_OK;
}

int gqa_kv_project(const void* x, const void* w_kv, void* k_out, void* v_out, int B, int T, int d_model,
                   int K, int d, int dtype, void* stream) {
  const char* fn = "gqa_kv_project";
  if (!x || !w_kv || !k_out || !v_out) return fail(GQA_ERR_INVALID, "%s: null pointer", fn);
  if (int r = validate_project(fn, B, T, d_model, K, d, dtype)) return r;
  if (!aligned16(x) || !aligned16(w_kv) || (reinterpret_cast<uintptr_t>(k_out) & 1u) ||
      (reinterpret_cast<uintptr_t>(v_out) & 1u))
    return fail(GQA_ERR_INVALID, "%s: misaligned pointer", fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int r;
  {
    TimedRegion timed(s);
    r = check_hip(gqa::launch_kv_project(x, w_kv, k_out, v_out, B, T, d_model, K, d, s), "projection launch");
  }
  return r ? r : ok();
}

size_t gqa_kv_project_workspace_bytes(int B, int T, int d_model, int K, int d) {
  if (B < 1 || T < 1 || K < 1 || d_model < 32 || d_model % 32 || (d != 64 && d != 128) ||
      (long long)B * T > (1LL << 24) || (long long)B * T * K * d > (1LL << 30))
    return 0;
  return 2 * (size_t)B * T * K * d * 2;  // the K and V rows, bf16
}

int gqa_kv_project_append(const void* x, const void* w_kv, void* k_cache, void* v_cache,
                          int32_t* seq_lens, void* workspace, size_t workspace_bytes, int B, int T,
                          int d_model, int K, int S_max, int d, int dtype, void* stream) {
  const char* fn = "gqa_kv_project_append";
  if (!x || !w_kv || !k_cache || !v_cache || !seq_lens) return fail(GQA_ERR_INVALID, "%s: null pointer", fn);
  if (S_max < 1) return fail(GQA_ERR_INVALID, "%s: sizes must be >= 1", fn);
  if (int r = validate_project(fn, B, T, d_model, K, d, dtype)) return r;
  if (!aligned16(x) || !aligned16(w_kv) || !aligned16(k_cache) || !aligned16(v_cache) ||
      (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return fail(GQA_ERR_INVALID, "%s: misaligned pointer", fn);
  const size_t rows_bytes = (size_t)B * T * K * d * 2;
  if (!workspace || workspace_bytes < 2 * rows_bytes || !aligned16(workspace))
    return fail(GQA_ERR_WORKSPACE, "%s: workspace needs %zu bytes (16-byte aligned), got %zu", fn,
                2 * rows_bytes, workspace ? workspace_bytes : (size_t)0);
  char* k_rows = static_cast<char*>(workspace);
  char* v_rows = k_rows + rows_bytes;  // rows_bytes is a multiple of 128
  hipStream_t s = static_cast<hipStream_t>(stream);
  int r;
  {
    TimedRegion timed(s);
    r = check_hip(gqa::launch_kv_project(x, w_kv, k_rows, v_rows, B, T, d_model, K, d, s), "projection launch");
  }
  if (r) return r;
  r = check_hip(gqa::launch_kv_append_rows(k_rows, v_rows, k_cache, v_cache, seq_lens, B, K, T, S_max, d * 2, s),
                "append launch");
  return r ? r : ok();
}

int gqa_meanpool_convert(const void* src, void* dst, int64_t outer, int H, int K, int64_t inner,
                         int dtype, void* stream) {
  if (!src || !dst) return fail(GQA_ERR_INVALID, "gqa_meanpool_convert: null pointer");
  if (outer < 1 || inner < 1 || H < 1 || K < 1)
    return fail(GQA_ERR_INVALID, "gqa_meanpool_convert: sizes must be >= 1");
  if (K > H || H % K) return fail(GQA_ERR_INVALID, "gqa_meanpool_convert: H=%d not a multiple of K=%d", H, K);
  if (!elem_bytes(dtype)) return fail(GQA_ERR_UNSUPPORTED, "gqa_meanpool_convert: dtype %d", dtype);
  if (!aligned16(src) || !aligned16(dst)) return fail(GQA_ERR_INVALID, "gqa_meanpool_convert: misaligned pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int r;
  {
    TimedRegion timed(s);
    r = check_hip(gqa::launch_meanpool(src, dst, outer, H, K, inner, dtype == GQA_BF16, s),
                  "gqa_meanpool_convert launch");
  }
  return r ? r : ok();
}

}  // extern "C"
