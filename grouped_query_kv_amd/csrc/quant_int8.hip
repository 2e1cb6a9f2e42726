// int8 KV cache: per-row quantisation of cache rows and the quantising
// append.
//
// pinghaoyang.com.cn "GQA 完全拆解", the related-work list after the KV
// ledger: quantising the cached K and V to INT8 is orthogonal to GQA and the
// savings multiply; aicoding.csdn.net "LLaMa3与DeepSeek采用的GQA技术",
// section 3 (deployment tips): an 8-bit KV cache halves its memory.  The
// pages fix no rule, so this library uses symmetric absmax quantisation per
// cached row (one (sequence, KV head, position) row of d elements), all in
// IEEE fp32 with correctly rounded division:
//     amax = max_i |x_i|,  inv = 127 / amax,  c_i = clamp(rint(x_i * inv), -127, 127),
//     scale = amax / 127   (a zero row gets codes 0 and scale 0)
// and the row reads back as c_i * scale.
//
// Lane layout: a row is spread over D / 8 consecutive lanes of a wavefront,
// each holding 8 consecutive elements; the row maximum is a butterfly over
// those lanes (the groups are aligned, so every exchange stays inside one
// row).
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]);

template <>
__device__ __forceinline__ void load8<__bf16>(const __bf16* p, float (&x)[8]) {
  const u32x4 w = ld16(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

// Quantise the 8 elements of this lane, whose row spans LPR aligned lanes.
// Returns the 8 codes packed little-endian; *scale gets the row's scale.
template <int LPR>
__device__ __forceinline__ uint2 quantize8(const float (&x)[8], float* scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int o = LPR / 2; o >= 1; o /= 2) amax = fmaxf(amax, __shfl_xor(amax, o));
  uint32_t w[2] = {0u, 0u};
  if (amax > 0.f) {
    const float inv = int8_inv(amax);
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i / 4] |= (uint32_t)(int8_code(x[i], inv) & 0xff) << (8 * (i % 4));
    *scale = int8_scale(amax);
  } else {
    *scale = 0.f;
  }
  return uint2{w[0], w[1]};
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(const T* __restrict__ src,
                                                                 int8_t* __restrict__ codes,
                                                                 float* __restrict__ scales,
                                                                 int64_t rows) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  const int li = threadIdx.x % LPR;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int64_t rr = r < rows ? r : rows - 1;  // every lane of a row group takes part
  float x[8];
  load8<T>(src + rr * D + 8 * li, x);
  float s;
  const uint2 c = quantize8<LPR>(x, &s);
  if (r < rows) {
    *reinterpret_cast<uint2*>(codes + r * D + 8 * li) = c;
    if (li == 0) scales[r] = s;
  }
}

// One workgroup per sequence (as the plain append): every thread reads
// seq_lens[b] before the barrier, thread 0 writes it after.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void kv_append_int8_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new, int8_t* __restrict__ k_codes,
    int8_t* __restrict__ v_codes, float* __restrict__ k_scales, float* __restrict__ v_scales,
    int32_t* __restrict__ seq_lens, int K, int S_max) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;
  const int b = blockIdx.x;
  const int L = seq_lens[b];
  __syncthreads();
  if (L < 0 || L >= S_max) return;  // full (or corrupt) entry: write nothing
  const int li = threadIdx.x % LPR;
  // rows 2k (K head k) and 2k+1 (V head k)
  for (int r0 = 0; r0 < 2 * K; r0 += RPB) {
    const int r = r0 + threadIdx.x / LPR;
    const int rc = r < 2 * K ? r : 2 * K - 1;
    const int k = rc >> 1;
    const T* src = ((rc & 1) ? v_new : k_new) + ((size_t)b * K + k) * D + 8 * li;
    float x[8];
    load8<T>(src, x);
    float s;
    const uint2 c = quantize8<LPR>(x, &s);
    if (r < 2 * K) {
      const size_t row = ((size_t)b * K + k) * S_max + L;
      *reinterpret_cast<uint2*>(((rc & 1) ? v_codes : k_codes) + row * D + 8 * li) = c;
      if (li == 0) ((rc & 1) ? v_scales : k_scales)[row] = s;
    }
  }
  if (threadIdx.x == 0) seq_lens[b] = L + 1;
}

}  // namespace

hipError_t launch_quantize_rows_int8(const void* src, void* codes, float* scales, int64_t rows,
                                     int d, bool bf16, hipStream_t stream) {
  const int rpb = kThreads / (d / 8);
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  auto c = static_cast<int8_t*>(codes);
#define GQA_Q(T, DD)                                                                            \
  hipLaunchKernelGGL((quantize_rows_kernel<T, DD>), grid, dim3(kThreads), 0, stream,            \
                     static_cast<const T*>(src), c, scales, rows)
  if (bf16) {
    if (d == 128) GQA_Q(__bf16, 128); else GQA_Q(__bf16, 64);
  } else {
    if (d == 128) GQA_Q(float, 128); else GQA_Q(float, 64);
  }
#undef GQA_Q
  return hipGetLastError();
}

hipError_t launch_kv_append_int8(const void* k_new, const void* v_new, void* k_codes, void* v_codes,
                                 float* k_scales, float* v_scales, int32_t* seq_lens, int B, int K,
                                 int S_max, int d, bool bf16, hipStream_t stream) {
  auto kc = static_cast<int8_t*>(k_codes);
  auto vc = static_cast<int8_t*>(v_codes);
#define GQA_A(T, DD)                                                                            \
  hipLaunchKernelGGL((kv_append_int8_kernel<T, DD>), dim3(B), dim3(kThreads), 0, stream,        \
                     static_cast<const T*>(k_new), static_cast<const T*>(v_new), kc, vc,         \
                     k_scales, v_scales, seq_lens, K, S_max)
  if (bf16) {
    if (d == 128) GQA_A(__bf16, 128); else GQA_A(__bf16, 64);
  } else {
    if (d == 128) GQA_A(float, 128); else GQA_A(float, 64);
  }
#undef GQA_A
  return hipGetLastError();
}

}  // namespace gqa
