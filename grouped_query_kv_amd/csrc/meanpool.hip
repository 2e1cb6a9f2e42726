// Mean-pool conversion of per-head weights into group weights:
//   dst[o, g, i] = (sum_{r < G} src[o, g*G + r, i]) / G.
//
// pinghaoyang.com.cn "GQA 完全拆解", section Uptraining：把现成 MHA 检查点改造成
// GQA (the key and value projections of a group are replaced by the mean of
// its heads' projections); compassingai.com "分組查詢注意力", section 技術原理
// (arithmetic mean over the H/K heads of a group; queries unchanged).
//
// Rounding rule: the sum runs in fp32 in head order r = 0..G-1 and is then
// divided once by G with IEEE division, then rounded to the element type.
// For G identical bf16 inputs every partial sum r*x is exact in fp32 (8
// significant bits times r < 2^16), so the result is exactly x.
//
// Memory-bound elementwise pass: each thread handles one 16-byte word of
// the output row (8 bf16 or 4 fp32 elements) and reads the G matching words
// (bytes per output word: 16 G read + 16 written).
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void meanpool_vec_kernel(const u32x4* __restrict__ src,
                                                           u32x4* __restrict__ dst, int64_t rows,
                                                           int H, int K, int64_t words) {
  constexpr int E = BF16 ? 8 : 4;  // elements per 16-byte word
  constexpr int R = 8;             // head words loaded together
  const int G = H / K;
  const float den = (float)G;
  // grid: y walks the output rows (o, g), x the 16-byte words of a row, so
  // no per-element division is needed; a row's G source rows are read with
  // up to R loads in flight per thread and summed in head order
  for (int64_t row = blockIdx.y; row < rows; row += gridDim.y) {
    const int64_t o = row / K;
    const int g = (int)(row - o * K);
    const u32x4* s0 = src + (o * H + (int64_t)g * G) * words;
    u32x4* d0 = dst + row * words;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x) {
      float s[E];
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] = 0.f;
      for (int r0 = 0; r0 < G; r0 += R) {
        u32x4 x[R];
#pragma unroll
        for (int j = 0; j < R; ++j) x[j] = r0 + j < G ? ld16_stream(s0 + (int64_t)(r0 + j) * words + i) : zero_u32x4();
#pragma unroll
        for (int j = 0; j < R; ++j) {
          if (r0 + j >= G) break;
          if (BF16) {
#pragma unroll
            for (int e = 0; e < E; ++e) s[e] += bf16_bits_to_f32((x[j][e / 2] >> (16 * (e & 1))) & 0xffffu);
          } else {
            // whole-vector reinterpretation (a per-element bit_cast of a vector
            // subscript is not used: it has been seen to read element 0 only)
            const f32x4 xf = __builtin_bit_cast(f32x4, x[j]);
#pragma unroll
            for (int e = 0; e < E; ++e) s[e] += xf[e];
          }
        }
      }
      u32x4 y;
      if (BF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = pack_bf16x2(s[2 * j] / den, s[2 * j + 1] / den);
      } else {
        y = __builtin_bit_cast(u32x4, f32x4{s[0] / den, s[1] / den, s[2] / den, s[3] / den});
      }
      d0[i] = y;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void meanpool_scalar_kernel(const T* __restrict__ src,
                                                              T* __restrict__ dst, int64_t outer,
                                                              int H, int K, int64_t inner) {
  const int G = H / K;
  const int64_t total = outer * K * inner;
  for (int64_t w = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; w < total;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = w % inner;
    const int64_t og = w / inner;
    const int g = (int)(og % K);
    const int64_t o = og / K;
    float s = 0.f;
    for (int r = 0; r < G; ++r) s += static_cast<float>(src[(o * H + (int64_t)g * G + r) * inner + i]);
    dst[w] = static_cast<T>(s / (float)G);
  }
}

int grid_for(int64_t total) {
  const int64_t blocks = (total + 255) / 256;
  return (int)(blocks < 65536 ? (blocks > 0 ? blocks : 1) : 65536);
}

}  // namespace

hipError_t launch_meanpool(const void* src, void* dst, int64_t outer, int H, int K, int64_t inner,
                           bool bf16, hipStream_t stream) {
  const int E = bf16 ? 8 : 4;
  if (inner % E == 0) {
    const int64_t words = inner / E;
    const int64_t rows = outer * K;
    const int64_t bx = (words + 255) / 256;
    const dim3 grid((unsigned)(bx < 4096 ? bx : 4096), (unsigned)(rows < 65535 ? rows : 65535));
    if (bf16)
      hipLaunchKernelGGL(meanpool_vec_kernel<true>, grid, dim3(256), 0, stream,
                         static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), rows, H, K, words);
    else
      hipLaunchKernelGGL(meanpool_vec_kernel<false>, grid, dim3(256), 0, stream,
                         static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), rows, H, K, words);
  } else {
    const int grid = grid_for(outer * K * inner);
    if (bf16)
      hipLaunchKernelGGL(meanpool_scalar_kernel<__bf16>, dim3(grid), dim3(256), 0, stream,
                         static_cast<const __bf16*>(src), static_cast<__bf16*>(dst), outer, H, K, inner);
    else
      hipLaunchKernelGGL(meanpool_scalar_kernel<float>, dim3(grid), dim3(256), 0, stream,
                         static_cast<const float*>(src), static_cast<float*>(dst), outer, H, K, inner);
  }
  return hipGetLastError();
}

}  // namespace gqa
