// Fused K/V projection (and cache append).
//
// pinghaoyang.com.cn "GQA 完全拆解", section 工程实现 (engineering): GQA's key
// and value projections are [K, d, d_model] each (K KV heads); inference
// frameworks merge them into one W_KV [K, 2d, d_model] so that one GEMM
// yields both K and V.  For token t of sequence b (hidden state x[b, t, :]):
//     K_k = W_KV[k, 0:d] x,   V_k = W_KV[k, d:2d] x     (fp32 accumulation, bf16 out)
// written as rows [B, K, T, d] -- the layout the appends take -- so a decode
// step can hand them to the fused append of the attention pass, or have
// them copied into the cache (gqa_kv_project_append).
//
// One 512-thread workgroup per (16 or 8 rows of W_KV, 16 tokens): the
// product Y^T[16 rows x 16 tokens] = W_tile[16 x d_model] . X^T runs on
// v_mfma_f32_16x16x32_bf16 with W rows as the A operand and token rows as
// the B operand (lane (n, g) at k-step s carries d_model entries
// 32 s + 8 g .. +7 of its row for both, so every operand is one 16-byte
// load).  The 8 wavefronts split d_model into 8 slices, issue up to 16
// k-steps of loads at once, and their partial tiles are summed through LDS.
// For a decode step (16 or fewer tokens) each W_KV byte is read from HBM
// exactly once.  When 16-row tiles would give fewer than 256 workgroups (a
// decode step: 128 tiles for Llama-3-8B's W_KV, half the CUs idle), tiles
// of 8 rows are used and the matrix cores' other 8 rows are zero: the
// product costs nothing here, the bytes in flight are spread over every CU
// (measured 11.0 -> 9.3 us on the Llama-3-8B decode step).  A tile never
// straddles the K/V halves or two heads (d is a multiple of 16).
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kWaves = 8;
constexpr int kUnroll = 16;  // k-steps whose loads are issued together

template <int D, int ROWS>
__global__ __launch_bounds__(64 * kWaves) void kv_project_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ w, __bf16* __restrict__ k_out,
    __bf16* __restrict__ v_out, int M, int T, int dm, int K) {
  __shared__ float red[kWaves][16][17];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int r0 = blockIdx.x * ROWS;  // first W_KV row (output feature) of the tile
  const int m0 = blockIdx.y * 16;  // first token of the tile
  // 32-wide k-steps of d_model, split as evenly as possible over the waves
  const int nsteps = dm / 32;
  const int per = (nsteps + kWaves - 1) / kWaves;
  const int s_begin = min(wave * per, nsteps);
  const int steps = min(per, nsteps - s_begin);

  const bool row_ok = n < ROWS;  // operand rows past the tile stay zero
  const __bf16* wrow = w + (size_t)(r0 + (row_ok ? n : 0)) * dm + 32 * s_begin + 8 * g;
  const bool tok_ok = m0 + n < M;
  const __bf16* xrow = x + (size_t)(tok_ok ? m0 + n : 0) * dm + 32 * s_begin + 8 * g;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < steps; s0 += kUnroll) {
    u32x4 a[kUnroll], bq[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool in = s0 + u < steps;
      a[u] = in && row_ok ? ld16(wrow + 32 * (s0 + u)) : zero_u32x4();
      bq[u] = in && tok_ok ? ld16(xrow + 32 * (s0 + u)) : zero_u32x4();
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[u]), as_bf16x8(bq[u]), acc, 0, 0, 0);
  }
  // lane holds Y^T[4g + i][n]: feature r0 + 4g + i of token m0 + n
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][4 * g + i][n] = acc[i];
  __syncthreads();
  if (tid < 16 * ROWS) {
    const int f = tid % ROWS;   // feature within the tile (fast index: contiguous stores)
    const int tk = tid / ROWS;  // token within the tile
    const int m = m0 + tk;
    if (m < M) {
      float y = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) y += red[v][f][tk];
      const int b = m / T;
      const int t = m - b * T;
      const int feat = r0 + f;
      const int head = feat / (2 * D);
      const int j = feat - head * 2 * D;
      __bf16* dst = j < D ? k_out : v_out;
      dst[(((size_t)b * K + head) * T + t) * D + (j < D ? j : j - D)] = static_cast<__bf16>(y);
    }
  }
}

}  // namespace

hipError_t launch_kv_project(const void* x, const void* w_kv, void* k_out, void* v_out, int B, int T,
                             int d_model, int K, int d, hipStream_t stream) {
  const int M = B * T;
  const bool narrow = (long long)(K * 2 * d / 16) * ((M + 15) / 16) < 256;
  const int rows = narrow ? 8 : 16;
  const dim3 grid(K * 2 * d / rows, (M + 15) / 16);
#define GQA_PROJ(DD, RR)                                                                        \
  hipLaunchKernelGGL((kv_project_kernel<DD, RR>), grid, dim3(64 * kWaves), 0, stream,            \
                     static_cast<const __bf16*>(x), static_cast<const __bf16*>(w_kv),             \
                     static_cast<__bf16*>(k_out), static_cast<__bf16*>(v_out), M, T, d_model, K)
  if (d == 128) {
    if (narrow) GQA_PROJ(128, 8); else GQA_PROJ(128, 16);
  } else {
    if (narrow) GQA_PROJ(64, 8); else GQA_PROJ(64, 16);
  }
#undef GQA_PROJ
  return hipGetLastError();
}

}  // namespace gqa
