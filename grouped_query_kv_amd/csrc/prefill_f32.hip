// GQA prefill family for fp32 inputs, on the vector ALUs (fp32 end to end):
// causal prefill, prefill of a chunk over a cache, non-causal
// cross-attention -- the same masks and layouts as the bf16 matrix-core
// kernel (prefill_bf16.hip):
//
// out[b,h,i,:] = sum_{j visible} softmax_j(scale q[b,h,i,:] . k[b,h/G,j,:]) v[b,h/G,j,:]
//
// with L_b keys (kv_lens[b], or S_kv for every sequence) and S queries: key
// j is visible to query i iff j < L_b and, when causal, j <= L_b - S + i; a
// query with no visible key gets a zero row.  (pinghaoyang.com.cn "GQA 完全拆解",
// sections 解码推理的内存账本 (prefill attends over the whole prefix; row i is
// decode step i) and 工程实现 (a group's shared K/V block is staged once
// and reused by all its query heads); compassingai.com "分組查詢注意力", 技術原理.)
//
// One 256-thread workgroup per (sequence, KV head, 4 heads of the group, 16
// query positions): 64 query rows that all read the same K/V tiles.  Thread
// t owns row r = t / 4 and quarter c = t % 4.  Per 32-key tile staged in LDS:
//   1. scores of row r against keys 8c .. 8c + 7 (query row broadcast from
//      LDS to the row's four threads);
//   2. base-2 online softmax of the row (max and sum over the row's four
//      threads by shuffles), weights to LDS;
//   3. O[r][D/4 dims of quarter c] += P[r][:] . V_tile (accumulators in
//      registers, rescaled when the row's max moves).
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;
constexpr int kQB = 16;     // query positions per workgroup
constexpr int kHW = 4;      // heads per workgroup
constexpr int kRows = kQB * kHW;
constexpr int kBN = 32;     // keys per tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kg, const float* __restrict__ vg,
    float* __restrict__ out, const int32_t* __restrict__ kv_lens, int H, int K, int S, int S_kv,
    int S_max, int head_chunks, float scale_log2) {
  constexpr int DQ = D / 4;       // dims per thread in phase 3
  constexpr int ROW = D + 4;      // padded LDS row (a 16-byte shift per row)
  constexpr int LOADS = kBN * D / 4 / kThreads;  // float4 per thread per tensor and tile

  __shared__ __attribute__((aligned(16))) float qs[kRows][ROW];
  __shared__ __attribute__((aligned(16))) float ks[kBN][ROW];
  __shared__ __attribute__((aligned(16))) float vs[kBN][D];
  __shared__ __attribute__((aligned(16))) float ps[kRows][kBN + 4];

  const int qb = blockIdx.x;
  const int k = blockIdx.y / head_chunks;
  const int hc = blockIdx.y - k * head_chunks;
  const int b = blockIdx.z;
  const int G = H / K;
  const int tid = threadIdx.x;
  const int r = tid >> 2;      // this thread's row: head r / 16, position r % 16
  const int c = tid & 3;       // quarter
  const int hl = hc * kHW + r / kQB;
  const bool hok = hl < G;
  const int pos = qb * kQB + r % kQB;  // query index within the S queries

  const int L = kv_lens ? kv_lens[b] : S_kv;
  const int q_off = CAUSAL ? L - S : 0;  // absolute position of query 0
  const int lim = pos < S ? (CAUSAL ? min(q_off + pos + 1, L) : L) : 0;  // keys [0, lim) visible
  // keys the workgroup needs
  const int kend = CAUSAL ? min(q_off + min(qb * kQB + kQB, S), L) : L;

  // stage the 64 query rows (zeros for rows past S or past the group)
  for (int i = tid; i < kRows * (D / 4); i += kThreads) {
    const int rr = i / (D / 4), c4 = i - rr * (D / 4);
    const int h2 = hc * kHW + rr / kQB, p2 = qb * kQB + rr % kQB;
    float4 v4 = float4{0.f, 0.f, 0.f, 0.f};
    if (h2 < G && p2 < S)
      v4 = reinterpret_cast<const float4*>(q + (((size_t)b * H + (size_t)k * G + h2) * S + p2) * D)[c4];
    *reinterpret_cast<float4*>(&qs[rr][4 * c4]) = v4;
  }

  const size_t kv_base = ((size_t)b * K + k) * (size_t)S_max * D;
  float acc[DQ];
#pragma unroll
  for (int j = 0; j < DQ; ++j) acc[j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // the row's state (replicated over its 4 threads)

  for (int kb0 = 0; kb0 < kend; kb0 += kBN) {
    __syncthreads();  // the previous tile is consumed (and the query rows staged)
    {
      float4 kv4[LOADS], vv4[LOADS];
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int i = tid + u * kThreads;
        const int row = i / (D / 4), c4 = i - row * (D / 4);
        const bool ok = kb0 + row < kend;
        const size_t off = kv_base + (size_t)(kb0 + row) * D;
        kv4[u] = ok ? reinterpret_cast<const float4*>(kg + off)[c4] : float4{0.f, 0.f, 0.f, 0.f};
        vv4[u] = ok ? reinterpret_cast<const float4*>(vg + off)[c4] : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < LOADS; ++u) {
        const int i = tid + u * kThreads;
        const int row = i / (D / 4), c4 = i - row * (D / 4);
        *reinterpret_cast<float4*>(&ks[row][4 * c4]) = kv4[u];
        *reinterpret_cast<float4*>(&vs[row][4 * c4]) = vv4[u];
      }
    }
    __syncthreads();
    // 1. scores of row r against keys 8c .. 8c + 7 (log2 units)
    float s[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) s[jj] = 0.f;
#pragma unroll 4
    for (int d4 = 0; d4 < D / 4; ++d4) {
      const float4 qv = *reinterpret_cast<const float4*>(&qs[r][4 * d4]);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float4 kv = *reinterpret_cast<const float4*>(&ks[8 * c + jj][4 * d4]);
        s[jj] = fmaf(qv.x, kv.x, s[jj]);
        s[jj] = fmaf(qv.y, kv.y, s[jj]);
        s[jj] = fmaf(qv.z, kv.z, s[jj]);
        s[jj] = fmaf(qv.w, kv.w, s[jj]);
      }
    }
    // 2. online softmax over the row's four threads
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const bool vis = kb0 + 8 * c + jj < lim;
      s[jj] = vis ? s[jj] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[jj]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    const float m_new = fmaxf(m_run, mx);
    // a row with no visible key so far keeps zero weights
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - mref);  // 0 while m_run = -inf
    float sum = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const float e = fast_exp2(s[jj] - mref);
      ps[r][8 * c + jj] = e;
      sum += e;
    }
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    l_run = l_run * alpha + sum;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < DQ; ++j) acc[j] *= alpha;
    __syncthreads();  // the row's weights are in LDS for its four threads
    // 3. O[r][c DQ .. c DQ + DQ) += P[r][:] . V_tile
#pragma unroll 4
    for (int j = 0; j < kBN; ++j) {
      const float p = ps[r][j];
#pragma unroll
      for (int e4 = 0; e4 < DQ / 4; ++e4) {
        const float4 v4 = *reinterpret_cast<const float4*>(&vs[j][c * DQ + 4 * e4]);
        acc[4 * e4 + 0] = fmaf(p, v4.x, acc[4 * e4 + 0]);
        acc[4 * e4 + 1] = fmaf(p, v4.y, acc[4 * e4 + 1]);
        acc[4 * e4 + 2] = fmaf(p, v4.z, acc[4 * e4 + 2]);
        acc[4 * e4 + 3] = fmaf(p, v4.w, acc[4 * e4 + 3]);
      }
    }
  }

  if (hok && pos < S) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;  // no visible key: zero row
    float* orow = out + (((size_t)b * H + (size_t)k * G + hl) * S + pos) * D + c * DQ;
#pragma unroll
    for (int e4 = 0; e4 < DQ / 4; ++e4)
      reinterpret_cast<float4*>(orow)[e4] =
          float4{acc[4 * e4] * inv, acc[4 * e4 + 1] * inv, acc[4 * e4 + 2] * inv, acc[4 * e4 + 3] * inv};
  }
}

}  // namespace

hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* out,
                              const int32_t* kv_lens, int B, int H, int K, int S, int S_kv, int S_max,
                              int d, float scale_log2, bool causal, hipStream_t stream) {
  const int G = H / K;
  const int head_chunks = (G + kHW - 1) / kHW;
  const dim3 grid((S + kQB - 1) / kQB, K * head_chunks, B);
  const dim3 block(kThreads);
  auto qp = static_cast<const float*>(q);
  auto kp = static_cast<const float*>(k);
  auto vp = static_cast<const float*>(v);
  auto op = static_cast<float*>(out);
#define GQA_PF32(DD, CA)                                                                         \
  hipLaunchKernelGGL((prefill_f32_kernel<DD, CA>), grid, block, 0, stream, qp, kp, vp, op,       \
                     kv_lens, H, K, S, S_kv, S_max, head_chunks, scale_log2)
  if (d == 128) {
    if (causal) GQA_PF32(128, true); else GQA_PF32(128, false);
  } else {
    if (causal) GQA_PF32(64, true); else GQA_PF32(64, false);
  }
#undef GQA_PF32
  return hipGetLastError();
}

}  // namespace gqa
