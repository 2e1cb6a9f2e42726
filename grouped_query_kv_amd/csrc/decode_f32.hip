// Decode partition pass for fp32 caches, on the vector ALUs.
//
// Same contract as the bf16 pass (see decode_bf16.hip): for partition
// [t0, t1) of sequence b, KV head k and a block of up to 16 query heads of
// that group it produces the base-2 online-softmax state (m, l, acc) that the
// combine pass merges.  fp32 keeps full single precision end to end (the
// matrix cores would round operands), which is what fp32 callers ask for.
//
// One 256-thread workgroup per (partition, KV head, head block, sequence);
// positions are processed in chunks of 64:
//   1. scores: thread (t, h0) dots position t's K row with heads h0, h0+4,
//      h0+8, h0+12 (query rows broadcast from LDS);
//   2. softmax: wave w updates (m, l) of heads w, w+4, w+8, w+12 with
//      wavefront max/sum reductions, leaving probabilities in LDS;
//   3. values: thread (dim c, head slice) accumulates p * V[t][c] for its
//      heads, reading each V row coalesced.
// The group's K and V rows are read from memory once per workgroup and
// serve every head of the block (pinghaoyang.com.cn "GQA 完全拆解", section
// 工程实现: the group's KV block is loaded once for all its query heads).
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunkF = 64;
constexpr int kHB = 16;  // heads per block

// APPEND: fused cache append, as in decode_bf16.hip.
template <int D, bool APPEND>
__global__ __launch_bounds__(kThreads) void decode_split_f32_kernel(
    const float* __restrict__ q, float* __restrict__ kc, float* __restrict__ vc,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_acc,
    float* __restrict__ part_ml, int H, int K, int S_max, int part_tokens, int parts,
    int head_blocks, float scale_log2, const float* __restrict__ k_new,
    const float* __restrict__ v_new, int32_t* __restrict__ lens_out) {
  constexpr int HEADS_PER_THREAD = kHB * D / kThreads;  // 8 (D=128) or 4 (D=64)

  __shared__ float qs[kHB][D];
  __shared__ float ps[kHB][kChunkF];
  __shared__ float alpha_s[kHB];
  __shared__ float m_s[kHB];
  __shared__ float l_s[kHB];

  const int p = blockIdx.x;
  const int k = blockIdx.y / head_blocks;
  const int hb = blockIdx.y - k * head_blocks;
  const int b = blockIdx.z;
  const int G = H / K;
  const int L_in = seq_lens[b];
  int L = L_in, newpos = -1;
  if (APPEND) {
    if (L_in < S_max) {
      newpos = L_in;
      L = L_in + 1;
    }
    if (p == 0 && blockIdx.y == 0 && threadIdx.x == 0) lens_out[b] = L;
  }
  const int pt_b = balanced_part_tokens(L, part_tokens);
  const int t0 = p * pt_b;
  if (t0 >= L) return;
  const int t1 = min(t0 + pt_b, L);
  const int nh = min(kHB, G - hb * kHB);  // real heads in this block

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const size_t hrow0 = (size_t)b * H + (size_t)k * G + (size_t)hb * kHB;

  for (int i = tid; i < kHB * D; i += kThreads) {
    const int h = i / D, c = i - h * D;
    qs[h][c] = h < nh ? q[(hrow0 + h) * D + c] : 0.f;
  }
  if (tid < kHB) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  const size_t head_base = ((size_t)b * K + k) * (size_t)S_max * D;
  float* kbase = kc + head_base;
  float* vbase = vc + head_base;
  const float* knew_row = APPEND ? k_new + ((size_t)b * K + k) * D : nullptr;
  const float* vnew_row = APPEND ? v_new + ((size_t)b * K + k) * D : nullptr;

  const int c_own = tid % D;            // value dimension owned in phase 3
  const int slice = tid / D;            // head slice owned in phase 3
  float acc[HEADS_PER_THREAD];
#pragma unroll
  for (int j = 0; j < HEADS_PER_THREAD; ++j) acc[j] = 0.f;
  __syncthreads();

  for (int c0 = t0; c0 < t1; c0 += kChunkF) {
    const int n_tok = min(kChunkF, t1 - c0);
    // 1. scores
    {
      const int t = tid & (kChunkF - 1);
      const int h0 = tid / kChunkF;  // 0..3
      float s[4] = {0.f, 0.f, 0.f, 0.f};
      if (t < n_tok) {
        const float* krow_p = APPEND && c0 + t == newpos ? knew_row : kbase + (size_t)(c0 + t) * D;
        const float4* krow = reinterpret_cast<const float4*>(krow_p);
#pragma unroll 4
        for (int c4 = 0; c4 < D / 4; ++c4) {
          const float4 kv = krow[c4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float* qq = &qs[h0 + 4 * r][4 * c4];
            s[r] = fmaf(kv.x, qq[0], s[r]);
            s[r] = fmaf(kv.y, qq[1], s[r]);
            s[r] = fmaf(kv.z, qq[2], s[r]);
            s[r] = fmaf(kv.w, qq[3], s[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
        ps[h0 + 4 * r][t] = t < n_tok ? s[r] * scale_log2 : -INFINITY;
    }
    __syncthreads();
    // 2. online softmax, wave w owns heads w, w+4, w+8, w+12
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = wave + 4 * r;
      const float x = ps[h][lane];
      float mx = x;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      const float m_old = m_s[h];
      const float m_new = fmaxf(m_old, mx);
      const float e = fast_exp2(x - m_new);
      float sum = e;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
      ps[h][lane] = e;
      if (lane == 0) {
        const float a = fast_exp2(m_old - m_new);
        alpha_s[h] = a;
        l_s[h] = l_s[h] * a + sum;
        m_s[h] = m_new;
      }
    }
    __syncthreads();
    // 3. values
#pragma unroll
    for (int j = 0; j < HEADS_PER_THREAD; ++j) acc[j] *= alpha_s[slice * HEADS_PER_THREAD + j];
    for (int t = 0; t < n_tok; ++t) {
      const float v = APPEND && c0 + t == newpos ? vnew_row[c_own] : vbase[(size_t)(c0 + t) * D + c_own];
#pragma unroll
      for (int j = 0; j < HEADS_PER_THREAD; ++j)
        acc[j] = fmaf(ps[slice * HEADS_PER_THREAD + j][t], v, acc[j]);
    }
    __syncthreads();
  }

  if (APPEND && hb == 0 && newpos >= t0 && newpos < t1 && tid < D) {
    // the appended rows join the cache
    kbase[(size_t)newpos * D + tid] = knew_row[tid];
    vbase[(size_t)newpos * D + tid] = vnew_row[tid];
  }
#pragma unroll
  for (int j = 0; j < HEADS_PER_THREAD; ++j) {
    const int h = slice * HEADS_PER_THREAD + j;
    if (h < nh) part_acc[((hrow0 + h) * parts + p) * D + c_own] = acc[j];
  }
  if (tid < nh) {
    float* ml = part_ml + ((hrow0 + tid) * parts + p) * 2;
    ml[0] = m_s[tid];
    ml[1] = l_s[tid];
  }
}

}  // namespace

hipError_t launch_decode_split_f32(const void* q, void* k_cache, void* v_cache,
                                   const int32_t* seq_lens, const DecodeWorkspace& ws,
                                   const DecodePlan& plan, int B, int H, int K, int S_max, int d,
                                   float scale_log2, const void* k_new, const void* v_new,
                                   hipStream_t stream) {
  const dim3 grid(plan.parts, K * plan.head_blocks, B);
  const dim3 block(kThreads);
  auto qp = static_cast<const float*>(q);
  auto kp = static_cast<float*>(k_cache);
  auto vp = static_cast<float*>(v_cache);
  auto kn = static_cast<const float*>(k_new);
  auto vn = static_cast<const float*>(v_new);
  const bool app = k_new != nullptr;
#define GQA_SPLIT(DD, AP)                                                                         \
  hipLaunchKernelGGL((decode_split_f32_kernel<DD, AP>), grid, block, 0, stream, qp, kp, vp,       \
                     seq_lens, ws.part_acc, ws.part_ml, H, K, S_max, plan.part_tokens, plan.parts, \
                     plan.head_blocks, scale_log2, kn, vn, ws.lens)
  if (d == 128) {
    if (app) GQA_SPLIT(128, true); else GQA_SPLIT(128, false);
  } else {
    if (app) GQA_SPLIT(64, true); else GQA_SPLIT(64, false);
  }
#undef GQA_SPLIT
  return hipGetLastError();
}

}  // namespace gqa
