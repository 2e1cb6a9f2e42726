// Decode partition pass for fp32 caches, on the vector ALUs.
//
// Same contract as the bf16 pass (see decode_bf16.hip): for partition
// [t0, t1) of sequence b, KV head k and a block of up to 16 query heads of
// that group it produces the base-2 online-softmax state (m, l, acc) that the
// combine pass merges.  fp32 keeps full single precision end to end (the
// matrix cores would round operands), which is what fp32 callers ask for.
//
// One 256-thread workgroup per flat range (decode_flat.h) and up to eight
// 16-head blocks of the group; positions are processed in chunks of CF (64
// for d = 64, 32 for d = 128):
//   0. the chunk's K and V rows are copied into LDS with every load of the
//      chunk in flight at once (one memory round trip per chunk);
//   then for each head block of the workgroup (the chunk stays in LDS):
//   1. scores: thread (t, hs) dots position t's K row with its heads
//      (query rows broadcast from LDS);
//   2. softmax: wave w updates (m, l) of heads w, w+4, w+8, w+12 with
//      wavefront max/sum reductions, leaving probabilities in LDS;
//   3. values: thread (dim c, head slice) accumulates p * V[t][c] for its
//      heads.
// The group's K and V rows are read from memory once per workgroup and
// serve every head of the group (pinghaoyang.com.cn "GQA 完全拆解", section
// 工程实现: the group's KV block is loaded once for all its query heads);
// only groups of more than 128 heads take several workgroups per range.
// With more than one head block the block's query rows are re-staged from
// the (cache-resident) queries for every chunk.
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

// 16-byte streaming load of four floats (non-temporal: read once per step)
__device__ __forceinline__ float4 ld_f4_stream(const float* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return float4{v[0], v[1], v[2], v[3]};
}

constexpr int kThreads = 256;
constexpr int kHB = 16;       // heads per block
constexpr int kMaxHB = 8;     // head blocks per workgroup

// APPEND: fused cache append, as in decode_bf16.hip.
template <int D, bool APPEND>
__global__ __launch_bounds__(kThreads) void decode_split_f32_kernel(
    const float* __restrict__ q, float* __restrict__ kc, float* __restrict__ vc,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_acc,
    float* __restrict__ part_ml, int B, int H, int K, int S_max, FlatArgs fa, int wg_per_range,
    float scale_log2, const float* __restrict__ k_new, const float* __restrict__ v_new,
    int32_t* __restrict__ meta) {
  constexpr int CF = D == 64 ? 64 : 32;                  // positions per chunk
  constexpr int HEADS_PER_THREAD = kHB * D / kThreads;   // phase 3: 8 (D=128) or 4 (D=64)
  constexpr int HPT1 = kHB * CF / kThreads;              // phase 1: 2 (D=128) or 4 (D=64)
  constexpr int KROW = D + 4;  // padded K row: a 16-byte shift per row spreads the
                               // phase-1 reads of consecutive rows over the banks
  constexpr int ROW4 = D / 4;  // float4 per row
  constexpr int LOADS = CF * ROW4 / kThreads;            // float4 per thread per tensor

  __shared__ __attribute__((aligned(16))) float qs[kHB][D];
  __shared__ __attribute__((aligned(16))) float ks[CF][KROW];
  __shared__ __attribute__((aligned(16))) float vs[CF][D];
  __shared__ __attribute__((aligned(16))) float ps[kHB][CF];
  __shared__ float alpha_s[kHB];
  __shared__ float m_s[kMaxHB][kHB];
  __shared__ float l_s[kMaxHB][kHB];

  const int w = blockIdx.x / wg_per_range;
  const int hg = blockIdx.x - w * wg_per_range;  // this workgroup's group of head blocks
  const int G = H / K;
  const int hb0 = hg * kMaxHB;
  const int nhb = min(kMaxHB, (G + kHB - 1) / kHB - hb0);  // head blocks of this workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // lengths clamped into [0, S_max], so no length can make a load leave the cache
  auto len_in = [&](int bb) -> int { return min(max(seq_lens[bb], 0), S_max); };
  auto len_of = [&](int bb) -> int {
    const int L_in = len_in(bb);
    return min(APPEND && L_in < S_max ? L_in + 1 : L_in, fa.max_len);
  };
  // the lengths attended over and the split, for the combine pass
  if (blockIdx.x == 0 && wave == 0) flat_publish(B, K, len_of, meta);
  const int total = flat_total(B, K, len_of);
  const int R = flat_range(total, fa);

  flat_for_each_segment(w, B, K, total, R, len_of,
                        [&](int b, int k, int t0, int t1, int L, int slot) {
  const int newpos = APPEND && L > len_in(b) ? L - 1 : -1;  // the appended row, if any
  const size_t grow0 = (size_t)b * H + (size_t)k * G;         // the group's first query row

  // query rows of head block hb (zeros past the group)
  auto stage_q = [&](int hb) {
    const int nh = min(kHB, G - hb * kHB);
    for (int i = tid; i < kHB * D; i += kThreads) {
      const int h = i / D, c = i - h * D;
      qs[h][c] = h < nh ? q[(grow0 + hb * kHB + h) * D + c] : 0.f;
    }
  };
  if (nhb == 1) stage_q(hb0);
  if (tid < kMaxHB * kHB) {
    m_s[tid / kHB][tid % kHB] = -INFINITY;
    l_s[tid / kHB][tid % kHB] = 0.f;
  }
  const size_t head_base = ((size_t)b * K + k) * (size_t)S_max * D;
  float* kbase = kc + head_base;
  float* vbase = vc + head_base;
  const float* knew_row = APPEND ? k_new + ((size_t)b * K + k) * D : nullptr;
  const float* vnew_row = APPEND ? v_new + ((size_t)b * K + k) * D : nullptr;

  const int c_own = tid % D;            // value dimension owned in phase 3
  const int slice = tid / D;            // head slice owned in phase 3
  float acc[kMaxHB][HEADS_PER_THREAD];
#pragma unroll
  for (int u = 0; u < kMaxHB; ++u)
#pragma unroll
    for (int j = 0; j < HEADS_PER_THREAD; ++j) acc[u][j] = 0.f;

  for (int c0 = t0; c0 < t1; c0 += CF) {
    const int n_tok = min(CF, t1 - c0);
    // 0. stage the chunk's K and V rows (rows past the segment: zeros)
    {
      float4 kv4[LOADS], vv4[LOADS];
#pragma unroll
      for (int r = 0; r < LOADS; ++r) {
        const int i = tid + r * kThreads;
        const int row = i / ROW4, c4 = i - row * ROW4;
        const int tok = c0 + row;
        const bool ok = row < n_tok;
        const float* kr = APPEND && tok == newpos ? knew_row : kbase + (size_t)tok * D;
        const float* vr = APPEND && tok == newpos ? vnew_row : vbase + (size_t)tok * D;
        // streaming loads: every cache byte is read once per step
        kv4[r] = ok ? ld_f4_stream(kr + 4 * c4) : float4{0.f, 0.f, 0.f, 0.f};
        vv4[r] = ok ? ld_f4_stream(vr + 4 * c4) : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int r = 0; r < LOADS; ++r) {
        const int i = tid + r * kThreads;
        const int row = i / ROW4, c4 = i - row * ROW4;
        *reinterpret_cast<float4*>(&ks[row][4 * c4]) = kv4[r];
        *reinterpret_cast<float4*>(&vs[row][4 * c4]) = vv4[r];
      }
    }
#pragma unroll
    for (int u = 0; u < kMaxHB; ++u) {
      if (u >= nhb) break;  // uniform
      if (nhb > 1) {
        __syncthreads();  // the previous head block is done with qs and ps
        stage_q(hb0 + u);
      }
      __syncthreads();
      // 1. scores
      {
        const int t = tid % CF;
        const int hs = tid / CF;  // heads hs, hs + 256/CF, ...
        float s[HPT1];
#pragma unroll
        for (int r = 0; r < HPT1; ++r) s[r] = 0.f;
#pragma unroll 8
        for (int c4 = 0; c4 < ROW4; ++c4) {
          const float4 kv = *reinterpret_cast<const float4*>(&ks[t][4 * c4]);
#pragma unroll
          for (int r = 0; r < HPT1; ++r) {
            const float* qq = &qs[hs + (kThreads / CF) * r][4 * c4];
            s[r] = fmaf(kv.x, qq[0], s[r]);
            s[r] = fmaf(kv.y, qq[1], s[r]);
            s[r] = fmaf(kv.z, qq[2], s[r]);
            s[r] = fmaf(kv.w, qq[3], s[r]);
          }
        }
#pragma unroll
        for (int r = 0; r < HPT1; ++r)
          ps[hs + (kThreads / CF) * r][t] = t < n_tok ? s[r] * scale_log2 : -INFINITY;
      }
      __syncthreads();
      // 2. online softmax, wave w owns heads w, w+4, w+8, w+12 (lane = position);
      // the four heads' reductions are interleaved (independent shuffle chains)
      {
        float x[4], mx[4], mnew[4], e[4], sum[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = lane < CF ? ps[wave + 4 * r][lane] : -INFINITY;
          mx[r] = x[r];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx[r] = fmaxf(mx[r], __shfl_xor(mx[r], off));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mnew[r] = fmaxf(m_s[u][wave + 4 * r], mx[r]);
          e[r] = fast_exp2(x[r] - mnew[r]);
          sum[r] = e[r];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
#pragma unroll
          for (int r = 0; r < 4; ++r) sum[r] += __shfl_xor(sum[r], off);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (lane < CF) ps[wave + 4 * r][lane] = e[r];
        if (lane == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int h = wave + 4 * r;
            const float a = fast_exp2(m_s[u][h] - mnew[r]);
            alpha_s[h] = a;
            l_s[u][h] = l_s[u][h] * a + sum[r];
            m_s[u][h] = mnew[r];
          }
        }
      }
      __syncthreads();
      // 3. values
#pragma unroll
      for (int j = 0; j < HEADS_PER_THREAD; ++j) acc[u][j] *= alpha_s[slice * HEADS_PER_THREAD + j];
      // eight positions per step, their LDS reads issued together
      int t = 0;
      for (; t + 8 <= n_tok; t += 8) {
        float v[8];
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) v[e8] = vs[t + e8][c_own];
#pragma unroll
        for (int j = 0; j < HEADS_PER_THREAD; ++j) {
          const float4 pa = *reinterpret_cast<const float4*>(&ps[slice * HEADS_PER_THREAD + j][t]);
          const float4 pb = *reinterpret_cast<const float4*>(&ps[slice * HEADS_PER_THREAD + j][t + 4]);
          acc[u][j] = fmaf(pa.x, v[0], acc[u][j]);
          acc[u][j] = fmaf(pa.y, v[1], acc[u][j]);
          acc[u][j] = fmaf(pa.z, v[2], acc[u][j]);
          acc[u][j] = fmaf(pa.w, v[3], acc[u][j]);
          acc[u][j] = fmaf(pb.x, v[4], acc[u][j]);
          acc[u][j] = fmaf(pb.y, v[5], acc[u][j]);
          acc[u][j] = fmaf(pb.z, v[6], acc[u][j]);
          acc[u][j] = fmaf(pb.w, v[7], acc[u][j]);
        }
      }
      for (; t < n_tok; ++t) {
        const float v = vs[t][c_own];
#pragma unroll
        for (int j = 0; j < HEADS_PER_THREAD; ++j)
          acc[u][j] = fmaf(ps[slice * HEADS_PER_THREAD + j][t], v, acc[u][j]);
      }
    }
    __syncthreads();  // every thread is done with ks, vs, ps before the next chunk
  }

  if (APPEND && hg == 0 && newpos >= t0 && newpos < t1 && tid < D) {
    // the appended rows join the cache
    kbase[(size_t)newpos * D + tid] = knew_row[tid];
    vbase[(size_t)newpos * D + tid] = vnew_row[tid];
  }
#pragma unroll
  for (int u = 0; u < kMaxHB; ++u) {
    if (u >= nhb) break;
    const int hb = hb0 + u;
    const int nh = min(kHB, G - hb * kHB);
    const size_t row0 = (size_t)slot * G + (size_t)hb * kHB;
#pragma unroll
    for (int j = 0; j < HEADS_PER_THREAD; ++j) {
      const int h = slice * HEADS_PER_THREAD + j;
      if (h < nh) part_acc[(row0 + h) * D + c_own] = acc[u][j];
    }
    if (tid < nh) {
      float* ml = part_ml + (row0 + tid) * 2;
      ml[0] = m_s[u][tid];
      ml[1] = l_s[u][tid];
    }
  }
  __syncthreads();  // m_s, l_s and qs are re-initialised by the next segment
                        });
}

}  // namespace

hipError_t launch_decode_split_f32(const void* q, void* k_cache, void* v_cache,
                                   const int32_t* seq_lens, const DecodeWorkspace& ws,
                                   const DecodePlan& plan, int B, int H, int K, int S_max, int d,
                                   float scale_log2, const void* k_new, const void* v_new,
                                   hipStream_t stream) {
  const int wg_per_range = (plan.head_blocks + kMaxHB - 1) / kMaxHB;
  const dim3 grid(plan.fa.n_wg * wg_per_range);
  const dim3 block(kThreads);
  auto qp = static_cast<const float*>(q);
  auto kp = static_cast<float*>(k_cache);
  auto vp = static_cast<float*>(v_cache);
  auto kn = static_cast<const float*>(k_new);
  auto vn = static_cast<const float*>(v_new);
  const bool app = k_new != nullptr;
#define GQA_SPLIT(DD, AP)                                                                         \
  hipLaunchKernelGGL((decode_split_f32_kernel<DD, AP>), grid, block, 0, stream, qp, kp, vp,       \
                     seq_lens, ws.part_acc, ws.part_ml, B, H, K, S_max, plan.fa, wg_per_range,     \
                     scale_log2, kn, vn, ws.meta)
  if (d == 128) {
    if (app) GQA_SPLIT(128, true); else GQA_SPLIT(128, false);
  } else {
    if (app) GQA_SPLIT(64, true); else GQA_SPLIT(64, false);
  }
#undef GQA_SPLIT
  return hipGetLastError();
}

}  // namespace gqa
