// Causal GQA prefill on the gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// out[b,h,i,:] = sum_{j<=i} softmax_j(scale q[b,h,i,:] . k[b,h/G,j,:]) v[b,h/G,j,:]
//
// pinghaoyang.com.cn "GQA 完全拆解": section 解码推理的内存账本 (prefill runs the
// whole prefix in parallel; row i is what decode step i computes) and section
// 工程实现 (engineering: a group-aware kernel stages the group's shared K/V
// block in on-chip memory once and reuses it for every query head of the
// group).  compassingai.com "分組查詢注意力", 技術原理: heads regrouped [K, G].
//
// Work decomposition: one 256-thread workgroup per (sequence b, KV head k,
// block of 16 query positions, chunk of up to 8 heads of the group).  Each of
// the 4 wavefronts owns two (head, 16 positions) row tiles, so one workgroup
// covers 8 heads x 16 positions = 128 rows that all read the same K/V tiles.
// The key loop walks 64-key tiles of [0, q0 + 16), staged in LDS:
//   K tile [64][D]  row-major, 16-byte chunks XOR-swizzled by key,
//   V tile [D][64]  transposed while being written, with the keys of every
//                   32-key step permuted into the order the second product
//                   consumes them, 16-byte chunks XOR-swizzled by dimension.
// Per tile and row tile:  S^T[64 x 16] = K_tile . Q^T  (v_mfma_f32_16x16x32_bf16),
// causal mask on the diagonal tile, base-2 online softmax in fp32,
// O[16 x D] += P[16 x 64] . V_tile.  The score layout of the first product is
// used directly as the P operand of the second (see decode_bf16.hip for the
// operand layouts and the contraction-slot argument).
// Blocks are issued last-position-first so the longest causal rows start
// earliest.
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kBN = 64;      // keys per tile
constexpr int kBQ = 16;      // query positions per workgroup
constexpr int kHeadsWG = 8;  // heads of the group per workgroup

__device__ __forceinline__ int vt_slot(int key) {  // key in [0, 64)
  const int ks = key >> 5, kk = key & 31;
  return ks * 32 + ((kk & 15) >> 2) * 8 + ((kk >> 4) << 2) + (kk & 3);
}
__device__ __forceinline__ int vt_swz(int row) { return (row ^ (row >> 3)) & 7; }

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(256) void prefill_causal_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kg, const __bf16* __restrict__ vg,
    void* __restrict__ out, int H, int K, int S, int S_max, int head_chunks, float scale_log2) {
  constexpr int KSTEPS = D / 32;
  constexpr int DT = D / 16;
  constexpr int CPR = D / 8;  // 16-byte chunks per K row

  __shared__ __attribute__((aligned(16))) uint16_t ks[kBN * D];
  __shared__ __attribute__((aligned(16))) uint16_t vts[D * kBN];

  const int nqb = (S + kBQ - 1) / kBQ;
  const int qb = nqb - 1 - (int)blockIdx.x;
  const int q0 = qb * kBQ;
  const int k = blockIdx.y / head_chunks;
  const int hc = blockIdx.y - k * head_chunks;
  const int b = blockIdx.z;
  const int G = H / K;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;

  // the wave's two row tiles: heads hl0, hl0+1 of the group
  int hglob[2];
  bool hok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int hl = hc * kHeadsWG + 2 * wave + j;
    hok[j] = hl < G;
    hglob[j] = k * G + (hok[j] ? hl : 0);
  }
  const int pos_n = q0 + n;  // query position of this lane's score column
  bf16x8 qf[2][KSTEPS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool ld = hok[j] && pos_n < S;
    const __bf16* qrow = q + (((size_t)b * H + hglob[j]) * S + (ld ? pos_n : 0)) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[j][s] = as_bf16x8(ld ? ld16(qrow + 32 * s + 8 * g) : zero_u32x4());
  }

  f32x4 acc[2][DT];
  float m_run[2], l_run[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t kv_base = ((size_t)b * K + k) * (size_t)S_max * D;
  const __bf16* kbase = kg + kv_base;
  const __bf16* vbase = vg + kv_base;
  const int kend = min(q0 + kBQ, S);
  const bool any_head = hok[0];

  for (int kb0 = 0; kb0 < kend; kb0 += kBN) {
    __syncthreads();  // previous tile fully consumed
    // ---- stage K and V tiles ----
#pragma unroll
    for (int r = 0; r < kBN * CPR / 256; ++r) {
      const int c = tid + 256 * r;
      const int key = c / CPR, cc = c - key * CPR;
      const bool ld = kb0 + key < kend;
      const size_t off = (size_t)(kb0 + key) * D + cc * 8;
      const u32x4 kw = ld ? ld16(kbase + off) : zero_u32x4();
      const u32x4 vw = ld ? ld16(vbase + off) : zero_u32x4();
      *reinterpret_cast<u32x4*>(&ks[key * D + ((cc ^ (key & (CPR - 1))) * 8)]) = kw;
      const int slot = vt_slot(key);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = cc * 8 + e;
        const int phys = ((slot >> 3) ^ vt_swz(row)) * 8 + (slot & 7);
        vts[row * kBN + phys] = (uint16_t)(vw[e >> 1] >> (16 * (e & 1)));
      }
    }
    __syncthreads();
    if (!any_head) continue;

    // ---- S^T = K_tile . Q^T for both row tiles ----
    f32x4 st[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) st[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int key = 16 * mt + n;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int cc = 4 * s + g;
        const bf16x8 a =
            as_bf16x8(*reinterpret_cast<const u32x4*>(&ks[key * D + ((cc ^ (key & (CPR - 1))) * 8)]));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          st[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[j][s], st[j][mt], 0, 0, 0);
      }
    }

    // ---- online softmax per row tile ----
    const bool diag = kb0 + kBN > q0;  // tile may hold keys beyond some rows
    bf16x8 pa[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float sv[16];
      float cmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb0 + 16 * mt + 4 * g + i;
          float x = st[j][mt][i] * scale_log2;
          if (diag && key > pos_n) x = -INFINITY;
          sv[4 * mt + i] = x;
          cmax = fmaxf(cmax, x);
        }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      const float m_new = fmaxf(m_run[j], cmax);
      const float alpha = fast_exp2(m_run[j] - m_new);
      float psum = 0.f;
      uint32_t pw[8];
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float e0 = fast_exp2(sv[e] - m_new);
        const float e1 = fast_exp2(sv[e + 1] - m_new);
        psum += e0 + e1;
        pw[e / 2] = pack_bf16x2(e0, e1);
      }
      psum += __shfl_xor(psum, 16);
      psum += __shfl_xor(psum, 32);
      l_run[j] = l_run[j] * alpha + psum;
      m_run[j] = m_new;
      // P operand of 32-key step ks: score tiles mt = 2ks, 2ks+1
      pa[j][0] = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
      pa[j][1] = as_bf16x8(u32x4{pw[4], pw[5], pw[6], pw[7]});
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = __shfl(alpha, 4 * g + i);
#pragma unroll
        for (int t = 0; t < DT; ++t) acc[j][t][i] *= a;
      }
    }

    // ---- O += P . V_tile ----
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const int row = 16 * t + n;
        const int phys = ((4 * kk + g) ^ vt_swz(row)) * 8;
        const bf16x8 vb = as_bf16x8(*reinterpret_cast<const u32x4*>(&vts[row * kBN + phys]));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[j][kk], vb, acc[j][t], 0, 0, 0);
      }
  }

  // ---- normalise and store rows 4g+i of each row tile ----
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (!hok[j]) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float l = __shfl(l_run[j], 4 * g + i);
      const int pos = q0 + 4 * g + i;
      if (pos >= S) continue;
      const float inv = 1.f / l;
      const size_t orow = (((size_t)b * H + hglob[j]) * S + pos) * D;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const float o = acc[j][t][i] * inv;
        if (OUT_BF16)
          static_cast<__bf16*>(out)[orow + 16 * t + n] = static_cast<__bf16>(o);
        else
          static_cast<float*>(out)[orow + 16 * t + n] = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill_causal_bf16(const void* q, const void* k, const void* v, void* out,
                                      int B, int H, int K, int S, int S_max, int d,
                                      float scale_log2, bool out_bf16, hipStream_t stream) {
  const int G = H / K;
  const int head_chunks = (G + kHeadsWG - 1) / kHeadsWG;
  const dim3 grid((S + kBQ - 1) / kBQ, K * head_chunks, B);
  const dim3 block(256);
  auto qp = static_cast<const __bf16*>(q);
  auto kp = static_cast<const __bf16*>(k);
  auto vp = static_cast<const __bf16*>(v);
#define GQA_PREFILL(DD, OB)                                                                     \
  hipLaunchKernelGGL((prefill_causal_kernel<DD, OB>), grid, block, 0, stream, qp, kp, vp, out, \
                     H, K, S, S_max, head_chunks, scale_log2)
  if (d == 128) {
    if (out_bf16) GQA_PREFILL(128, true); else GQA_PREFILL(128, false);
  } else {
    if (out_bf16) GQA_PREFILL(64, true); else GQA_PREFILL(64, false);
  }
#undef GQA_PREFILL
  return hipGetLastError();
}

}  // namespace gqa
