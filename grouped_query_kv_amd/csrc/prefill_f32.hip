// GQA prefill family for fp32 inputs on the gfx950 matrix cores in fp32
// (v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulation; fp32 softmax
// weights): causal prefill, prefill of a chunk over a cache, non-causal
// cross-attention -- the same masks, layouts and work decomposition as the
// bf16 kernel (prefill_bf16.hip):
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
// One 256-thread workgroup per (sequence b, KV head k, span of query
// positions, chunk of heads of the group): each of the 4 wavefronts owns two
// (head, 16 positions) row tiles, 8 heads x 16 positions (or, for groups of
// fewer than 8 heads, G rounded up to a power of two heads x more position
// blocks), all reading the same K/V tiles.  The key loop walks 32-key tiles
// of [0, q0 + span), copied from global memory straight into LDS
// (global_load_lds_dwordx4), double-buffered, one barrier per tile; blocks
// are issued last-position-first and renumbered so that all blocks of one
// (sequence, KV head) run on one XCD (xcd_order.h), as in the bf16 kernel.
// Per tile and row tile:
//   S^T[32 x 16] = K_tile . Q^T   (two 16-key tiles, D/4 products each; one
//                                   16-byte LDS read of a K row feeds four
//                                   products: lane (n, g)'s contraction slot of
//                                   product (j, c) is dimension 16j + 4g + c)
//   mask on the diagonal (or last) tile, lazy base-2 online softmax in fp32
//   O[16 x D] += P . V_tile       (P straight from the score layout: lane
//                                   (n = query row, g) holds keys 16mt + 4g + i,
//                                   its contraction slot of product (mt, i);
//                                   V[16mt + 4g + i][16t + n] is one 4-byte
//                                   LDS read feeding both row tiles)
// LDS rows are whole rows of D floats with 16-byte chunks XOR-swizzled by
// row -- K: chunk ^ (row % 16), V: chunk ^ 4 ((row / 4) % 4) -- which makes
// both reads conflict-free (the layout of the fp32 decode pass).
#include <type_traits>

#include "common.h"
#include "gqa_internal.h"
#include "xcd_order.h"

namespace gqa {
namespace {

constexpr int kBN = 32;      // keys per tile
constexpr int kBQ = 16;      // query positions per row tile
constexpr int kHeadsWG = 8;  // row tiles per workgroup (heads of the group per workgroup)

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kg, const float* __restrict__ vg,
    float* __restrict__ out, const int32_t* __restrict__ kv_lens, int H, int K, int S, int S_kv,
    int S_max, int head_chunks, int hpw_log2, float scale_log2) {
  constexpr int CPR = D / 4;                  // 16-byte chunks per row
  constexpr int DJ = D / 16;                  // float4 query pieces per lane
  constexpr int DT = D / 16;                  // 16-dim output tiles
  constexpr int TILE = kBN * D;               // floats per staged tile
  constexpr int COPIES = TILE / 256 / 4;      // 1 KB copies per wave per tile and tensor

  // two stages of the K and V tiles as four distinct LDS objects, so the
  // compiler can tell that reads of one stage never touch the stage the
  // asynchronous copies are filling
  __shared__ __attribute__((aligned(16))) float k_lds0[TILE];
  __shared__ __attribute__((aligned(16))) float k_lds1[TILE];
  __shared__ __attribute__((aligned(16))) float v_lds0[TILE];
  __shared__ __attribute__((aligned(16))) float v_lds1[TILE];

  // the 8 row tiles of a workgroup: hpw heads x (8 / hpw) blocks of 16 positions
  const int hpw = 1 << hpw_log2;
  const int qspan = kBQ * (kHeadsWG >> hpw_log2);  // query positions per workgroup
  const int nqb = (S + qspan - 1) / qspan;
  const int nbx = gridDim.x, nby = gridDim.y;
  const int wid = (int)blockIdx.x + nbx * ((int)blockIdx.y + nby * (int)blockIdx.z);
  const int lid = xcd_block_id(wid, nbx * nby * (int)gridDim.z);
  const int bx = lid % nbx, byz = lid / nbx;
  const int by = byz % nby;
  const int qb = nqb - 1 - bx;
  const int q0 = qb * qspan;
  const int k = by / head_chunks;
  const int hc = by - k * head_chunks;
  const int b = byz / nby;
  const int G = H / K;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;

  const int L = kv_lens ? kv_lens[b] : S_kv;  // keys of this sequence
  const int q_off = CAUSAL ? L - S : 0;        // absolute position of query 0
  // Row tile j of this wave: head hglob[j], positions rq0[j] .. +15; this
  // lane's score column is position rq0[j] + n, which sees keys [0, lim[j]).
  int hglob[2], rq0[2], lim[2];
  bool hok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 2 * wave + j;
    const int hl = hc * hpw + (r & (hpw - 1));
    hok[j] = hl < G;
    hglob[j] = k * G + (hok[j] ? hl : 0);
    rq0[j] = q0 + kBQ * (r >> hpw_log2);
    lim[j] = CAUSAL ? min(q_off + rq0[j] + n + 1, L) : L;
  }
  const int kend = CAUSAL ? min(q_off + q0 + qspan, L) : L;
  const int mask_from = CAUSAL ? min(q_off + q0 + 1, L) : L;
  // queries as float4 pieces 16j + 4g .. +3 of row rq0 + n (zeros past S or the group)
  f32x4 qf[2][DJ];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int pos_n = rq0[j] + n;
    const bool ld = hok[j] && pos_n < S;
    const float* qrow = q + (((size_t)b * H + hglob[j]) * S + (ld ? pos_n : 0)) * D;
#pragma unroll
    for (int jj = 0; jj < DJ; ++jj)
      qf[j][jj] = ld ? *reinterpret_cast<const f32x4*>(qrow + 16 * jj + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // acc[j][t]: O rows 4g+i, dims 16t+n of row tile j; l_run: this lane's
  // share of row n's denominator
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
  const float* kbase = kg + kv_base;
  const float* vbase = vg + kv_base;
  const int ntiles = kend > 0 ? (kend + kBN - 1) / kBN : 0;
  const bool any_head = hok[0];

  // Copy r of this wave is instruction i = wave + 4r of a tile: lane l fills
  // LDS chunk 64 i + l = row (64 i + l) / CPR, physical chunk l % CPR, with
  // the logical chunk the swizzle puts there.  Rows past the last key are
  // fetched from the last key instead (finite values; masked).
  int crow[COPIES], koff[COPIES], voff[COPIES];
#pragma unroll
  for (int r = 0; r < COPIES; ++r) {
    const int c = 64 * (wave + 4 * r) + lane;
    const int row = c / CPR, cp = c - row * CPR;
    crow[r] = row;
    koff[r] = 4 * (cp ^ (row & 15));
    voff[r] = 4 * (cp ^ (((row >> 2) & 3) << 2));
  }
  auto copy_tile = [&](int kb0, auto stage_c) {
    constexpr int ST = decltype(stage_c)::value;
#pragma unroll
    for (int r = 0; r < COPIES; ++r) {
      const int row = min(kb0 + crow[r], kend - 1);
      const char* kp = reinterpret_cast<const char*>(kbase + (size_t)row * D + koff[r]);
      const char* vp = reinterpret_cast<const char*>(vbase + (size_t)row * D + voff[r]);
      __builtin_amdgcn_global_load_lds(kp, (__attribute__((address_space(3))) void*)((ST == 0 ? k_lds0 : k_lds1) + (wave + 4 * r) * 256), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vp, (__attribute__((address_space(3))) void*)((ST == 0 ? v_lds0 : v_lds1) + (wave + 4 * r) * 256), 16, 0, 0);
    }
  };

  // loop-invariant LDS offsets (floats): K piece jj of key tile mt is row
  // 16mt + n, logical chunk 4jj + g; V read of product (mt, i), tile t is
  // row 16mt + 4g + i, logical chunk 4t + n/4, float n % 4
  int ka_off[DJ], vb_off[DT];
#pragma unroll
  for (int jj = 0; jj < DJ; ++jj) ka_off[jj] = n * D + 4 * ((4 * jj + g) ^ n);
#pragma unroll
  for (int t = 0; t < DT; ++t) vb_off[t] = 4 * g * D + 4 * ((4 * t + (n >> 2)) ^ (g << 2)) + (n & 3);
  // lazy rescaling, as in the bf16 kernel: a row's max moves only when a
  // tile exceeds it by more than 2^kLazy
  constexpr float kLazy = 8.f;

  auto tile = [&](int kb0, auto stage_c) {
    constexpr int ST = decltype(stage_c)::value;
    const float* kt = ST == 0 ? k_lds0 : k_lds1;
    const float* vt = ST == 0 ? v_lds0 : v_lds1;
    // ---- S^T = K_tile . Q^T for both row tiles (raw q.k) ----
    f32x4 st[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) st[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < DJ; ++jj)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&kt[16 * mt * D + ka_off[jj]]);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            st[j][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c], qf[j][jj][c], st[j][mt], 0, 0, 0);
      }
    if (kb0 + kBN > mask_from) {  // diagonal / last tile: drop keys >= the row's limit
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kb0 + 16 * mt + 4 * g + i >= lim[j]) st[j][mt][i] = -INFINITY;
    }
    // ---- online softmax per row tile ----
    float p[2][2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float lmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, st[j][mt][i]);
      if (__any(lmax * scale_log2 > m_run[j] + kLazy)) {  // scale > 0
        float cmax = fmaxf(lmax, __shfl_xor(lmax, 16));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
        const float m_new = fmaxf(m_run[j], cmax * scale_log2);
        const float alpha = fast_exp2(m_run[j] - m_new);
        m_run[j] = m_new;
        l_run[j] *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = __shfl(alpha, 4 * g + i);
#pragma unroll
          for (int t = 0; t < DT; ++t) acc[j][t][i] *= a;
        }
      }
      // a row that has seen no visible key yet keeps all weights at zero
      const float mneg = m_run[j] == -INFINITY ? 0.f : -m_run[j];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[j][mt][i] = fast_exp2(fmaf(st[j][mt][i], scale_log2, mneg));
          l_run[j] += p[j][mt][i];
        }
    }
    // ---- O += P . V_tile ----
#pragma unroll
    for (int t = 0; t < DT; ++t)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = vt[vb_off[t] + (16 * mt + i) * D];
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[j][mt][i], v, acc[j][t], 0, 0, 0);
        }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  if (ntiles > 0) copy_tile(0, S0{});
  // tiles alternate between the two LDS stages; the loop is unrolled by two
  // so each stage's addresses are compile-time offsets
  for (int j = 0; j < ntiles; j += 2) {
    const int kb0 = j * kBN;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's copies of tile j landed
    __syncthreads();                     // tile j staged; tile j-1 fully consumed
    if (j + 1 < ntiles) copy_tile(kb0 + kBN, S1{});  // next tile streams during this one
    if (any_head) tile(kb0, S0{});
    if (j + 1 >= ntiles) break;
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if (j + 2 < ntiles) copy_tile(kb0 + 2 * kBN, S0{});
    if (any_head) tile(kb0 + kBN, S1{});
  }

  // ---- normalise and store rows 4g+i of each row tile ----
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float l = l_run[j] + __shfl_xor(l_run[j], 16);
    l += __shfl_xor(l, 32);  // row n's denominator, in every lane of row n
    if (!hok[j]) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lr = __shfl(l, 4 * g + i);
      const int pos = rq0[j] + 4 * g + i;
      if (pos >= S) continue;
      const float inv = lr > 0.f ? 1.f / lr : 0.f;  // no visible key: zero row
      float* orow = out + (((size_t)b * H + hglob[j]) * S + pos) * D;
#pragma unroll
      for (int t = 0; t < DT; ++t) orow[16 * t + n] = acc[j][t][i] * inv;
    }
  }
}

}  // namespace

hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* out,
                              const int32_t* kv_lens, int B, int H, int K, int S, int S_kv, int S_max,
                              int d, float scale_log2, bool causal, hipStream_t stream) {
  const int G = H / K;
  // heads per workgroup: the group's heads rounded up to a power of two (at
  // most 8); the remaining row tiles take further blocks of positions
  int hpw_log2 = 0;
  while ((1 << hpw_log2) < G && (1 << hpw_log2) < kHeadsWG) ++hpw_log2;
  const int head_chunks = (G + (1 << hpw_log2) - 1) >> hpw_log2;
  const int qspan = kBQ * (kHeadsWG >> hpw_log2);
  const dim3 grid((S + qspan - 1) / qspan, K * head_chunks, B);
  const dim3 block(256);
  auto qp = static_cast<const float*>(q);
  auto kp = static_cast<const float*>(k);
  auto vp = static_cast<const float*>(v);
  auto op = static_cast<float*>(out);
#define GQA_PF32(DD, CA)                                                                         \
  hipLaunchKernelGGL((prefill_f32_kernel<DD, CA>), grid, block, 0, stream, qp, kp, vp, op,       \
                     kv_lens, H, K, S, S_kv, S_max, head_chunks, hpw_log2, scale_log2)
  if (d == 128) {
    if (causal) GQA_PF32(128, true); else GQA_PF32(128, false);
  } else {
    if (causal) GQA_PF32(64, true); else GQA_PF32(64, false);
  }
#undef GQA_PF32
  return hipGetLastError();
}

}  // namespace gqa
