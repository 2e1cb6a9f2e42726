// GQA prefill on the gfx950 matrix cores (bf16 in, fp32 accumulate): causal
// prefill, prefill of a chunk over a cache, and non-causal cross-attention.
//
// out[b,h,i,:] = sum_{j visible} softmax_j(scale q[b,h,i,:] . k[b,h/G,j,:]) v[b,h/G,j,:]
//
// With L_b keys in the cache (kv_lens[b], or S_kv for every sequence) and
// S query positions, key j is visible to query i iff j < L_b and, when
// causal, j <= L_b - S + i: the queries are the last S positions of the
// sequence (L_b = S is plain causal prefill; L_b > S is a chunk appended to
// a cache holding L_b - S earlier rows).  Non-causal: every j < L_b (GQA in
// cross-attention, pinghaoyang.com.cn "GQA 完全拆解", GQA section).  A query
// with no visible key gets a zero row.
//
// pinghaoyang.com.cn "GQA 完全拆解": section 解码推理的内存账本 (prefill runs the
// whole prefix in parallel; row i is what decode step i computes) and section
// 工程实现 (engineering: a group-aware kernel stages the group's shared K/V
// block in on-chip memory once and reuses it for every query head of the
// group).  compassingai.com "分組查詢注意力", 技術原理: heads regrouped [K, G].
//
// Work decomposition: one 256-thread workgroup per (sequence b, KV head k,
// span of query positions, chunk of heads of the group).  Each of the 4
// wavefronts owns two (head, 16 positions) row tiles, so one workgroup
// covers 128 rows that all read the same K/V tiles: 8 heads x 16 positions
// when the group has 8 or more heads, else hpw heads (G rounded up to a
// power of two) x 8/hpw blocks of 16 positions, so that small groups (G =
// 4 in Llama-3-8B, G = 1 in MHA) still fill every row tile.
// The key loop walks 64-key tiles of [0, q0 + 16), copied from global memory
// straight into LDS (global_load_lds_dwordx4: lane i of a wavefront lands
// its 16 bytes at LDS base + 16 i, with no register staging).  Rows are kept
// whole and their 16-byte chunks XOR-swizzled by row, which each lane
// realises by fetching the global chunk that belongs in its LDS slot; the
// swizzle makes the 16-byte and the transposed 8-byte reads conflict-free:
//   K tile [64][D]  read as the A operand of S^T = K . Q^T (ds_read_b128),
//   V tile [64][D]  read transposed as the B operand of O += P . V
//                   (ds_read_b64_tr_b16, see decode_bf16.hip for the layout).
// The tiles are double-buffered: the copies of tile j+1 are in flight while
// tile j is multiplied, and one barrier per tile orders the buffers.
// Per tile and row tile: S^T[64 x 16] = K_tile . Q^T (v_mfma_f32_16x16x32_bf16),
// mask only on the diagonal (or last) tile, base-2 online softmax in fp32 with
// lazy rescaling, O[16 x D] += P[16 x 64] . V_tile, where the score layout of
// the first product is used directly as the P operand of the second, and the
// softmax denominators come from the same product against a block of ones.
// Blocks are issued last-position-first so the longest causal rows start
// earliest, and renumbered so that all blocks of one (sequence, KV head) run
// on one XCD: gfx950 deals workgroups to its 8 XCDs round-robin, and
// without the renumbering every XCD's L2 holds the K/V of every pair in
// flight (L2 hit rate 0.89 -> 0.93, 7% faster at S = 4096).
#include <type_traits>

#include "common.h"
#include "gqa_internal.h"
#include "xcd_order.h"

namespace gqa {
namespace {

constexpr int kBN = 64;      // keys per tile
constexpr int kBQ = 16;      // query positions per workgroup
constexpr int kHeadsWG = 8;  // heads of the group per workgroup

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) void*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, r);
}

template <int D, bool OUT_BF16, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void prefill_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ kg, const __bf16* __restrict__ vg,
    void* __restrict__ out, const int32_t* __restrict__ kv_lens, int H, int K, int S, int S_kv,
    int S_max, int head_chunks, int hpw_log2, float scale_log2) {
  constexpr int KSTEPS = D / 32;
  constexpr int DT = D / 16;
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int TILE = kBN * D;             // elements per staged tile
  constexpr int COPIES = kBN * CPR / 64 / 4;  // 1 KB copies per wave per tile and tensor

  // The two stages of the K and V tiles are four distinct LDS objects, so
  // the compiler can tell that reads of one stage never touch the stage the
  // asynchronous copies are filling and does not make them wait for those
  // copies.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t k_lds1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds1[TILE];

  // the 8 row tiles of a workgroup: hpw heads x (8 / hpw) blocks of 16
  // positions (hpw = 8 unless the group has fewer heads)
  const int hpw = 1 << hpw_log2;
  const int qspan = kBQ * (8 >> hpw_log2);  // query positions per workgroup
  const int nqb = (S + qspan - 1) / qspan;
  // Workgroup (query block, KV head and head chunk, sequence), numbered so
  // that all query blocks of one (sequence, KV head) run on one XCD, whose L2
  // then holds that pair's K/V prefix for all of them.
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
  // The workgroup needs keys [0, kend); keys >= mask_from are hidden from
  // some of its rows.
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
  bf16x8 qf[2][KSTEPS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int pos_n = rq0[j] + n;
    const bool ld = hok[j] && pos_n < S;
    const __bf16* qrow = q + (((size_t)b * H + hglob[j]) * S + (ld ? pos_n : 0)) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[j][s] = as_bf16x8(ld ? ld16(qrow + 32 * s + 8 * g) : zero_u32x4());
  }

  // acc[jj][t]: O rows 4g+i, dims 16t+n.  lsum[jj]: the same rows' softmax
  // denominators, produced by one extra P.V column block whose V is all ones
  // (so the denominator sums exactly the bf16 weights the numerator uses).
  f32x4 acc[2][DT];
  f32x4 lsum[2];
  float m_run[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    m_run[j] = -INFINITY;
    lsum[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < DT; ++t) acc[j][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16x8 ones = as_bf16x8(u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

  const size_t kv_base = ((size_t)b * K + k) * (size_t)S_max * D;
  const __bf16* kbase = kg + kv_base;
  const __bf16* vbase = vg + kv_base;
  const int ntiles = kend > 0 ? (kend + kBN - 1) / kBN : 0;
  const bool any_head = hok[0];

  // LDS layout of a staged tile: whole rows of D bf16, their 16-byte chunks
  // XOR-swizzled by row -- K: chunk ^ (row % CPR), which spreads the eight
  // rows of a 16-byte operand read over distinct banks; V: chunk ^
  // 2 (row % (CPR/2)), which keeps the two chunks of a 32-byte transposed
  // read adjacent and puts consecutive rows in distinct 32-byte bank groups.
  // Copy ii of a tensor fills LDS chunks [64 ii, 64 ii + 64); lane l's chunk
  // is row (64 ii + l) / CPR, physical chunk l % CPR, so the lane fetches the
  // global chunk that belongs there.  Rows past the last key are fetched from
  // the last key instead (finite values; the mask gives them zero weight).
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  int crow[COPIES], koff[COPIES], voff[COPIES];
#pragma unroll
  for (int r = 0; r < COPIES; ++r) {
    const int c = 64 * (wave_s + 4 * r) + lane;
    const int row = c / CPR, cp = c - row * CPR;
    crow[r] = row;
    koff[r] = row * D + (cp ^ (row & (CPR - 1))) * 8;
    voff[r] = row * D + (cp ^ ((row & (CPR / 2 - 1)) << 1)) * 8;
  }
  auto copy_tile = [&](int kb0, auto stage_c) {
    constexpr int ST = decltype(stage_c)::value;
    const char* k0 = reinterpret_cast<const char*>(kbase + (size_t)kb0 * D);
    const char* v0 = reinterpret_cast<const char*>(vbase + (size_t)kb0 * D);
    const bool full = kb0 + kBN <= kend;  // uniform: only the last tile is ragged
#pragma unroll
    for (int r = 0; r < COPIES; ++r) {
      int ko = koff[r], vo = voff[r];
      if (!full) {
        const int past = kb0 + crow[r] - (kend - 1);
        if (past > 0) {
          ko -= past * D;
          vo -= past * D;
        }
      }
      // uniform base + 32-bit byte offset: the scalar-base addressing form
      __builtin_amdgcn_global_load_lds(k0 + (uint32_t)(2 * ko), (__attribute__((address_space(3))) void*)((ST == 0 ? k_lds0 : k_lds1) + (wave_s + 4 * r) * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(v0 + (uint32_t)(2 * vo), (__attribute__((address_space(3))) void*)((ST == 0 ? v_lds0 : v_lds1) + (wave_s + 4 * r) * 512), 16, 0, 0);
    }
  };

  // Loop-invariant LDS read offsets (elements).  K operand of k-step s: row
  // 16mt + n, logical chunk 4s + g.  V transposed read for dim block t: row
  // 32kk + 16hi + 4g + n/4, logical chunk 2t + (n%4)/2, half (n%2).
  int ka_off[KSTEPS], vb_off[DT];
#pragma unroll
  for (int s2 = 0; s2 < KSTEPS; ++s2) ka_off[s2] = n * D + (((4 * s2 + g) ^ (n & (CPR - 1))) * 8);
  {
    const int tr_row = 4 * g + (n >> 2);
    const int swz = (tr_row & (CPR / 2 - 1)) << 1;
#pragma unroll
    for (int t = 0; t < DT; ++t)
      vb_off[t] = tr_row * D + (((2 * t + ((n & 3) >> 1)) ^ swz) * 8) + 4 * (n & 1);
  }
  // A row's running max is only raised (and its accumulators rescaled) when
  // a tile's scores exceed it by more than 2^kLazy; otherwise the stale max
  // is kept, the weights stay <= 2^kLazy, and numerator and denominator
  // share it, so the quotient is unchanged.
  constexpr float kLazy = 8.f;

  auto tile = [&](int kb0, auto stage_c) {
    constexpr int ST = decltype(stage_c)::value;
    const uint16_t* kt = ST == 0 ? k_lds0 : k_lds1;
    const uint16_t* vt = ST == 0 ? v_lds0 : v_lds1;
    // ---- S^T = K_tile . Q^T for both row tiles (raw q.k) ----
    f32x4 st[2][4];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) st[jj][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    // k-step outer: the four K operands of a step are read together and feed
    // eight independent accumulation chains (bitwise the same sums; ~0.8%
    // faster than key-tile outer)
    for (int s2 = 0; s2 < KSTEPS; ++s2) {
      bf16x8 a[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        a[mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(&kt[ka_off[s2] + 16 * mt * D]));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          st[jj][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt], qf[jj][s2], st[jj][mt], 0, 0, 0);
    }
    // The K operands of k-step s + 1 are read while the MFMAs of k-step s
    // run (the compiler left on its own waits for each step's reads).
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int s2 = 0; s2 < KSTEPS; ++s2) {
      if (s2 + 2 < KSTEPS) __builtin_amdgcn_sched_group_barrier(0x008, 8, 0), __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      else __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    if (kb0 + kBN > mask_from) {  // diagonal / last tile: drop keys >= the row's limit
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kb0 + 16 * mt + 4 * g + i >= lim[jj]) st[jj][mt][i] = -INFINITY;
    }

    // ---- online softmax per row tile ----
    bf16x8 pa[2][2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      // lane-local max of this lane's 16 scores of row n; the wave only
      // needs the row's exact max (a cross-lane reduction) when some score
      // exceeds the stale max by more than 2^kLazy
      float lmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, st[jj][mt][i]);
      if (__any(lmax * scale_log2 > m_run[jj] + kLazy)) {  // scale > 0
        float cmax = fmaxf(lmax, __shfl_xor(lmax, 16));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
        const float m_new = fmaxf(m_run[jj], cmax * scale_log2);
        const float alpha = fast_exp2(m_run[jj] - m_new);
        m_run[jj] = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = __shfl(alpha, 4 * g + i);
          lsum[jj][i] *= a;
#pragma unroll
          for (int t = 0; t < DT; ++t) acc[jj][t][i] *= a;
        }
      }
      // a row that has seen no visible key yet keeps all weights at zero
      const float mneg = m_run[jj] == -INFINITY ? 0.f : -m_run[jj];
      uint32_t pw[8];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; i += 2)
          pw[2 * mt + i / 2] = pack_bf16x2(fast_exp2(fmaf(st[jj][mt][i], scale_log2, mneg)),
                                           fast_exp2(fmaf(st[jj][mt][i + 1], scale_log2, mneg)));
      // P operand of 32-key step kk: score tiles mt = 2kk, 2kk+1
      pa[jj][0] = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
      pa[jj][1] = as_bf16x8(u32x4{pw[4], pw[5], pw[6], pw[7]});
    }

    // ---- O += P . V_tile, and the denominators via the all-ones block ----
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const uint2 lo = lds_read_tr16(vt + vb_off[t] + 32 * kk * D);
        const uint2 hi = lds_read_tr16(vt + vb_off[t] + (32 * kk + 16) * D);
        const bf16x8 vb = as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
          acc[jj][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[jj][kk], vb, acc[jj][t], 0, 0, 0);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        lsum[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[jj][kk], ones, lsum[jj], 0, 0, 0);
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  if (ntiles > 0) copy_tile(0, S0{});
  // Tiles alternate between the two LDS stages; the loop is unrolled by two
  // so each stage's addresses are compile-time offsets.
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
  for (int jj = 0; jj < 2; ++jj) {
    if (!hok[jj]) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = rq0[jj] + 4 * g + i;
      if (pos >= S) continue;
      const float inv = lsum[jj][i] > 0.f ? 1.f / lsum[jj][i] : 0.f;  // no visible key: zero row
      const size_t orow = (((size_t)b * H + hglob[jj]) * S + pos) * D;
#pragma unroll
      for (int t = 0; t < DT; ++t) {
        const float o = acc[jj][t][i] * inv;
        if (OUT_BF16)
          static_cast<__bf16*>(out)[orow + 16 * t + n] = static_cast<__bf16>(o);
        else
          static_cast<float*>(out)[orow + 16 * t + n] = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* out,
                               const int32_t* kv_lens, int B, int H, int K, int S, int S_kv,
                               int S_max, int d, float scale_log2, bool out_bf16, bool causal,
                               hipStream_t stream) {
  const int G = H / K;
  // heads per workgroup: the group's heads rounded up to a power of two (at
  // most 8); the remaining row tiles take further blocks of positions
  int hpw_log2 = 0;
  while ((1 << hpw_log2) < G && (1 << hpw_log2) < kHeadsWG) ++hpw_log2;
  const int head_chunks = (G + (1 << hpw_log2) - 1) >> hpw_log2;
  const int qspan = kBQ * (kHeadsWG >> hpw_log2);
  const dim3 grid((S + qspan - 1) / qspan, K * head_chunks, B);
  const dim3 block(256);
  auto qp = static_cast<const __bf16*>(q);
  auto kp = static_cast<const __bf16*>(k);
  auto vp = static_cast<const __bf16*>(v);
#define GQA_PREFILL(DD, OB, CA)                                                                 \
  hipLaunchKernelGGL((prefill_kernel<DD, OB, CA>), grid, block, 0, stream, qp, kp, vp, out,      \
                     kv_lens, H, K, S, S_kv, S_max, head_chunks, hpw_log2, scale_log2)
#define GQA_PREFILL_C(DD, OB)                                                                   \
  if (causal) GQA_PREFILL(DD, OB, true); else GQA_PREFILL(DD, OB, false);
  if (d == 128) {
    if (out_bf16) { GQA_PREFILL_C(128, true) } else { GQA_PREFILL_C(128, false) }
  } else {
    if (out_bf16) { GQA_PREFILL_C(64, true) } else { GQA_PREFILL_C(64, false) }
  }
#undef GQA_PREFILL_C
#undef GQA_PREFILL
  return hipGetLastError();
}

}  // namespace gqa
