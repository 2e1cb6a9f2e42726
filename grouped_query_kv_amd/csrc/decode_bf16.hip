// Decode partition pass for bf16 caches, on the gfx950 matrix cores.
//
// What it computes (compassingai.com "分組查詢注意力", section 技術原理: the
// G query heads of group g attend to the one shared K_g, V_g with
// softmax(Q_g K_g^T / sqrt(d_k)) V_g): for a partition [t0, t1) of the
// positions of sequence b and KV head k, and every query head h of the
// group, the un-normalised online-softmax state
//     m_h   = max_j s_hj            (s_hj = scale * log2(e) * q_h . k_j)
//     l_h   = sum_j 2^(s_hj - m_h)
//     acc_h = sum_j 2^(s_hj - m_h) v_j
// which the combine pass merges across partitions.  Working in base 2 with
// log2(e) folded into the scale gives the same softmax.
//
// How (pinghaoyang.com.cn "GQA 完全拆解", section 工程实现 (engineering): the
// group's shared KV block is loaded once and reused by all its query heads):
// one wavefront owns one flat range of (sequence, KV head, position) -- the
// split of decode_flat.h, equal ranges for every workgroup however ragged
// the batch -- and streams each of its segments in chunks of 32 positions.
// Each K row is read from HBM once, straight into matrix-core operand
// registers, and multiplies all (up to 16) query heads of the group in one
// v_mfma_f32_16x16x32_bf16:  S^T[32 x 16] = K_chunk[32 x d] . Q_g^T[d x 16].
// Each V row is read from HBM once, staged through LDS to be re-laid out as
// the matrix-core operand, and then serves all heads:
//     O[16 x d] += P[16 x 32] . V_chunk[32 x d].
//
// Operand layouts of v_mfma_f32_16x16x32_bf16 (wave64, lane l, n = l % 16,
// g = l / 16): A row m = n holds 8 k-values selected by g; B column n holds
// the same 8 k-values; C/D lane l holds D[4g + i][n], i = 0..3.  Because the
// k-index of both operands is chosen by (g, element) in the same way, any
// relabelling of the contraction index that is applied to both operands
// gives the same product.  This kernel uses that freedom twice:
//   * Q.K: lane (n, g) at k-step s carries head dimensions 32s + 8g .. +7, so
//     every K operand is one 16-byte load from a K row;
//   * P.V: the scores come out of the first product as lane (n = head, g)
//     holding positions {4g+i, 16+4g+i}; those eight positions are used as
//     that lane's contraction slots, so P needs no data movement.
// V is staged row-major in LDS and read back transposed with
// ds_read_b64_tr_b16: within each 16-lane group, the 64-bit reads of lanes
// 4r..4r+3 form row r of a 4 x 16 block of bf16 and lane i receives column i.
// Pointing the four lanes of row r at V[position r][16t .. 16t+15] gives lane
// (n, g) the values V[p][16t + n] of four positions p, which is exactly half
// of its B operand; two such reads give the eight contraction slots.
//
// Loads of chunk c+1 are issued before the arithmetic of chunk c so the
// wavefront always has a chunk of K and V in flight.  The cache is streamed
// with non-temporal loads (every byte is read once per step).
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kChunk = 32;   // positions per inner iteration
// bf16 elements of padding per LDS row: a 32-byte shift per row puts the
// four rows of one 16-lane transposed read in distinct 32-byte bank groups
constexpr int kVPad = 16;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed 64-bit LDS read (see the layout note above).
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) void*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, r);
}

// APPEND: fused cache append.  The step's new K/V rows (k_new, v_new) sit at
// position L_in = seq_lens[b] (when the cache has room -- paged: when L_in is
// below the table's capacity and the block id at L_in is a valid one, the
// standalone paged append's rule): the segment that covers it reads that row
// from k_new/v_new and writes it into the cache (head block 0 only; nothing
// else reads that row in this launch).  Workgroup 0 records the lengths
// attended over (after the append) with the split for the combine pass,
// which publishes them to seq_lens.
//
// PAGED: kc/vc are block pools [num_blocks, K, block_size, D] and position j
// of sequence b lives in physical block block_table[b][j / block_size], row
// j % block_size.  block_size is a multiple of 16, so every 16-row load group
// lies in one block and its block id is wave-uniform: each wavefront loads
// the block ids of its partition once (one per lane) and takes them with
// readlane.  Ids are clamped into [0, num_blocks) and lengths to the table's
// capacity, so a malformed table cannot make a load leave the pool.
template <int D, bool APPEND, bool PAGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_split_bf16_kernel(
    const __bf16* __restrict__ q, __bf16* __restrict__ kc, __bf16* __restrict__ vc,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_acc,
    float* __restrict__ part_ml, int B, int H, int K, int S_max, FlatArgs fa, int head_blocks,
    float scale_log2, const __bf16* __restrict__ k_new, const __bf16* __restrict__ v_new,
    int32_t* __restrict__ meta, PagedArgs pg) {
  static_assert(D == 64 || D == 128, "head dimension");
  constexpr int KSTEPS = D / 32;        // contraction steps of Q.K
  constexpr int NTILES = D / 16;        // 16-wide output tiles of P.V
  constexpr int LANES_PER_ROW = D / 8;  // 16-byte words per V row
  constexpr int ROWS_PER_LOAD = 64 / LANES_PER_ROW;
  constexpr int VLOADS = kChunk / ROWS_PER_LOAD;
  constexpr int LDS_ROW = D + kVPad;

  __shared__ __attribute__((aligned(16))) uint16_t vt[kChunk * LDS_ROW];

  // Work of this workgroup: head block hb of the flat range w (see
  // decode_flat.h; groups of more than 128 heads run several head blocks,
  // each re-reading the range).
  const int w = blockIdx.x / head_blocks;
  const int hb = blockIdx.x - w * head_blocks;
  const int G = H / K;
  const int cap = PAGED ? pg.max_blocks * pg.block_size : S_max;  // positions the cache holds
  // lengths clamped into [0, cap], so no length can make a load leave the cache
  auto len_in = [&](int bb) -> int { return min(max(seq_lens[bb], 0), cap); };
  // length attended over: after the fused append when the cache has room
  auto len_of = [&](int bb) -> int {
    const int L_in = len_in(bb);
    if (!APPEND) return min(L_in, fa.max_len);
    bool room = L_in < cap;
    if (PAGED && room) {
      const int id = pg.block_table[(size_t)bb * pg.max_blocks + L_in / pg.block_size];
      room = id >= 0 && id < pg.num_blocks;
    }
    return min(room ? L_in + 1 : L_in, fa.max_len);
  };
  // the lengths attended over and the split, for the combine pass
  const int l0 = first_lengths(B, len_of);  // lengths of sequences 0..63, one per lane
  if (blockIdx.x == 0) flat_publish(B, K, l0, len_of, meta);
  const int total = flat_total(B, K, l0, len_of);
  const int R = flat_range(total, fa);

  flat_for_each_segment(w, B, K, total, R, l0, len_of,
                        [&](int b, int k, int t0, int t1, int L, int slot) {
  const int newpos = APPEND && L > len_in(b) ? L - 1 : -1;  // the appended row, if any
  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int g = lane >> 4;

  // Q^T operand: lane (n, g) holds head hb*16+n, dims 32s+8g..+7.
  const int hq = hb * 16 + n;
  const bool hq_ok = hq < G;
  bf16x8 qf[KSTEPS];
  {
    const __bf16* qrow = q + ((size_t)b * H + (size_t)k * G + (hq_ok ? hq : 0)) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qf[s] = as_bf16x8(hq_ok ? ld16(qrow + 32 * s + 8 * g) : zero_u32x4());
  }

  const size_t head_base = PAGED ? 0 : ((size_t)b * K + k) * (size_t)S_max * D;
  __bf16* kbase = kc + head_base;
  __bf16* vbase = vc + head_base;
  // paged: lane i holds the physical id of logical block lb0 + i
  const int lb0 = PAGED ? t0 / pg.block_size : 0;
  int blk_id = 0;
  if (PAGED) {
    const int nb = (t1 - 1) / pg.block_size - lb0 + 1;  // <= 64 by the split plan
    if (threadIdx.x < nb)
      blk_id = min(max(pg.block_table[(size_t)b * pg.max_blocks + lb0 + threadIdx.x], 0), pg.num_blocks - 1);
  }
  // first element of cache row `tok`, where `tok0` is a wave-uniform position
  // of the same 16-row group
  auto row_of = [&](__bf16* base, int tok0, int tok) -> __bf16* {
    if (!PAGED) return base + (size_t)tok * D;
    const int blk = __builtin_amdgcn_readlane(blk_id, tok0 / pg.block_size - lb0);
    return base + (((size_t)blk * K + k) * pg.block_size + (tok - (tok0 / pg.block_size) * pg.block_size)) * D;
  };
  const __bf16* knew_row = APPEND ? k_new + ((size_t)b * K + k) * D : nullptr;
  const __bf16* vnew_row = APPEND ? v_new + ((size_t)b * K + k) * D : nullptr;

  float m_run = -INFINITY;  // running max of head n (replicated over g)
  float l_run = 0.f;        // this lane's share of the running sum of head n
  f32x4 acc[NTILES];
#pragma unroll
  for (int t = 0; t < NTILES; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int vrow = lane / LANES_PER_ROW;
  const int vcol = (lane % LANES_PER_ROW) * 8;
  // transposed-read source of this lane: row 4g + (n/4) (+16 for slots 4..7),
  // dims 16t + 4*(n%4)
  const uint16_t* tr_src = &vt[(4 * g + (n >> 2)) * LDS_ROW + 4 * (n & 3)];

  // K operands of two chunks, used in turn (the loop is unrolled by two), so
  // the prefetch of chunk c+1 is never copied between registers; measured
  // 1.5-2% faster on the decode workloads than one set
  u32x4 ka0[2][KSTEPS], ka1[2][KSTEPS];
  u32x4 vr[VLOADS];
  // Rows past the partition are fetched from its last row instead (valid
  // memory; their scores are masked and their weights are zero), so no load
  // is predicated.  A clamped row stays in the clamped load group, so a
  // paged group still lies in one block.
  const int last = t1 - 1;
  auto load_k = [&](u32x4 (&ka)[2][KSTEPS], int c0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int tok0 = min(c0 + 16 * mt, last & ~15);
      const int tok = min(c0 + 16 * mt + n, last);
      const __bf16* krow = (APPEND && tok == newpos ? knew_row : row_of(kbase, tok0, tok)) + 8 * g;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) ka[mt][s] = ld16_stream(krow + 32 * s);
    }
  };
  auto load_v = [&](int c0) {
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int tok0 = min(c0 + i * ROWS_PER_LOAD, last & ~(ROWS_PER_LOAD - 1));
      const int tok = min(c0 + i * ROWS_PER_LOAD + vrow, last);
      const __bf16* vrow_p = APPEND && tok == newpos ? vnew_row : row_of(vbase, tok0, tok);
      vr[i] = ld16_stream(vrow_p + vcol);
    }
  };
  load_k(ka0, t0);
  load_v(t0);

  auto chunk = [&](u32x4 (&ka)[2][KSTEPS], u32x4 (&ka_next)[2][KSTEPS], int c0) {
    const bool more = c0 + kChunk < t1;
    // ---- S^T = K . Q^T for the two 16-position tiles ----
    f32x4 st[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
        st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[mt][s]), qf[s], st[mt], 0, 0, 0);
    }
    if (more) load_k(ka_next, c0 + kChunk);  // next chunk's K streams during this chunk

    // ---- online softmax for head n over positions {16mt + 4g + i} ----
    // A head's running max is raised (and its accumulators rescaled) only
    // when some score of the chunk exceeds it by more than 2^kLazy;
    // otherwise the stale max stays, the weights stay below 2^kLazy, and
    // numerator and denominator share it (the combine pass takes any max).
    // l_run holds this lane's share of the denominator (its positions); the
    // shares are summed over the lane groups once, after the loop.
    constexpr float kLazy = 8.f;
    // Raw scores; positions past the segment (only in its last chunk) get
    // -inf.  scale > 0, so the largest scaled score is the largest raw score
    // times the scale, and each weight is one fma and one exponential.
    if (c0 + kChunk > t1) {  // uniform
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c0 + 16 * mt + 4 * g + i >= t1) st[mt][i] = -INFINITY;
    }
    float lmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, st[mt][i]);
    if (__any(lmax * scale_log2 > m_run + kLazy)) {  // always on the first chunk (m_run = -inf)
      float cmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      const float m_new = fmaxf(m_run, cmax * scale_log2);  // finite: the chunk has >= 1 position
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      // acc rows are heads 4g+i; their rescale factors live in lanes 4g+i.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = __shfl(alpha, 4 * g + i);
#pragma unroll
        for (int t = 0; t < NTILES; ++t) acc[t][i] *= a;
      }
    }
    const float mneg = -m_run;
    uint32_t pw[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float e0 = fast_exp2(fmaf(st[j >> 2][j & 3], scale_log2, mneg));
      const float e1 = fast_exp2(fmaf(st[(j + 1) >> 2][(j + 1) & 3], scale_log2, mneg));
      l_run += e0 + e1;
      pw[j / 2] = pack_bf16x2(e0, e1);
    }

    // ---- V chunk -> LDS (row-major), then transposed reads as B operand ----
#pragma unroll
    for (int i = 0; i < VLOADS; ++i)
      *reinterpret_cast<u32x4*>(&vt[(i * ROWS_PER_LOAD + vrow) * LDS_ROW + vcol]) = vr[i];
    __syncthreads();
    if (more) load_v(c0 + kChunk);  // next chunk's V streams during P.V
    const bf16x8 pa = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
    for (int t = 0; t < NTILES; ++t) {
      const uint2 lo = lds_read_tr16(tr_src + 16 * t);
      const uint2 hi = lds_read_tr16(tr_src + 16 * LDS_ROW + 16 * t);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y}),
                                                       acc[t], 0, 0, 0);
    }
    __syncthreads();  // LDS reads done before the next chunk overwrites vt
  };

  for (int c0 = t0;; c0 += 2 * kChunk) {
    chunk(ka0, ka1, c0);
    if (c0 + kChunk >= t1) break;
    chunk(ka1, ka0, c0 + kChunk);
    if (c0 + 2 * kChunk >= t1) break;
  }

  if (APPEND && hb == 0 && newpos >= t0 && newpos < t1) {  // wave-uniform
    // the appended rows join the cache (bit copy)
    __bf16* kdst = row_of(kbase, newpos, newpos);
    __bf16* vdst = row_of(vbase, newpos, newpos);
    if (lane < LANES_PER_ROW) {
      *reinterpret_cast<u32x4*>(kdst + 8 * lane) = ld16(knew_row + 8 * lane);
      *reinterpret_cast<u32x4*>(vdst + 8 * lane) = ld16(vnew_row + 8 * lane);
    }
  }

  l_run += __shfl_xor(l_run, 16);  // the head's denominator: sum of the lane groups' shares
  l_run += __shfl_xor(l_run, 32);

  // ---- write the segment's partial state (slot rows = the group's heads) ----
  const size_t row0 = (size_t)slot * G + (size_t)hb * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hl = 4 * g + i;
    if (hb * 16 + hl < G) {
      float* dst = part_acc + (row0 + hl) * D;
#pragma unroll
      for (int t = 0; t < NTILES; ++t) dst[16 * t + n] = acc[t][i];
    }
  }
  if (g == 0 && hq_ok) {
    float* ml = part_ml + (row0 + n) * 2;
    ml[0] = m_run;
    ml[1] = l_run;
  }
                        });
}

}  // namespace

hipError_t launch_decode_split_bf16(const void* q, void* k_cache, void* v_cache,
                                    const int32_t* seq_lens, const DecodeWorkspace& ws,
                                    const DecodePlan& plan, int B, int H, int K, int S_max, int d,
                                    float scale_log2, const void* k_new, const void* v_new,
                                    const PagedArgs* paged, hipStream_t stream) {
  if (decode_wide_supported(plan.head_blocks))  // G > 16: one KV read for all head blocks
    return launch_decode_wide_bf16(q, k_cache, v_cache, seq_lens, ws, plan, B, H, K, S_max, d,
                                   scale_log2, k_new, v_new, paged, stream);
  const dim3 grid(plan.fa.n_wg * plan.head_blocks);
  const dim3 block(64);
  auto qp = static_cast<const __bf16*>(q);
  auto kp = static_cast<__bf16*>(k_cache);
  auto vp = static_cast<__bf16*>(v_cache);
  auto kn = static_cast<const __bf16*>(k_new);
  auto vn = static_cast<const __bf16*>(v_new);
  const PagedArgs pg = paged ? *paged : PagedArgs{nullptr, 16, 0, 1};
#define GQA_SPLIT(DD, AP, PG)                                                                     \
  hipLaunchKernelGGL((decode_split_bf16_kernel<DD, AP, PG>), grid, block, 0, stream, qp, kp, vp,  \
                     seq_lens, ws.part_acc, ws.part_ml, B, H, K, S_max, plan.fa, plan.head_blocks,  \
                     scale_log2, kn, vn, ws.meta, pg)
#define GQA_SPLIT_D(DD)                                                                           \
  if (paged) {                                                                                    \
    if (k_new) GQA_SPLIT(DD, true, true); else GQA_SPLIT(DD, false, true);                        \
  } else {                                                                                        \
    if (k_new) GQA_SPLIT(DD, true, false); else GQA_SPLIT(DD, false, false);                      \
  }
  if (d == 128) {
    GQA_SPLIT_D(128)
  } else {
    GQA_SPLIT_D(64)
  }
#undef GQA_SPLIT_D
#undef GQA_SPLIT
  return hipGetLastError();
}

}  // namespace gqa
