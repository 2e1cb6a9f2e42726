// Decode partition pass for groups of more than 16 query heads (bf16).
//
// The one-wave pass (decode_bf16.hip) multiplies a K chunk held in registers
// by the 16 query heads one matrix-core instruction covers; a group of G > 16
// heads (MQA shapes: one KV head for 32, 64 or 71 query heads) would need
// ceil(G / 16) such waves, each reading the same K and V rows from memory.
// The pages' engineering rule is that a group's shared KV block is loaded
// once for all of its heads (pinghaoyang.com.cn "GQA 完全拆解", section 工程实现;
// its MQA section: all heads share one K/V head).  So here one workgroup of W
// waves, one per 16-head block of the group (the last may hold fewer heads),
// owns a partition of one KV head: the waves copy the partition's K and V
// rows together into LDS, once, and each wave multiplies them with its own
// heads.
//
// Rows are staged in blocks of 32*SUB positions through a ring of NS LDS
// buffers, filled by direct global-to-LDS copies (global_load_lds_dwordx4:
// lane i of a wave instruction lands its 16 bytes at LDS base + 16 i, no
// registers involved), so NS-1 blocks are in flight per workgroup at no
// register cost.  Per block: wait for this wave's copies
// of the block, barrier, issue the copies of block j+NS-1 into the buffer
// the previous block used, then per 32-position chunk and per wave S^T =
// K_chunk . Q_hb^T (K operands read from LDS, same operand layout and
// contraction relabelling as the one-wave pass), the lazy base-2 online
// softmax, and O += P . V_chunk (V read transposed from LDS).  The partial
// state written per head is the one-wave pass's, so the same combine pass
// merges it.
//
// What bounds it (measured on multi-query shapes, d = 64 and 128, 2 to 5
// head blocks): the copy stream.  A variant that only copies takes as long
// as the whole pass, one that only computes takes 65-75% of it; deeper
// rings, 64-position blocks, register-staged copies and other workgroup
// counts do not speed the copies up, the non-temporal cache policy does
// (5-12%).  The arithmetic is kept lean all the same (about 40 vector
// instructions per wave and chunk): the appended row is written into the
// cache before the ring starts, so no copy needs a select; a copy address is
// the block's first row (scalar) plus a small per-lane offset; the running
// sum takes the packed bf16 weights with one dot-product instruction per
// pair.
//
// LDS layout of a staged tensor: whole unpadded rows of D bf16 whose 16-byte
// chunks are XOR-swizzled by row, K: chunk ^ (row % (D/8)), V: chunk ^
// 2 (row % (D/16)) at d = 128 (the prefill kernel's layout) and chunk ^
// 2 ((row / 2) % 4) at d = 64, where the rows are half as long and the
// d = 128 rule puts rows r and r + 4 of a transposed read in the same banks
// (bank-conflict counter: 1.05M cycles per launch -> 0).  Each lane fetches
// the global chunk that belongs in its LDS slot.
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

// Cache policy of the global-to-LDS copies of the cache: non-temporal (every
// byte is read once per step).  Measured on multi-query shapes: 5-12% faster
// than the default policy; the scope bits (sc0, sc1) add nothing.
constexpr int kStreamAux = 2;  // the nt bit of the instruction's cache-policy field

constexpr int kChunk = 32;  // positions per inner iteration
// LDS buffers in the ring and 32-position chunks per block.  Measured on
// five multi-query shapes (d = 64 and 128, 2 to 5 head blocks, 67-537 MB of
// cache): two buffers of one chunk -- 16 KB of K and V at d = 128, 8 KB at
// d = 64, so that many workgroups fit a CU's LDS -- beat three or four
// buffers (3-25% slower) and two-chunk blocks at d = 64 (0-6% slower).
constexpr int kRing = 2;
constexpr int kSub = 1;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) void*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, r);
}

// physical-chunk XOR of a staged V row r (the layout described above)
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  return D == 64 ? ((r >> 1) & 3) << 1 : (r & 7) << 1;
}

// s_waitcnt immediate (gfx9 encoding): vector-memory count <= vm, LDS count 0
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | (7 << 4) | (((vm >> 4) & 3) << 14); }

// Four workgroups of W waves per CU: from W = 5 on, the d = 64 pass must fit six
// waves per SIMD (at most 80 registers) so that four workgroups stay resident.
template <int D, int W>
constexpr int wide_min_waves() { return D == 64 && W >= 5 ? 6 : 1; }

template <int D, bool APPEND, bool PAGED, int W, int SUB, int NS>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(wide_min_waves<D, W>()))) void decode_wide_bf16_kernel(
    const __bf16* __restrict__ q, __bf16* __restrict__ kc, __bf16* __restrict__ vc,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_acc,
    float* __restrict__ part_ml, int B, int H, int K, int S_max, FlatArgs fa,
    float scale_log2, const __bf16* __restrict__ k_new, const __bf16* __restrict__ v_new,
    int32_t* __restrict__ meta, PagedArgs pg) {
  static_assert(D == 64 || D == 128, "head dimension");
  static_assert(NS >= 2 && NS <= 4, "ring depth");
  constexpr int KSTEPS = D / 32;
  constexpr int NTILES = D / 16;
  constexpr int LPR = D / 8;                  // 16-byte chunks per row
  constexpr int RPW = 64 / LPR;               // rows per wave instruction
  constexpr int RCH = kChunk * SUB;           // rows per staged block
  constexpr int TILE = RCH * D;               // bf16 elements per staged tensor
  constexpr int NINST = RCH / RPW;            // 1 KB copies per tensor and block
  constexpr int NI = (NINST + W - 1) / W;     // copies per wave per tensor and block
  constexpr bool SURPLUS = NINST % W != 0;    // some waves have one copy too many
  static_assert(NINST * 512 == TILE, "copies cover a staged tensor");
  static_assert(2 * NI * (NS - 2) < 64, "vector-memory counter range");

  __shared__ __attribute__((aligned(16))) uint16_t lds[NS][2][TILE];  // [buffer][K|V]
  // target of the surplus copies (they repeat a real copy; their bytes are
  // never read), so every wave issues the same number of copies per block
  __shared__ __attribute__((aligned(16))) uint16_t sink[SURPLUS ? 512 : 8];

  const int G = H / K;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int hb = wave;  // this wave's block of 16 heads

  const int cap = PAGED ? pg.max_blocks * pg.block_size : S_max;
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
  if (blockIdx.x == 0 && wave == 0) flat_publish(B, K, l0, len_of, meta);
  const int total = flat_total(B, K, l0, len_of);
  const int R = flat_range(total, fa);

  flat_for_each_segment(blockIdx.x, B, K, total, R, l0, len_of,
                        [&](int b, int k, int t0, int t1, int L, int slot) {
  const int newpos = APPEND && L > len_in(b) ? L - 1 : -1;  // the appended row, if any
  const int last = t1 - 1;

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
  const int lb0 = PAGED ? t0 / pg.block_size : 0;
  int blk_id = 0;
  if (PAGED) {
    const int nb = (t1 - 1) / pg.block_size - lb0 + 1;  // <= 64 by the split plan
    if (lane < nb)
      blk_id = min(max(pg.block_table[(size_t)b * pg.max_blocks + lb0 + lane], 0), pg.num_blocks - 1);
  }
  // first element of cache row `tok`; `tok0` is a wave-uniform position of
  // the same RPW-row group (inside one block: block_size is a multiple of 16)
  auto row_of = [&](__bf16* base, int tok0, int tok) -> __bf16* {
    if (!PAGED) return base + (size_t)tok * D;
    const int blk = __builtin_amdgcn_readlane(blk_id, tok0 / pg.block_size - lb0);
    return base + (((size_t)blk * K + k) * pg.block_size + (tok - (tok0 / pg.block_size) * pg.block_size)) * D;
  };
  // The fused append: the workgroup whose partition holds the appended
  // position writes the new K and V rows into the cache before anything is
  // copied, so every copy below reads the cache alone.  Wave 0 waits for
  // its stores to complete (vmcnt(0): a workgroup-scope release alone
  // compiles to no wait here) before the barrier, so no other wave's copy of
  // the row can overtake them.
  if (APPEND && newpos >= t0 && newpos < t1) {  // uniform
    if (wave == 0 && lane < LPR) {
      const __bf16* knew_row = k_new + ((size_t)b * K + k) * D;
      const __bf16* vnew_row = v_new + ((size_t)b * K + k) * D;
      *reinterpret_cast<u32x4*>(row_of(kbase, newpos, newpos) + 8 * lane) = ld16(knew_row + 8 * lane);
      *reinterpret_cast<u32x4*>(row_of(vbase, newpos, newpos) + 8 * lane) = ld16(vnew_row + 8 * lane);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }

  // Copy slot c of this wave is instruction i = wave + c W of the block
  // (surplus slots, i >= NINST: with a ring of three or more buffers they
  // repeat instruction i - NINST into the sink, so that every wave issues the
  // same number of copies per block as the ring's counted waits assume; with
  // two, whose waits are for every copy, they are skipped): lane l fills LDS chunk 64 i + l = row r, physical chunk l % LPR, with the
  // logical chunk that the swizzle puts there (ck, cv: that chunk's byte
  // offset inside its K and V row).  Rows past the partition end are fetched
  // from its last row (valid memory; masked).
  int crow[NI];
  uint32_t ck[NI], cv[NI];
#pragma unroll
  for (int c = 0; c < NI; ++c) {
    const int i = (wave + c * W) % NINST;
    const int r = (64 * i + lane) / LPR, ph = lane % LPR;
    crow[c] = r;
    ck[c] = 16 * (ph ^ (r & (LPR - 1)));
    cv[c] = 16 * (ph ^ v_swizzle<D>(r));
  }
  auto copy_block = [&](int b0, int buf) {
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      const int i = wave + c * W;  // uniform
      if (NS < 3 && i >= NINST) continue;
      const int ir = i % NINST;
      const char* kp;
      const char* vp;
      if (!PAGED) {
        // the block's first row (uniform) plus a small per-lane offset
        const uint32_t ro = (uint32_t)min(crow[c], last - b0) * (uint32_t)(2 * D);
        kp = reinterpret_cast<const char*>(kbase + (size_t)b0 * D) + (ro + ck[c]);
        vp = reinterpret_cast<const char*>(vbase + (size_t)b0 * D) + (ro + cv[c]);
      } else {
        const int tok0 = min(b0 + ir * RPW, last & ~(RPW - 1));
        const int tok = min(b0 + crow[c], last);
        kp = reinterpret_cast<const char*>(row_of(kbase, tok0, tok)) + ck[c];
        vp = reinterpret_cast<const char*>(row_of(vbase, tok0, tok)) + cv[c];
      }
      uint16_t* kd = i < NINST ? &lds[buf][0][i * 512] : sink;
      uint16_t* vd = i < NINST ? &lds[buf][1][i * 512] : sink;
      // (a char source pointer: with a __bf16 one the host pass drops the
      // kernel's launch stub without a diagnostic)
      __builtin_amdgcn_global_load_lds(kp, (__attribute__((address_space(3))) void*)kd, 16, 0, kStreamAux);
      __builtin_amdgcn_global_load_lds(vp, (__attribute__((address_space(3))) void*)vd, 16, 0, kStreamAux);
    }
  };

  // loop-invariant LDS offsets (elements): K operand of k-step s is row
  // 16mt + n of a chunk, logical chunk 4s + g; the transposed V read of dim
  // block t is row 4g + n/4 (+16), logical chunk 2t + (n%4)/2, half n%2
  int ka_off[KSTEPS], vb_off[NTILES];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) ka_off[s] = n * D + (((4 * s + g) ^ (n & (LPR - 1))) * 8);
  {
    const int tr_row = 4 * g + (n >> 2);
    const int swz = v_swizzle<D>(tr_row);  // the same for tr_row + 16
#pragma unroll
    for (int t = 0; t < NTILES; ++t)
      vb_off[t] = tr_row * D + (((2 * t + ((n & 3) >> 1)) ^ swz) * 8) + 4 * (n & 1);
  }

  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's share of the running sum of head n
  f32x4 acc[NTILES];
#pragma unroll
  for (int t = 0; t < NTILES; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr float kLazy = 8.f;  // see the one-wave pass: lazy running max
  const bf16x2 kOnes2 = __builtin_bit_cast(bf16x2, 0x3F803F80u);

  auto compute_block = [&](int b0, int buf) {
#pragma unroll
    for (int sc = 0; sc < SUB; ++sc) {
      const int c0 = b0 + kChunk * sc;
      if (c0 >= t1) break;  // uniform
      const uint16_t* kt = &lds[buf][0][kChunk * sc * D];
      const uint16_t* vt = &lds[buf][1][kChunk * sc * D];
      // ---- S^T = K . Q^T (K operands from LDS) ----
      f32x4 st[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(&kt[16 * mt * D + ka_off[s]]);
          st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qf[s], st[mt], 0, 0, 0);
        }
      }
      // ---- online softmax for head n over positions {16mt + 4g + i} ----
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
      if (__any(lmax * scale_log2 > m_run + kLazy)) {
        float cmax = fmaxf(lmax, __shfl_xor(lmax, 16));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
        const float m_new = fmaxf(m_run, cmax * scale_log2);
        const float alpha = fast_exp2(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = __shfl(alpha, 4 * g + i);
#pragma unroll
          for (int t = 0; t < NTILES; ++t) acc[t][i] *= a;
        }
      }
      const float mneg = -m_run;  // finite: the segment's first chunk set it
      uint32_t pw[4];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const float e0 = fast_exp2(fmaf(st[j >> 2][j & 3], scale_log2, mneg));
        const float e1 = fast_exp2(fmaf(st[(j + 1) >> 2][(j + 1) & 3], scale_log2, mneg));
        pw[j / 2] = pack_bf16x2(e0, e1);
        // the running sum takes the rounded weights that multiply V
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[j / 2]), kOnes2, l_run, false);
      }
      // ---- O += P . V (V read transposed from LDS) ----
      const bf16x8 pa = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
      for (int t = 0; t < NTILES; ++t) {
        const uint2 lo = lds_read_tr16(vt + vb_off[t]);
        const uint2 hi = lds_read_tr16(vt + vb_off[t] + 16 * D);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y}),
                                                         acc[t], 0, 0, 0);
      }
    }
  };

  // ---- the ring: NS-1 blocks in flight ----
  const int nblk = (t1 - t0 + RCH - 1) / RCH;
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < nblk) copy_block(t0 + j * RCH, j);
  for (int j = 0; j < nblk; ++j) {
    // this wave's copies of block j have landed once at most the copies of
    // the blocks issued after it are outstanding (2 NI per block)
    const int ahead = min(NS - 2, nblk - 1 - j);
    if (NS >= 4 && ahead >= 2) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(4 * NI));
    } else if (NS >= 3 && ahead >= 1) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * NI));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    }
    // block j is in LDS for every wave, and every wave is done reading block
    // j-1 (its buffer is refilled next).  A bare s_barrier: a workgroup fence
    // would also wait for the copies still in flight.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (j + NS - 1 < nblk) copy_block(t0 + (j + NS - 1) * RCH, (j + NS - 1) % NS);
    compute_block(t0 + j * RCH, j % NS);
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

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
  // every wave is done with the ring before the next segment refills it
  __syncthreads();
                        });
}

}  // namespace

bool decode_wide_supported(int head_blocks) { return head_blocks > 1 && head_blocks <= 8; }

hipError_t launch_decode_wide_bf16(const void* q, void* k_cache, void* v_cache,
                                   const int32_t* seq_lens, const DecodeWorkspace& ws,
                                   const DecodePlan& plan, int B, int H, int K, int S_max, int d,
                                   float scale_log2, const void* k_new, const void* v_new,
                                   const PagedArgs* paged, hipStream_t stream) {
  const dim3 grid(plan.fa.n_wg);
  auto qp = static_cast<const __bf16*>(q);
  auto kp = static_cast<__bf16*>(k_cache);
  auto vp = static_cast<__bf16*>(v_cache);
  auto kn = static_cast<const __bf16*>(k_new);
  auto vn = static_cast<const __bf16*>(v_new);
  const PagedArgs pg = paged ? *paged : PagedArgs{nullptr, 16, 0, 1};
  // one wave per 16-head block
#define GQA_WIDE(DD, AP, PG, WW)                                                                  \
  hipLaunchKernelGGL((decode_wide_bf16_kernel<DD, AP, PG, WW, kSub, kRing>), grid,               \
                     dim3(64 * WW), 0, stream, qp, kp, vp, seq_lens, ws.part_acc, ws.part_ml, B, H, K, \
                     S_max, plan.fa, scale_log2, kn, vn, ws.meta, pg)
#define GQA_WIDE_W(DD, AP, PG)                                                                   \
  switch (plan.head_blocks) {                                                                     \
    case 2: GQA_WIDE(DD, AP, PG, 2); break;                                                       \
    case 3: GQA_WIDE(DD, AP, PG, 3); break;                                                       \
    case 4: GQA_WIDE(DD, AP, PG, 4); break;                                                       \
    case 5: GQA_WIDE(DD, AP, PG, 5); break;                                                       \
    case 6: GQA_WIDE(DD, AP, PG, 6); break;                                                       \
    case 7: GQA_WIDE(DD, AP, PG, 7); break;                                                       \
    default: GQA_WIDE(DD, AP, PG, 8); break;                                                      \
  }
#define GQA_WIDE_D(DD)                                                                           \
  if (paged) {                                                                                    \
    if (k_new) { GQA_WIDE_W(DD, true, true) } else { GQA_WIDE_W(DD, false, true) }                \
  } else {                                                                                        \
    if (k_new) { GQA_WIDE_W(DD, true, false) } else { GQA_WIDE_W(DD, false, false) }              \
  }
  if (d == 128) {
    GQA_WIDE_D(128)
  } else {
    GQA_WIDE_D(64)
  }
#undef GQA_WIDE_D
#undef GQA_WIDE_W
#undef GQA_WIDE
  return hipGetLastError();
}

}  // namespace gqa
