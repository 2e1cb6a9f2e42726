// Decode partition pass for fp32 caches, on the gfx950 matrix cores in fp32.
//
// Same contract as the bf16 passes (decode_bf16.hip, decode_wide_bf16.hip):
// for partition [t0, t1) of sequence b and KV head k it produces, for every
// query head of the group, the base-2 online-softmax state (m, l, acc) that
// the combine pass merges.  Everything stays in single precision:
// v_mfma_f32_16x16x4_f32 multiplies fp32 operands and accumulates in fp32
// (on this GPU its error over a 128-term dot product equals that of a chain
// of fp32 fma instructions), and the softmax weights are not rounded.
//
// Structure (that of the multi-wave bf16 pass): one workgroup of W waves per
// flat range (decode_flat.h), one wave per 16-head block of the group (up to
// 8 blocks; larger groups take several workgroups per range, each re-reading
// the range), so the K and V rows of the range are read from memory once for
// all heads of the group (pinghaoyang.com.cn "GQA 完全拆解", section 工程实现:
// the group's KV block is loaded once and reused by its query heads).  Rows
// are staged in chunks of CH positions (16 at d = 128, 32 at d = 64) through a
// two-buffer LDS ring filled by direct global-to-LDS copies
// (global_load_lds_dwordx4; non-temporal in one-wave workgroups); per chunk
// and wave:
//   S^T[CH x 16] = K_chunk . Q^T   (CH/16 16-position tiles, D/4 products each)
//   lazy base-2 online softmax of head n over the chunk (fp32 weights)
//   O[16 x D]   += P . V_chunk     (D/16 tiles, 8 products each)
//
// Operand layouts of v_mfma_f32_16x16x4_f32 (wave64, lane l, n = l % 16,
// g = l / 16): A row m = n holds one k-value chosen by g; B column n holds
// the same k-value; C/D lane l holds D[4g + i][n], i = 0..3.  As in the bf16
// passes the contraction index is relabelled on both sides alike:
//   Q.K: product (j, c) of a tile gives lane (n, g) head dimension
//        16j + 4g + c, so one 16-byte LDS read of a K row feeds four products
//        and the queries sit in registers as matching float4s;
//   P.V: the scores come out as lane (n = head, g) holding positions
//        16mt + 4g + i, which become that lane's contraction slots (product
//        (mt, i)), so P needs no data movement; V[16mt + 4g + i][16t + n]
//        is one 4-byte LDS read per product.
// LDS rows are whole rows of D floats, 16-byte chunks XOR-swizzled by row:
// K: chunk ^ (row % 16) puts the 16 rows of a K read in 16 distinct bank
// groups; V: chunk ^ 4 ((row / 4) % 4) puts the four rows of a V read (rows
// 4g + i for the four lane groups) in four distinct 64-byte bank ranges.
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kHB = 16;      // heads per block (one wave)
constexpr int kMaxW = 8;     // head blocks (waves) per workgroup
// cache policy of the copies: non-temporal (the nt bit of the instruction's
// cache-policy field; each cache byte is read once per step) for one-wave
// workgroups, which stream at the rate of HBM (10% faster on an fp32
// Llama-3-8B-shaped layer), the default for multi-wave ones, which are bound
// by their products (2-5% faster without it on multi-query layers)
constexpr int kStreamAuxOneWave = 2;

// s_waitcnt immediate (gfx9 encoding): vector-memory count 0, LDS count 0
constexpr int kWaitAll = 0x0070;

// CH: positions per chunk (16 or 32)
template <int D, bool APPEND, int W, int CH>
__global__ __launch_bounds__(64 * W) void decode_split_f32_kernel(
    const float* __restrict__ q, float* __restrict__ kc, float* __restrict__ vc,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part_acc,
    float* __restrict__ part_ml, int B, int H, int K, int S_max, FlatArgs fa, int wg_per_range,
    float scale_log2, const float* __restrict__ k_new, const float* __restrict__ v_new,
    int32_t* __restrict__ meta) {
  static_assert(D == 64 || D == 128, "head dimension");
  static_assert(CH == 16 || CH == 32, "chunk length");
  constexpr int kChunk = CH;
  constexpr int MT = CH / 16;                // 16-position score tiles per chunk
  constexpr int CPR = D / 4;                 // 16-byte chunks per row
  constexpr int TILE = kChunk * D;           // floats per staged tensor
  constexpr int NINST = TILE / 256;          // 1 KB copies per tensor and chunk
  constexpr int NI = (NINST + W - 1) / W;    // copies per wave per tensor and chunk
  constexpr int DJ = D / 16;                 // float4 query pieces per lane
  constexpr int NTILES = D / 16;             // 16-dim output tiles

  __shared__ __attribute__((aligned(16))) float lds[2][2][TILE];  // [buffer][K|V]

  const int w = blockIdx.x / wg_per_range;
  const int hg = blockIdx.x - w * wg_per_range;  // this workgroup's group of head blocks
  const int G = H / K;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int hb = hg * kMaxW + wave;              // this wave's block of 16 heads
  const bool has_heads = hb * kHB < G;           // wave-uniform

  // lengths clamped into [0, S_max], so no length can make a load leave the cache
  auto len_in = [&](int bb) -> int { return min(max(seq_lens[bb], 0), S_max); };
  auto len_of = [&](int bb) -> int {
    const int L_in = len_in(bb);
    return min(APPEND && L_in < S_max ? L_in + 1 : L_in, fa.max_len);
  };
  // the lengths attended over and the split, for the combine pass
  const int l0 = first_lengths(B, len_of);  // lengths of sequences 0..63, one per lane
  if (blockIdx.x == 0 && wave == 0) flat_publish(B, K, l0, len_of, meta);
  const int total = flat_total(B, K, l0, len_of);
  const int R = flat_range(total, fa);

  flat_for_each_segment(w, B, K, total, R, l0, len_of,
                        [&](int b, int k, int t0, int t1, int L, int slot) {
  const int newpos = APPEND && L > len_in(b) ? L - 1 : -1;  // the appended row, if any
  const int last = t1 - 1;
  const size_t head_base = ((size_t)b * K + k) * (size_t)S_max * D;
  float* kbase = kc + head_base;
  float* vbase = vc + head_base;

  // The fused append: the workgroup(s) whose partition holds the appended
  // position write the new rows into the cache before anything is copied
  // (every workgroup of the range writes the same values), so the copies
  // read the cache alone; wave 0 waits for its stores to complete
  // (vmcnt(0): a workgroup-scope release alone compiles to no wait here)
  // before the barrier, so no other wave's copy of the row can overtake them.
  if (APPEND && newpos >= t0 && newpos < t1) {  // uniform
    if (wave == 0 && lane < CPR) {
      const float* kn = k_new + ((size_t)b * K + k) * D;
      const float* vn = v_new + ((size_t)b * K + k) * D;
      *reinterpret_cast<f32x4*>(kbase + (size_t)newpos * D + 4 * lane) =
          *reinterpret_cast<const f32x4*>(kn + 4 * lane);
      *reinterpret_cast<f32x4*>(vbase + (size_t)newpos * D + 4 * lane) =
          *reinterpret_cast<const f32x4*>(vn + 4 * lane);
    }
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }

  // queries of head hb*16 + n as float4 pieces 16j + 4g .. +3 (zeros past the group)
  const int hq = hb * kHB + n;
  const bool hq_ok = hq < G;
  f32x4 qf[DJ];
  {
    const float* qrow = q + ((size_t)b * H + (size_t)k * G + (hq_ok ? hq : 0)) * D;
#pragma unroll
    for (int j = 0; j < DJ; ++j)
      qf[j] = hq_ok ? *reinterpret_cast<const f32x4*>(qrow + 16 * j + 4 * g) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Copy slot c of this wave is instruction i = wave + c W of the chunk
  // (slots past the last instruction, i >= NINST, issue nothing): lane l fills LDS chunk 64 i + l = row r, physical chunk l % CPR, with the
  // logical chunk the swizzle puts there (ck, cv: its byte offset in the row).
  // Rows past the partition end are fetched from its last row (valid memory;
  // their scores are masked).
  int crow[NI];
  uint32_t ck[NI], cv[NI];
#pragma unroll
  for (int c = 0; c < NI; ++c) {
    const int i = (wave + c * W) % NINST;
    const int r = (64 * i + lane) / CPR, ph = lane % CPR;
    crow[c] = r;
    ck[c] = 16 * (ph ^ (r & 15));
    cv[c] = 16 * (ph ^ (((r >> 2) & 3) << 2));
  }
  constexpr int kAux = W == 1 ? kStreamAuxOneWave : 0;
  auto copy_chunk = [&](int c0, int buf) {
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      const int i = wave + c * W;  // uniform
      if (i >= NINST) continue;
      // the chunk's first row (uniform) plus a small per-lane offset
      const uint32_t ro = (uint32_t)min(crow[c], last - c0) * (uint32_t)(4 * D);
      const char* kp = reinterpret_cast<const char*>(kbase + (size_t)c0 * D) + (ro + ck[c]);
      const char* vp = reinterpret_cast<const char*>(vbase + (size_t)c0 * D) + (ro + cv[c]);
      float* kd = &lds[buf][0][i * 256];
      float* vd = &lds[buf][1][i * 256];
      __builtin_amdgcn_global_load_lds(kp, (__attribute__((address_space(3))) void*)kd, 16, 0, kAux);
      __builtin_amdgcn_global_load_lds(vp, (__attribute__((address_space(3))) void*)vd, 16, 0, kAux);
    }
  };

  // loop-invariant LDS offsets (floats): K piece j of tile mt is row 16mt + n,
  // logical chunk 4j + g; V read of product (mt, i), tile t is row
  // 16mt + 4g + i, logical chunk 4t + n/4, float n % 4
  int ka_off[DJ];
#pragma unroll
  for (int j = 0; j < DJ; ++j) ka_off[j] = n * D + 4 * ((4 * j + g) ^ n);
  const int vswz = g << 2;  // ((row / 4) % 4) << 2 for rows 16mt + 4g + i
  int vb_off[NTILES];
#pragma unroll
  for (int t = 0; t < NTILES; ++t) vb_off[t] = 4 * g * D + 4 * ((4 * t + (n >> 2)) ^ vswz) + (n & 3);

  float m_run = -INFINITY;  // running max of head n (replicated over g)
  float l_run = 0.f;        // this lane's share of the running sum of head n
  f32x4 acc[NTILES];
#pragma unroll
  for (int t = 0; t < NTILES; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // A head's running max is raised (and its accumulators rescaled) only when
  // some score of the chunk exceeds it by more than 2^kLazy; otherwise the
  // stale max stays and numerator and denominator share it.
  constexpr float kLazy = 8.f;

  auto compute_chunk = [&](int c0, int buf) {
    const float* kt = lds[buf][0];
    const float* vt = lds[buf][1];
    // ---- S^T = K . Q^T (raw q.k) ----
    f32x4 st[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < DJ; ++j) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(&kt[16 * mt * D + ka_off[j]]);
#pragma unroll
        for (int c = 0; c < 4; ++c)
          st[mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c], qf[j][c], st[mt], 0, 0, 0);
      }
    }
    // positions past the segment (only in its last chunk) get -inf
    if (c0 + kChunk > t1) {  // uniform
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (c0 + 16 * mt + 4 * g + i >= t1) st[mt][i] = -INFINITY;
    }
    // ---- lazy online softmax for head n over positions {16mt + 4g + i} ----
    // scale > 0: the largest scaled score is the largest raw score times the scale
    float lmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
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
    float p[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[mt][i] = fast_exp2(fmaf(st[mt][i], scale_log2, mneg));
        l_run += p[mt][i];
      }
    // ---- O += P . V ----
#pragma unroll
    for (int t = 0; t < NTILES; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[mt][i], vt[vb_off[t] + (16 * mt + i) * D], acc[t],
                                                        0, 0, 0);
  };

  // ---- the ring: one chunk in flight while the previous one is multiplied ----
  const int nchunk = (t1 - t0 + kChunk - 1) / kChunk;
  copy_chunk(t0, 0);
  for (int j = 0; j < nchunk; ++j) {
    // this wave's copies of chunk j have landed; after the barrier every
    // wave's have, and every wave is done reading chunk j-1 (whose buffer is
    // refilled next).  A bare s_barrier: a fence would also wait for the
    // copies of chunk j+1 issued after it.
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (j + 1 < nchunk) copy_chunk(t0 + (j + 1) * kChunk, (j + 1) & 1);
    if (has_heads) compute_chunk(t0 + j * kChunk, j & 1);
  }

  if (has_heads) {
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    const size_t row0 = (size_t)slot * G + (size_t)hb * kHB;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hl = 4 * g + i;
      if (hb * kHB + hl < G) {
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
  }
  // every wave is done with the ring before the next segment refills it
  __syncthreads();
                        });
}

}  // namespace

hipError_t launch_decode_split_f32(const void* q, void* k_cache, void* v_cache,
                                   const int32_t* seq_lens, const DecodeWorkspace& ws,
                                   const DecodePlan& plan, int B, int H, int K, int S_max, int d,
                                   float scale_log2, const void* k_new, const void* v_new,
                                   hipStream_t stream) {
  // one wave per 16-head block, at most kMaxW per workgroup
  const int wg_per_range = (plan.head_blocks + kMaxW - 1) / kMaxW;
  const int W = plan.head_blocks < kMaxW ? plan.head_blocks : kMaxW;
  const dim3 grid(plan.fa.n_wg * wg_per_range);
  auto qp = static_cast<const float*>(q);
  auto kp = static_cast<float*>(k_cache);
  auto vp = static_cast<float*>(v_cache);
  auto kn = static_cast<const float*>(k_new);
  auto vn = static_cast<const float*>(v_new);
  const bool app = k_new != nullptr;
// chunks of 16 positions at d = 128 (32 KB of LDS per workgroup), 32 at d = 64
#define GQA_F32(DD, AP, WW)                                                                        \
  hipLaunchKernelGGL((decode_split_f32_kernel<DD, AP, WW, DD == 128 ? 16 : 32>), grid, dim3(64 * WW),  \
                     0, stream, qp, kp, vp, seq_lens, ws.part_acc, ws.part_ml, B, H, K, S_max, plan.fa, \
                     wg_per_range, scale_log2, kn, vn, ws.meta)
#define GQA_F32_W(DD, AP)                                                                         \
  switch (W) {                                                                                    \
    case 1: GQA_F32(DD, AP, 1); break;                                                            \
    case 2: GQA_F32(DD, AP, 2); break;                                                            \
    case 3: GQA_F32(DD, AP, 3); break;                                                            \
    case 4: GQA_F32(DD, AP, 4); break;                                                            \
    case 5: GQA_F32(DD, AP, 5); break;                                                            \
    case 6: GQA_F32(DD, AP, 6); break;                                                            \
    case 7: GQA_F32(DD, AP, 7); break;                                                            \
    default: GQA_F32(DD, AP, 8); break;                                                           \
  }
  if (d == 128) {
    if (app) { GQA_F32_W(128, true) } else { GQA_F32_W(128, false) }
  } else {
    if (app) { GQA_F32_W(64, true) } else { GQA_F32_W(64, false) }
  }
#undef GQA_F32_W
#undef GQA_F32
  return hipGetLastError();
}

}  // namespace gqa
