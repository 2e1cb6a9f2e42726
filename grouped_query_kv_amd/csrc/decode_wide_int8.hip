// Decode partition pass over an int8 KV cache for groups of more than 16
// query heads.
//
// The int8 pass (decode_int8.hip) runs one wave per 16-head block of a group,
// so a group of G > 16 heads (multi-query shapes) would read every K/V code
// ceil(G / 16) times.  As in the wide bf16 pass (decode_wide_bf16.hip; the
// pages' rule that a group's shared KV block is loaded once for all of its
// heads, pinghaoyang.com.cn "GQA 完全拆解", section 工程实现), one workgroup
// with one wave per head block owns a partition of one KV head; the waves
// copy each 32-position chunk of codes and scales once into LDS, straight
// from HBM (global_load_lds_dwordx4), through a ring of two buffers, and each
// wave multiplies it with its own heads.  The arithmetic is the int8 pass's:
//     s_j  = scale * (q . c^K_j) * sk_j,
//     acc += sum_j 2^(s_j - m) * sv_j * c^V_j,   l += sum_j 2^(s_j - m),
// with codes converted to bf16 (exact; see below) and the value scale
// folded into each position's bf16 weight, and the same quantising append.
//
// Fused append: the workgroup whose partition holds the new position (the
// last position of its sequence) quantises the step's K and V rows by the
// int8 pass's fp32 rule (shared helpers) straight into the cache row and its
// two scales before its first copy; the writing wave waits for its stores
// to complete (vmcnt(0)) and a barrier follows, so the copies that stage
// that row afterwards read the new codes.  Holding the quantised row in
// registers through the loop instead (and patching it into LDS) cost the
// registers that kept four five-wave workgroups per CU resident: 124 against
// 95 us on a 71-head int8 layer at d = 64.
//
// Each chunk's codes are converted to bf16 once, by the threads of the
// workgroup together (each 16-byte piece of K or V by one thread), into bf16
// tiles in LDS laid out as in the wide bf16 pass; every wave then reads its
// operands from there exactly as that pass does (K as 16-byte operand reads,
// V with transposed ds_read_b64_tr_b16 reads), so the conversion work is not
// repeated per head block.  The 16-byte pieces of the staged int8 rows and
// the 16-byte chunks of the bf16 rows are XOR-swizzled by row (each lane
// copies the global piece that belongs in its slot).
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

// Cache policy of the global-to-LDS copies of the cache: the default.  (The
// non-temporal bit, 5-12% faster in the bf16 multi-wave pass, measured 2-4%
// slower here, before the occupancy bound below: 128 against 124.5 us on a
// 71-head int8 layer at d = 64, 80 against 78 us with 32 heads per KV head
// at d = 128.)
constexpr int kStreamAux = 0;

constexpr int kChunk = 32;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) void*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, r);
}

// Four int8 codes (one little-endian dword) -> four bf16 values (exact).
__device__ __forceinline__ uint2 codes_to_bf16x4(uint32_t w) {
  const float f0 = (float)((int32_t)(w << 24) >> 24), f1 = (float)((int32_t)(w << 16) >> 24);
  const float f2 = (float)((int32_t)(w << 8) >> 24), f3 = (float)((int32_t)w >> 24);
  return uint2{pack_bf16x2(f0, f1), pack_bf16x2(f2, f3)};
}

// bf16 V chunk swizzle, as in the wide bf16 pass
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  return D == 64 ? ((r >> 1) & 3) << 1 : (r & 7) << 1;
}

// Physical 16-byte piece of logical piece c in a staged int8 row r.
template <int D>
__device__ __forceinline__ int piece_swizzle(int r) {
  return r & (D / 16 - 1);
}

// Four workgroups per CU: from W = 5 on, the d = 64 pass is held to five
// waves per SIMD (at most 96 registers; two pointers spill outside the
// loop).  Measured on a 71-head layer at d = 64: 95 against 124 us without
// the bound.
template <int D, int W>
constexpr int wide_int8_min_waves() { return D == 64 && W >= 5 ? 5 : 1; }

template <int D, bool APPEND, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(wide_int8_min_waves<D, W>()))) void decode_wide_int8_kernel(
    const __bf16* __restrict__ q, int8_t* __restrict__ kc, int8_t* __restrict__ vc,
    float* __restrict__ ks, float* __restrict__ vs, const int32_t* __restrict__ seq_lens,
    float* __restrict__ part_acc, float* __restrict__ part_ml, int B, int H, int K, int S_max,
    FlatArgs fa, float scale_log2, const __bf16* __restrict__ k_new,
    const __bf16* __restrict__ v_new, int32_t* __restrict__ meta) {
  static_assert(D == 64 || D == 128, "head dimension");
  constexpr int KSTEPS = D / 32;
  constexpr int NTILES = D / 16;
  constexpr int LPR = D / 8;                // 16-byte chunks per bf16 row
  constexpr int CPR = D / 16;               // 16-byte pieces per code row
  constexpr int NPIECE = kChunk * CPR;      // pieces per staged code tile
  constexpr int NUNIT = 2 * NPIECE;         // conversion units: the K pieces, then the V pieces
  constexpr int NCONV = (NUNIT + 64 * W - 1) / (64 * W);  // units per thread
  static_assert(NPIECE % 64 == 0, "a wave's units are all K or all V");
  constexpr int TILE = kChunk * D;          // bytes of a staged code tile
  constexpr int NINST = TILE / 1024;        // 1 KB copies per tensor and chunk
  constexpr int NI = (NINST + W - 1) / W;   // copies per wave per tensor and chunk
  constexpr bool SURPLUS = NINST % W != 0;

  __shared__ __attribute__((aligned(16))) int8_t kq[2][TILE];
  __shared__ __attribute__((aligned(16))) int8_t vq[2][TILE];
  __shared__ __attribute__((aligned(16))) float ksc[2][kChunk];
  __shared__ __attribute__((aligned(16))) float vsc[2][kChunk];
  // the current chunk as bf16 (the wide bf16 pass's layout)
  __shared__ __attribute__((aligned(16))) uint16_t kt[kChunk * D];
  __shared__ __attribute__((aligned(16))) uint16_t vt[kChunk * D];
  // target of the surplus copies (they repeat a real copy; never read)
  __shared__ __attribute__((aligned(16))) int8_t sink[SURPLUS ? 1024 : 16];

  const int G = H / K;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int hb = wave;  // this wave's block of 16 heads

  // length attended over: after the fused append when the cache has room
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

  flat_for_each_segment(blockIdx.x, B, K, total, R, l0, len_of,
                        [&](int b, int k, int t0, int t1, int L, int slot_id) {
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

  const size_t head_row0 = ((size_t)b * K + k) * (size_t)S_max;  // first row of (b, k)
  int8_t* kbase = kc + head_row0 * D;
  int8_t* vbase = vc + head_row0 * D;
  float* ksb = ks + head_row0;
  float* vsb = vs + head_row0;

  // The fused append: the workgroup whose partition holds the new position
  // quantises the step's K and V rows (wave 0, lane l elements E l ..
  // E l + E - 1) straight into the cache row and its scale before anything
  // is copied, so every copy below reads the cache alone.  Wave 0 waits for
  // its stores to complete (vmcnt(0)) before the barrier, so no other wave's
  // copy of the row can overtake them.
  constexpr int E = D / 64;  // elements per lane
  if (APPEND && newpos >= t0 && newpos < t1) {  // uniform
    if (wave == 0) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const __bf16* src = (r == 0 ? k_new : v_new) + ((size_t)b * K + k) * D + E * lane;
        float x[E];
        float amax = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          x[e] = static_cast<float>(src[e]);
          amax = fmaxf(amax, fabsf(x[e]));
        }
#pragma unroll
        for (int o = 32; o >= 1; o /= 2) amax = fmaxf(amax, __shfl_xor(amax, o));
        const float inv = amax > 0.f ? int8_inv(amax) : 0.f;
        uint32_t w = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e)
          w |= (uint32_t)(uint8_t)(amax > 0.f ? (int8_t)int8_code(x[e], inv) : (int8_t)0) << (8 * e);
        int8_t* dst = (r == 0 ? kbase : vbase) + (size_t)newpos * D + E * lane;
        if (E == 2)
          *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
        else
          *dst = (int8_t)w;
        if (lane == 0) (r == 0 ? ksb : vsb)[newpos] = amax > 0.f ? int8_scale(amax) : 0.f;
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0): the stores are complete
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }

  // Copy slot c of this wave: instruction i = wave + c W of a chunk (surplus
  // slots, i >= NINST, repeat instruction i - NINST into the sink: skipping
  // them instead, as the bf16 and fp32 passes do, measured 25% slower here --
  // 102 against 82 us on a 71-head layer at d = 64 -- for reasons not found);
  // lane l fills LDS piece 64 i + l = row crow, physical piece l % CPR.
  int crow[NI], ckoff[NI], cvoff[NI];
#pragma unroll
  for (int c = 0; c < NI; ++c) {
    const int i = (wave + c * W) % NINST;
    const int pc = 64 * i + lane;
    crow[c] = pc / CPR;
    const int ph = pc % CPR, sw = piece_swizzle<D>(crow[c]);
    ckoff[c] = 16 * (ph ^ sw);
    cvoff[c] = 16 * (ph ^ sw);
  }
  auto copy_chunk = [&](int c0, int buf) {
#pragma unroll
    for (int c = 0; c < NI; ++c) {
      const int i = wave + c * W;  // uniform
      const int tok = min(c0 + crow[c], last);
      const int8_t* ksrc = kbase + (size_t)tok * D + ckoff[c];
      const int8_t* vsrc = vbase + (size_t)tok * D + cvoff[c];
      int8_t* kd = i < NINST ? &kq[buf][1024 * i] : sink;
      int8_t* vd = i < NINST ? &vq[buf][1024 * i] : sink;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(ksrc),
                                       (__attribute__((address_space(3))) void*)kd, 16, 0, kStreamAux);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(vsrc),
                                       (__attribute__((address_space(3))) void*)vd, 16, 0, kStreamAux);
    }
    // scales: lanes 0..7 of waves 0 (K) and 1 (V) copy the chunk's 32 scales,
    // 4 per lane (groups past the partition end repeat its last group; S_max
    // is a multiple of 4, so a group never leaves the cache)
    if (wave < 2 && lane < kChunk / 4) {
      const int s0 = min(c0 + 4 * lane, last & ~3);
      const float* src = (wave == 0 ? ksb : vsb) + s0;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src),
                                       (__attribute__((address_space(3))) void*)(wave == 0 ? ksc[buf] : vsc[buf]),
                                       16, 0, kStreamAux);
    }
  };

  // conversion share of this thread: unit u = tid + 64 W i, the staged K
  // piece u (u < NPIECE) or V piece u - NPIECE (row pc / CPR, logical piece
  // pc % CPR) -> bf16 chunks 2 lp, 2 lp + 1.  Each unit is converted by one
  // thread; threads past the last unit (whole waves) convert nothing.
  int cv_src[NCONV], cv_dst[NCONV];
  bool cv_isv[NCONV], cv_on[NCONV];  // wave-uniform
#pragma unroll
  for (int i = 0; i < NCONV; ++i) {
    const int u = (int)threadIdx.x + 64 * W * i;
    cv_on[i] = u < NUNIT;
    const int uu = min(u, NUNIT - 1);
    cv_isv[i] = uu >= NPIECE;
    const int pc = cv_isv[i] ? uu - NPIECE : uu;
    const int r = pc / CPR, lp = pc % CPR;
    cv_src[i] = r * D + 16 * (lp ^ piece_swizzle<D>(r));
    // chunk 2 lp; chunk 2 lp + 1 is its neighbour ^ 1
    cv_dst[i] = r * D + 8 * ((2 * lp) ^ (cv_isv[i] ? v_swizzle<D>(r) : (r & (LPR - 1))));
  }
  auto convert = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NCONV; ++i) {
      if (!cv_on[i]) continue;  // uniform
      const u32x4 c = *reinterpret_cast<const u32x4*>(&(cv_isv[i] ? vq : kq)[buf][cv_src[i]]);
      const uint2 w0 = codes_to_bf16x4(c[0]), w1 = codes_to_bf16x4(c[1]);
      const uint2 w2 = codes_to_bf16x4(c[2]), w3 = codes_to_bf16x4(c[3]);
      // chunk 2lp ^ s lands at s, chunk 2lp+1 at s ^ 8 elements (the swizzle
      // flips whole 16-byte chunks and keeps pairs (2c, 2c+1) together)
      uint16_t* dst = cv_isv[i] ? vt : kt;
      *reinterpret_cast<u32x4*>(&dst[cv_dst[i]]) = u32x4{w0.x, w0.y, w1.x, w1.y};
      *reinterpret_cast<u32x4*>(&dst[cv_dst[i] ^ 8]) = u32x4{w2.x, w2.y, w3.x, w3.y};
    }
  };
  // bf16 operand offsets, as in the wide bf16 pass
  int ka_off[KSTEPS], vb_off[NTILES];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) ka_off[s] = n * D + (((4 * s + g) ^ (n & (LPR - 1))) * 8);
  {
    const int tr_row = 4 * g + (n >> 2);
    const int swz = v_swizzle<D>(tr_row);
#pragma unroll
    for (int t = 0; t < NTILES; ++t)
      vb_off[t] = tr_row * D + (((2 * t + ((n & 3) >> 1)) ^ swz) * 8) + 4 * (n & 1);
  }

  float m_run = -INFINITY;
  float l_run = 0.f;  // this lane's share of head n's denominator
  f32x4 acc[NTILES];
#pragma unroll
  for (int t = 0; t < NTILES; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr float kLazy = 8.f;  // see the bf16 pass: lazy running max

  copy_chunk(t0, 0);
  int buf = 0;
  for (int c0 = t0; c0 < t1; c0 += kChunk, buf ^= 1) {
    // this wave's copies of the chunk have landed; after the barrier every
    // wave's have, and every wave is done with the other buffer
    __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0), lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (c0 + kChunk < t1) copy_chunk(c0 + kChunk, buf ^ 1);
    convert(buf);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this thread's bf16 stores are done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();        // the bf16 tiles are complete
    asm volatile("" ::: "memory");

    // ---- S^T = K . Q^T (bf16 operands from LDS) ----
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
    float x[8], sv[8];
    float lmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const f32x4 skv = *reinterpret_cast<const f32x4*>(&ksc[buf][16 * mt + 4 * g]);
      const f32x4 svv = *reinterpret_cast<const f32x4*>(&vsc[buf][16 * mt + 4 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = c0 + 16 * mt + 4 * g + i < t1;
        const float xv = ok ? st[mt][i] * (skv[i] * scale_log2) : -INFINITY;
        x[4 * mt + i] = xv;
        sv[4 * mt + i] = ok ? svv[i] : 0.f;  // rows past the end never reach the sum
        lmax = fmaxf(lmax, xv);
      }
    }
    if (__any(lmax > m_run + kLazy)) {
      float cmax = fmaxf(lmax, __shfl_xor(lmax, 16));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
      const float m_new = fmaxf(m_run, cmax);
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
    uint32_t pw[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const float e0 = fast_exp2(x[j] - m_run);
      const float e1 = fast_exp2(x[j + 1] - m_run);
      l_run += e0 + e1;
      pw[j / 2] = pack_bf16x2(e0 * sv[j], e1 * sv[j + 1]);
    }
    // ---- O += P . V (bf16 V read transposed from LDS) ----
    const bf16x8 pa = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
    for (int t = 0; t < NTILES; ++t) {
      const uint2 lo = lds_read_tr16(vt + vb_off[t]);
      const uint2 hi = lds_read_tr16(vt + vb_off[t] + 16 * D);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y}),
                                                       acc[t], 0, 0, 0);
    }
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  const size_t row0 = (size_t)slot_id * G + (size_t)hb * 16;
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
  // every wave is done with the ring and the bf16 tiles before the next
  // segment refills them
  __syncthreads();
                        });
}

}  // namespace

hipError_t launch_decode_wide_int8(const void* q, void* k_codes, void* v_codes, float* k_scales,
                                   float* v_scales, const int32_t* seq_lens,
                                   const DecodeWorkspace& ws, const DecodePlan& plan, int B, int H,
                                   int K, int S_max, int d, float scale_log2, const void* k_new,
                                   const void* v_new, hipStream_t stream) {
  const dim3 grid(plan.fa.n_wg);
  auto qp = static_cast<const __bf16*>(q);
  auto kp = static_cast<int8_t*>(k_codes);
  auto vp = static_cast<int8_t*>(v_codes);
  auto kn = static_cast<const __bf16*>(k_new);
  auto vn = static_cast<const __bf16*>(v_new);
#define GQA_WI8(DD, AP, WW)                                                                      \
  hipLaunchKernelGGL((decode_wide_int8_kernel<DD, AP, WW>), grid, dim3(64 * WW), 0, stream, qp,  \
                     kp, vp, k_scales, v_scales, seq_lens, ws.part_acc, ws.part_ml, B, H, K,     \
                     S_max, plan.fa, scale_log2, kn, vn, ws.meta)
#define GQA_WI8_W(DD, AP)                                                                        \
  switch (plan.head_blocks) {                                                                     \
    case 2: GQA_WI8(DD, AP, 2); break;                                                            \
    case 3: GQA_WI8(DD, AP, 3); break;                                                            \
    case 4: GQA_WI8(DD, AP, 4); break;                                                            \
    case 5: GQA_WI8(DD, AP, 5); break;                                                            \
    case 6: GQA_WI8(DD, AP, 6); break;                                                            \
    case 7: GQA_WI8(DD, AP, 7); break;                                                            \
    default: GQA_WI8(DD, AP, 8); break;                                                           \
  }
  if (d == 128) {
    if (k_new) { GQA_WI8_W(128, true) } else { GQA_WI8_W(128, false) }
  } else {
    if (k_new) { GQA_WI8_W(64, true) } else { GQA_WI8_W(64, false) }
  }
#undef GQA_WI8_W
#undef GQA_WI8
  return hipGetLastError();
}

}  // namespace gqa
