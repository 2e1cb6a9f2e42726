// Decode partition pass over an int8 KV cache, on the gfx950 matrix cores.
//
// The cache holds int8 codes c and one fp32 scale per row (sequence, KV
// head, position); a row reads back as c * scale (the quantisation rule is
// in quant_int8.hip).  pinghaoyang.com.cn "GQA 完全拆解": quantising the KV
// cache is orthogonal to GQA and multiplies its savings; aicoding.csdn.net
// "LLaMa3与DeepSeek采用的GQA技术", section 3: 8-bit caches halve the bytes.
// Decode is bound by those bytes, so this pass reads 2 * (d + 4) bytes per
// position and KV head instead of 4 * d.
//
// It computes the same partial online-softmax state as the bf16 pass
// (decode_bf16.hip, where the algorithm and the operand layouts of
// v_mfma_f32_16x16x32_bf16 are described), with the scales moved out of the
// products:
//     s_j  = scale * (q . c^K_j) * sk_j                   (score of position j)
//     acc += sum_j 2^(s_j - m) * sv_j * c^V_j,   l += sum_j 2^(s_j - m)
// Codes of magnitude <= 127 are exact in bf16, so the matrix cores multiply
// the bf16 query by the codes converted in registers; the value scale is
// folded into the bf16 softmax weight of each position.
//
// Layouts: K rows go straight from HBM into operand registers.  Lane (n, g)
// at k-step s carries head dimensions (d/4) g + 8 s .. +7 (a relabelling of
// the contraction index applied to Q and K alike), so each lane reads one
// contiguous d/4-byte piece of its K row.  V codes are converted to bf16 on
// the way into LDS and read back transposed exactly as in the bf16 pass.
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kChunk = 32;
constexpr int kVPad = 16;

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) void*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(uint2, r);
}

// Four int8 codes (one dword, little-endian) -> four bf16 values (exact).
__device__ __forceinline__ uint2 i8x4_to_bf16x4(uint32_t w) {
  const float f0 = (float)((int32_t)(w << 24) >> 24);
  const float f1 = (float)((int32_t)(w << 16) >> 24);
  const float f2 = (float)((int32_t)(w << 8) >> 24);
  const float f3 = (float)((int32_t)w >> 24);
  return uint2{pack_bf16x2(f0, f1), pack_bf16x2(f2, f3)};
}

// Eight codes (two dwords) -> one bf16x8 operand.
__device__ __forceinline__ bf16x8 i8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  const uint2 a = i8x4_to_bf16x4(lo);
  const uint2 b = i8x4_to_bf16x4(hi);
  return as_bf16x8(u32x4{a.x, a.y, b.x, b.y});
}

// The 16 values of a row of 16 lanes, lane j's value to every lane of the
// row (v_mov_b32 DPP row_newbcast:j): lo[j] for j < 8, hi[j - 8] after.
template <int J>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + J, 0xF, 0xF, false));
}
__device__ __forceinline__ void row_bcast8(float x, float (&lo)[8], float (&hi)[8]) {
  lo[0] = row_bcast<0>(x);  lo[1] = row_bcast<1>(x);  lo[2] = row_bcast<2>(x);  lo[3] = row_bcast<3>(x);
  lo[4] = row_bcast<4>(x);  lo[5] = row_bcast<5>(x);  lo[6] = row_bcast<6>(x);  lo[7] = row_bcast<7>(x);
  hi[0] = row_bcast<8>(x);  hi[1] = row_bcast<9>(x);  hi[2] = row_bcast<10>(x); hi[3] = row_bcast<11>(x);
  hi[4] = row_bcast<12>(x); hi[5] = row_bcast<13>(x); hi[6] = row_bcast<14>(x); hi[7] = row_bcast<15>(x);
}

// Two resident waves per SIMD (at most 256 registers, no spills): the flat
// split runs eight workgroups per CU (the in-flight K/V chunk of a wave is
// half the bytes of the bf16 pass, so more waves than the bf16 pass's three
// per CU are needed to keep the same bytes in flight; measured on the
// Llama-3-8B layer: eight per CU 54.5 us, six 60.8 us, twelve 60.8 us).
//
// APPEND: the quantising append fused in.  The step's new rows k_new, v_new
// (bf16) belong at position L_in = seq_lens[b] when the cache has room; it is
// the last position of the sequence, so only the segment that ends the
// sequence reads that cache row.  Before its first load that segment's
// workgroup quantises the rows by the cache rule (the same fp32 operations
// as the standalone append, so the same codes and scales) straight into the
// cache row and scale, and fences so that its own loads see them.  With
// several head blocks each of their workgroups writes the same bytes before
// reading them; no other workgroup of the launch reads that row.  Workgroup
// 0 records the lengths after the append with the split (decode_flat.h) for
// the combine pass.
template <int D, bool APPEND>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_split_int8_kernel(
    const __bf16* __restrict__ q, int8_t* __restrict__ kc, int8_t* __restrict__ vc,
    float* __restrict__ ks, float* __restrict__ vs, const int32_t* __restrict__ seq_lens,
    float* __restrict__ part_acc, float* __restrict__ part_ml, int B, int H, int K, int S_max,
    FlatArgs fa, int head_blocks, float scale_log2, const __bf16* __restrict__ k_new,
    const __bf16* __restrict__ v_new, int32_t* __restrict__ meta) {
  static_assert(D == 64 || D == 128, "head dimension");
  constexpr int KSTEPS = D / 32;
  constexpr int NTILES = D / 16;
  constexpr int KSEG = D / 4;                 // bytes of a K row per lane
  constexpr int KWORDS = KSEG / 16;           // 16-byte loads per K row piece
  constexpr int LANES_PER_ROW = D / 16;       // 16-byte words per V row
  constexpr int ROWS_PER_LOAD = 64 / LANES_PER_ROW;
  constexpr int VLOADS = kChunk / ROWS_PER_LOAD;
  constexpr int LDS_ROW = D + kVPad;

  __shared__ __attribute__((aligned(16))) uint16_t vt[kChunk * LDS_ROW];

  // head block hb of flat range w (decode_flat.h; several head blocks only
  // for groups of more than 128 heads)
  const int w = blockIdx.x / head_blocks;
  const int hb = blockIdx.x - w * head_blocks;
  const int G = H / K;
  // length attended over: after the fused append when the cache has room
  // lengths clamped into [0, S_max], so no length can make a load leave the cache
  auto len_in = [&](int bb) -> int { return min(max(seq_lens[bb], 0), S_max); };
  auto len_of = [&](int bb) -> int {
    const int L_in = len_in(bb);
    return min(APPEND && L_in < S_max ? L_in + 1 : L_in, fa.max_len);
  };
  // the lengths attended over and the split, for the combine pass
  const int l0 = first_lengths(B, len_of);  // lengths of sequences 0..63, one per lane
  if (blockIdx.x == 0) flat_publish(B, K, l0, len_of, meta);
  const int total = flat_total(B, K, l0, len_of);
  const int R = flat_range(total, fa);

  flat_for_each_segment(w, B, K, total, R, l0, len_of,
                        [&](int b, int k, int t0, int t1, int L, int slot_id) {
  const int newpos = APPEND && L > len_in(b) ? L - 1 : -1;  // the appended row, if any
  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int g = lane >> 4;

  const int hq = hb * 16 + n;
  const bool hq_ok = hq < G;
  bf16x8 qf[KSTEPS];
  {
    const __bf16* qrow = q + ((size_t)b * H + (size_t)k * G + (hq_ok ? hq : 0)) * D + KSEG * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = as_bf16x8(hq_ok ? ld16(qrow + 8 * s) : zero_u32x4());
  }

  const size_t head_row0 = ((size_t)b * K + k) * (size_t)S_max;  // first row of (b, k)
  int8_t* kbase = kc + head_row0 * D;
  int8_t* vbase = vc + head_row0 * D;
  float* ksb = ks + head_row0;
  float* vsb = vs + head_row0;

  // The new rows of the fused append, quantised into the cache before any load.
  const bool has_new = APPEND && newpos >= t0 && newpos < t1;  // wave-uniform
  if (has_new) {
    constexpr int E = D / 64;  // elements per lane
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
      int8_t* dst = (r == 0 ? kbase : vbase) + (size_t)newpos * D + E * lane;
#pragma unroll
      for (int e = 0; e < E; ++e) dst[e] = amax > 0.f ? (int8_t)int8_code(x[e], inv) : 0;
      if (lane == 0) (r == 0 ? ksb : vsb)[newpos] = amax > 0.f ? int8_scale(amax) : 0.f;
    }
    // this workgroup's loads below see the stores (workgroup scope: the same
    // wave writes and reads; an agent-scope fence would write back and
    // invalidate the L2 in every segment that ends a sequence)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 acc[NTILES];
#pragma unroll
  for (int t = 0; t < NTILES; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int vrow = lane / LANES_PER_ROW;
  const int vcol = (lane % LANES_PER_ROW) * 16;
  const uint16_t* tr_src = &vt[(4 * g + (n >> 2)) * LDS_ROW + 4 * (n & 3)];

  u32x4 ka[2][KWORDS];
  u32x4 vr[VLOADS];
  // Scales: one dword per lane per chunk.  Row g of the wave (lanes 16 g ..
  // 16 g + 15; its lanes' scores are positions 16 mt + 4 g + i, i < 4) fetches
  // the 16 scales the row needs -- lane j: tensor j / 8 (K, then V), tile
  // (j / 4) % 2, position i = j % 4 -- and each lane takes its own from the
  // row by broadcasts (DPP row_newbcast).  A chunk's scale traffic is then
  // 256 bytes per wave instead of sixteen copies of every 16-byte group.
  float scl;
  // Rows past the partition are fetched from its last row instead (valid
  // memory, finite codes; their scores and weights are masked below), so no
  // load is predicated.
  const int last = t1 - 1;
  const float* sc_src = n < 8 ? ksb : vsb;
  const int sc_off = 16 * ((n >> 2) & 1) + 4 * g + (n & 3);
  auto load_k = [&](int c0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int tok = min(c0 + 16 * mt + n, last);
      const int8_t* krow = kbase + (size_t)tok * D + KSEG * g;
#pragma unroll
      for (int w = 0; w < KWORDS; ++w) ka[mt][w] = ld16_stream(krow + 16 * w);
    }
    scl = sc_src[min(c0 + sc_off, last)];
  };
  auto load_v = [&](int c0) {
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int tok = min(c0 + i * ROWS_PER_LOAD + vrow, last);
      vr[i] = ld16_stream(vbase + (size_t)tok * D + vcol);
    }
  };
  // A head's running max is raised (and its accumulators rescaled) only
  // when some score of the chunk exceeds it by more than 2^kLazy; otherwise
  // the stale max stays, the weights stay below 2^kLazy, and numerator and
  // denominator share it (the combine pass takes any max).  l_run holds this
  // lane's share of the denominator (its positions); the shares are summed
  // over the lane groups once, after the loop.
  constexpr float kLazy = 8.f;
  load_k(t0);
  load_v(t0);

  for (int c0 = t0; c0 < t1; c0 += kChunk) {
    const bool more = c0 + kChunk < t1;
    // ---- S^T = K . Q^T (codes) for the two 16-position tiles ----
    f32x4 st[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      st[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const u32x4 w = ka[mt][s / 2];
        const bf16x8 kf = (s & 1) ? i8x8_to_bf16x8(w[2], w[3]) : i8x8_to_bf16x8(w[0], w[1]);
        st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], st[mt], 0, 0, 0);
      }
    }
    float sk[8], sv[8];
    row_bcast8(scl, sk, sv);
    if (more) load_k(c0 + kChunk);

    // ---- online softmax for head n over positions {16mt + 4g + i} ----
    float x[8];
    float lmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * mt + i] = st[mt][i] * (sk[4 * mt + i] * scale_log2);
    if (c0 + kChunk > t1) {  // uniform: positions past the segment, only in its last chunk
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c0 + 16 * (j >> 2) + 4 * g + (j & 3) >= t1) {
          x[j] = -INFINITY;
          sv[j] = 0.f;  // rows past the end never reach the sum
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) lmax = fmaxf(lmax, x[j]);
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

    // ---- V codes -> bf16 rows in LDS, then transposed reads ----
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      uint16_t* dst = &vt[(i * ROWS_PER_LOAD + vrow) * LDS_ROW + vcol];
      const uint2 a = i8x4_to_bf16x4(vr[i][0]);
      const uint2 b2 = i8x4_to_bf16x4(vr[i][1]);
      const uint2 c = i8x4_to_bf16x4(vr[i][2]);
      const uint2 d2 = i8x4_to_bf16x4(vr[i][3]);
      *reinterpret_cast<u32x4*>(dst) = u32x4{a.x, a.y, b2.x, b2.y};
      *reinterpret_cast<u32x4*>(dst + 8) = u32x4{c.x, c.y, d2.x, d2.y};
    }
    __syncthreads();
    if (more) load_v(c0 + kChunk);
    const bf16x8 pa = as_bf16x8(u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
    for (int t = 0; t < NTILES; ++t) {
      const uint2 lo = lds_read_tr16(tr_src + 16 * t);
      const uint2 hi = lds_read_tr16(tr_src + 16 * LDS_ROW + 16 * t);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(u32x4{lo.x, lo.y, hi.x, hi.y}),
                                                       acc[t], 0, 0, 0);
    }
    __syncthreads();
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
                        });
}

}  // namespace

hipError_t launch_decode_split_int8(const void* q, void* k_codes, void* v_codes, float* k_scales,
                                    float* v_scales, const int32_t* seq_lens,
                                    const DecodeWorkspace& ws, const DecodePlan& plan, int B, int H,
                                    int K, int S_max, int d, float scale_log2, const void* k_new,
                                    const void* v_new, hipStream_t stream) {
  if (decode_wide_supported(plan.head_blocks))  // G > 16: one code read for all head blocks
    return launch_decode_wide_int8(q, k_codes, v_codes, k_scales, v_scales, seq_lens, ws, plan, B,
                                   H, K, S_max, d, scale_log2, k_new, v_new, stream);
  const dim3 grid(plan.fa.n_wg * plan.head_blocks);
  auto qp = static_cast<const __bf16*>(q);
  auto kp = static_cast<int8_t*>(k_codes);
  auto vp = static_cast<int8_t*>(v_codes);
  auto kn = static_cast<const __bf16*>(k_new);
  auto vn = static_cast<const __bf16*>(v_new);
#define GQA_I8(DD, AP)                                                                          \
  hipLaunchKernelGGL((decode_split_int8_kernel<DD, AP>), grid, dim3(64), 0, stream, qp, kp, vp,  \
                     k_scales, v_scales, seq_lens, ws.part_acc, ws.part_ml, B, H, K, S_max,      \
                     plan.fa, plan.head_blocks, scale_log2, kn, vn, ws.meta)
  if (d == 128) {
    if (k_new) GQA_I8(128, true); else GQA_I8(128, false);
  } else {
    if (k_new) GQA_I8(64, true); else GQA_I8(64, false);
  }
#undef GQA_I8
  return hipGetLastError();
}

}  // namespace gqa
