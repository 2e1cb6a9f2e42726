// Decode combine pass: merges the partitions' online-softmax states.
//
// For query head h of sequence b (KV head k = h / G), the partition pass left
// one partial state per workgroup whose flat range met pair (b, k) (the flat
// split of decode_flat.h, recomputed here from the same lengths); n such
// partials (m_p, l_p, acc_p) in base-2 units merge as
//     M = max_p m_p,  w_p = 2^(m_p - M),
//     out = (sum_p w_p acc_p) / (sum_p w_p l_p),
// which equals softmax-weighted sum over all L_b positions (the block-wise
// computation with an online softmax that the foundit.cn GQA article and
// pinghaoyang.com.cn "GQA 完全拆解" (section 质量与速度的实测权衡, on
// FlashAttention being complementary to GQA) name; the merge rule follows
// from exp(a) = exp(a - M) exp(M)).  L_b = 0 gives a zero row.
//
// One 64-thread workgroup per (b, h); lane c owns dims [c*D/64, (c+1)*D/64).
#include "common.h"
#include "gqa_internal.h"

namespace gqa {
namespace {

// The lengths come from the workspace (the partition pass recorded them with
// the split).  PUBLISH_LENS: after a fused append the (b, h = 0) workgroup
// writes them to seq_lens -- no workgroup of this pass reads seq_lens, so
// there is no race.
template <int D, bool OUT_BF16, bool PUBLISH_LENS>
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float* __restrict__ part_acc, const float* __restrict__ part_ml,
    int32_t* __restrict__ seq_lens, const int32_t* __restrict__ meta, void* __restrict__ out,
    int B, int H, int K, FlatArgs fa) {
  constexpr int PER = D / 64;  // dims per lane
  __shared__ float wsh[64];
  const int bh = blockIdx.x;
  const int b = bh / H;
  const int h = bh - b * H;
  const int G = H / K;
  const int k = h / G;
  const int lane = threadIdx.x;
  // the split the partition pass recorded: length, flat start, total (read
  // before any arithmetic on them, so that the three loads are in flight
  // together)
  const int L = meta[b];
  const int start_b = meta[B + b];
  const int total = meta[2 * B];
  const int R = flat_range(total, fa);
  const int base = start_b + k * pad32(L);  // flat start of pair (b, k)
  const int w0 = base / R;
  const int n = L > 0 ? (base + L - 1) / R - w0 + 1 : 0;  // partials of this pair
  // partial p is slot w0 + p + b K + k, row h - k G
  const size_t row = (size_t)(w0 + b * K + k) * G + (h - k * G);
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + row;
  const float* pa = part_acc + row * D + lane * PER;
  const size_t stride = (size_t)G;  // rows between consecutive slots

  // The first kEarly partitions' numerators are loaded up front, together
  // with the (max, sum) pairs, so the common case costs one memory round
  // trip after the length; any further partitions are streamed below.
  constexpr int kEarly = 32;
  float early[kEarly][PER];
#pragma unroll
  for (int p = 0; p < kEarly; ++p)
#pragma unroll
    for (int j = 0; j < PER; ++j) early[p][j] = p < n ? pa[(size_t)p * stride * D + j] : 0.f;

  // global max over the partitions (lane-parallel loads)
  float M = -INFINITY;
  for (int p = lane; p < n; p += 64) M = fmaxf(M, ml[p * stride].x);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));

  // weights of up to 64 partitions at a time, shared through LDS; every lane
  // then sums its dims over those partitions
  float num[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) num[j] = 0.f;
  float den = 0.f;
  for (int p0 = 0; p0 < n; p0 += 64) {
    const int p = p0 + lane;
    float w = 0.f;
    if (p < n) {
      const float2 x = ml[p * stride];
      w = fast_exp2(x.x - M);
      den = fmaf(w, x.y, den);
    }
    wsh[lane] = w;
    __syncthreads();
    const int cnt = min(64, n - p0);
    if (p0 == 0) {
#pragma unroll
      for (int q = 0; q < kEarly; ++q) {
        const float wq = wsh[q];  // zero beyond n
#pragma unroll
        for (int j = 0; j < PER; ++j) num[j] = fmaf(wq, early[q][j], num[j]);
      }
    }
    for (int j2 = p0 == 0 ? kEarly : 0; j2 < cnt; ++j2) {
      const float wj = wsh[j2];
      const float* src = pa + (size_t)(p0 + j2) * stride * D;
#pragma unroll
      for (int j = 0; j < PER; ++j) num[j] = fmaf(wj, src[j], num[j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
  const float inv = n > 0 ? 1.f / den : 0.f;
  if (PUBLISH_LENS && h == 0 && lane == 0) seq_lens[b] = L;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const float o = n > 0 ? num[j] * inv : 0.f;
    const size_t idx = (size_t)bh * D + lane * PER + j;
    if (OUT_BF16)
      static_cast<__bf16*>(out)[idx] = static_cast<__bf16>(o);
    else
      static_cast<float*>(out)[idx] = o;
  }
}

}  // namespace

hipError_t launch_decode_combine(const DecodeWorkspace& ws, int32_t* seq_lens, void* out,
                                 const DecodePlan& plan, int B, int H, int K, int d, bool out_bf16,
                                 bool publish_lens, hipStream_t stream) {
  const dim3 grid(B * H), block(64);
#define GQA_COMBINE(DD, OB, LW)                                                                  \
  hipLaunchKernelGGL((decode_combine_kernel<DD, OB, LW>), grid, block, 0, stream, ws.part_acc,   \
                     ws.part_ml, seq_lens, ws.meta, out, B, H, K, plan.fa)
#define GQA_COMBINE_D(DD)                                                                        \
  if (out_bf16) {                                                                                \
    if (publish_lens) GQA_COMBINE(DD, true, true); else GQA_COMBINE(DD, true, false);            \
  } else {                                                                                       \
    if (publish_lens) GQA_COMBINE(DD, false, true); else GQA_COMBINE(DD, false, false);          \
  }
  if (d == 128) {
    GQA_COMBINE_D(128)
  } else {
    GQA_COMBINE_D(64)
  }
#undef GQA_COMBINE_D
#undef GQA_COMBINE
  return hipGetLastError();
}

}  // namespace gqa
