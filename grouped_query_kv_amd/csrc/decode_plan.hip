// Split planning and workspace layout of the decode calls (host side): how
// many workgroups each partition pass runs and how the caller's workspace is
// carved.  The device side of the split is decode_flat.h.
#include <algorithm>

#include "gqa_internal.h"

namespace gqa {

namespace {

// Workgroups of each partition pass.  Every workgroup streams the same
// number of positions, so the pass takes as long as the CU with the most
// workgroups: counts are whole multiples of the 256 CUs (measured on the
// decode workloads: a count just above a multiple of 256 leaves a few CUs one
// range more and costs up to 20%).  Measured best per pass: the one-wave
// bf16 pass three workgroups per CU (2-5% ahead of four, 10% ahead of two
// and of eight); the int8 pass eight (two waves per SIMD); a multi-wave pass
// (groups of more than 16 heads, one wave per 16-head block) four; the fp32
// pass four one-wave workgroups (groups of up to 16 heads; 26% ahead of two
// at d = 128) and two multi-wave ones.
constexpr int kCUs = 256;
int target_wgs(PassKind kind, int head_blocks) {
  if (kind == PassKind::kF32) return head_blocks > 1 ? 2 * kCUs : 4 * kCUs;
  if (head_blocks > 1) return 4 * kCUs;
  return kind == PassKind::kInt8 ? 8 * kCUs : 3 * kCUs;
}
// the most workgroups any partition pass runs for these group sizes (what
// the workspace is sized for, so one size serves every decode entry point)
int max_target_wgs(int head_blocks) {
  return std::max({target_wgs(PassKind::kBf16, head_blocks), target_wgs(PassKind::kInt8, head_blocks),
                   target_wgs(PassKind::kF32, head_blocks)});
}

// Workgroups a call may need at most: the target, or more when a range is
// capped (paged: the block ids of a segment fit one per lane) -- enough that
// n_wg ranges of the capped length cover the largest possible total, still a
// multiple of the CU count.
long long needed_wgs(int B, int K, int max_seq_len, int r_max, long long target) {
  if (r_max <= 0) return target;
  const long long r = r_max / 32 * 32 - 32;  // flat_range may step 32 below the cap
  const long long tmax = (long long)K * B * pad32(max_seq_len);
  const long long n = (tmax + r - 1) / r;
  return std::max(target, (n + kCUs - 1) / kCUs * kCUs);
}

}  // namespace

DecodePlan plan_decode(int B, int H, int K, int max_seq_len, int d, PassKind kind, int r_max) {
  DecodePlan p{};
  p.G = H / K;
  p.head_blocks = (p.G + 15) / 16;
  const int eb = kind == PassKind::kF32 ? 4 : (kind == PassKind::kInt8 ? 1 : 2);
  p.fa.n_wg = (int)needed_wgs(B, K, max_seq_len, r_max, target_wgs(kind, p.head_blocks));
  p.fa.row_bytes = d * eb;
  p.fa.r_min = 32;
  p.fa.r_max = r_max > 0 ? r_max / 32 * 32 : (1 << 30);
  p.fa.max_len = max_seq_len;
  p.slots = needed_wgs(B, K, max_seq_len, r_max, max_target_wgs(p.head_blocks)) + (long long)B * K;
  return p;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t workspace_bytes_for(const DecodePlan& p, int B, int K, int d) {
  const size_t rows = (size_t)p.slots * p.G;
  return align256(rows * d * sizeof(float)) + align256(rows * 2 * sizeof(float)) +
         align256((size_t)(2 * B + 1) * sizeof(int32_t));
}

size_t decode_workspace_bytes(int B, int H, int K, int max_seq_len, int d, int r_max) {
  const DecodePlan p = plan_decode(B, H, K, max_seq_len, d, PassKind::kBf16, r_max);
  return workspace_bytes_for(p, B, K, d);
}

DecodeWorkspace carve_decode_workspace(void* base, const DecodePlan& p, int B, int K, int d) {
  const size_t rows = (size_t)p.slots * p.G;
  char* c = static_cast<char*>(base);
  DecodeWorkspace w;
  w.part_acc = reinterpret_cast<float*>(c);
  c += align256(rows * d * sizeof(float));
  w.part_ml = reinterpret_cast<float*>(c);
  c += align256(rows * 2 * sizeof(float));
  w.meta = reinterpret_cast<int32_t*>(c);
  return w;
}

}  // namespace gqa
