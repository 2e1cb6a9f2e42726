// Flat work split of a decode call, shared by every partition pass and the
// combine pass.
//
// The cached positions of all (sequence b, KV head k) pairs are laid end to
// end in the order (b, k, position), each pair's run padded to a multiple of
// 32 positions: with Lp_b = pad32(L_b) (L_b the length the pass attends
// over, after a fused append), pair (b, k) occupies the flat positions
//     [start_b + k Lp_b, start_b + (k + 1) Lp_b),   start_b = K sum_{b' < b} Lp_b'.
// Workgroup w of a launch of n_wg workgroups takes the flat range
// [w R, (w + 1) R), R a multiple of 32 derived from the total, so every
// workgroup streams the same number of positions however ragged the batch
// is.  Its part of a pair (a "segment": positions [t0, t1) of (b, k), t0 a
// multiple of 32) is processed like a split-S partition, and its partial
// online-softmax state goes to slot w + b K + k: distinct (w, pair) give
// distinct slots, because a later pair only meets workgroups at or after the
// last one of an earlier pair.  The combine pass recomputes the same split
// from the same lengths and merges, for pair (b, k), the slots of
// workgroups floor(base / R) .. floor((base + L_b - 1) / R), base = the pair's
// flat start.
//
// All values here are wave-uniform; every function is called by a whole
// wave (each wave of a multi-wave workgroup computes them itself).
#pragma once

#include "common.h"

namespace gqa {

// Host-chosen constants of one call's split (the same for the partition
// pass and the combine pass of the call).
struct FlatArgs {
  int n_wg;       // workgroups of the partition pass
  int row_bytes;  // bytes of one cache row (d * element size)
  int r_min;      // smallest range, a multiple of 32
  int r_max;      // largest range, a multiple of 32 (paged: block ids of a
                  // segment must fit one per lane)
  int max_len;    // the call's max_seq_len: lengths are clamped to it, so the
                  // total never exceeds what the host sized the split for
};

__host__ __device__ inline int pad32(int L) { return (L + 31) & ~31; }

// Range length for `total` flat positions: ceil(total / n_wg) rounded up to
// a multiple of 32 and clamped to [r_min, r_max].  Ranges whose rows span a
// multiple of 64 KiB would start every workgroup of a head on the same HBM
// channel (measured 8-15% slower): such lengths are stepped past.
__device__ inline int flat_range(int total, const FlatArgs& fa) {
  int r = pad32((total + fa.n_wg - 1) / fa.n_wg);
  r = max(r, fa.r_min);
  if (((long long)r * fa.row_bytes) % 65536 == 0) r += 32;
  if (r > fa.r_max) {
    r = fa.r_max;
    if (((long long)r * fa.row_bytes) % 65536 == 0 && r > 32) r -= 32;
  }
  return r;
}

// Wave-uniform values computed from lane values are moved into scalar
// registers explicitly, so that everything derived from them (the segment's
// sequence, head and cache addresses) stays scalar too.
__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ inline int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return uniform(x);
}

// Inclusive prefix sum over the 64 lanes.
__device__ inline int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// The lengths of sequences 0..63 are read once per wave, one per lane (l0 =
// len_of(lane) for lane < B, else 0), and passed to the functions below, so
// the split's total, its sequence search and the recorded split cost one
// round trip to memory between them; sequences past 63 are read as needed.
template <class LenFn>
__device__ inline int first_lengths(int B, LenFn len_of) {
  const int lane = threadIdx.x & 63;
  return lane < B ? len_of(lane) : 0;
}

// Length of sequence i0 + lane (i0 a multiple of 64, wave-uniform).
template <class LenFn>
__device__ inline int chunk_length(int B, int i0, int l0, LenFn len_of) {
  const int i = i0 + (threadIdx.x & 63);
  return i0 == 0 ? l0 : (i < B ? len_of(i) : 0);
}

// K * sum_b pad32(len_of(b)).
template <class LenFn>
__device__ inline int flat_total(int B, int K, int l0, LenFn len_of) {
  int sum = 0;
  for (int i0 = 0; i0 < B; i0 += 64) sum += wave_sum(pad32(chunk_length(B, i0, l0, len_of)));
  return K * sum;
}

// The sequence whose flat run [start_b, start_b + K pad32(L_b)) holds flat
// position `pos` (0 <= pos < total): sets b, start_b and L_b.
template <class LenFn>
__device__ inline void flat_find(int B, int K, int pos, int l0, LenFn len_of, int& b, int& start_b,
                                 int& L_b) {
  int run = 0;  // flat start of sequence i0
  for (int i0 = 0; i0 < B; i0 += 64) {
    const int L = chunk_length(B, i0, l0, len_of);
    const int incl = wave_incl_scan(K * pad32(L));
    const unsigned long long hit = __ballot(run + incl > pos);
    if (hit) {
      const int j = uniform(__ffsll((long long)hit) - 1);
      b = i0 + j;
      start_b = run + uniform(__shfl(incl - K * pad32(L), j));
      L_b = uniform(__shfl(L, j));
      return;
    }
    run += uniform(__shfl(incl, 63));
  }
  b = B;  // not reached for pos < total
  start_b = run;
  L_b = 0;
}

// K * sum_{b' < b} pad32(len_of(b')).
template <class LenFn>
__device__ inline int flat_start_of(int B, int K, int b, LenFn len_of) {
  const int lane = threadIdx.x & 63;
  int sum = 0;
  for (int i0 = 0; i0 < b; i0 += 64) {
    const int i = i0 + lane;
    sum += wave_sum(i < b && i < B ? pad32(len_of(i)) : 0);
  }
  return K * sum;
}

// Records the split for the combine pass (called by one wave of workgroup
// 0): meta[b] = the length of sequence b attended over, meta[B + b] = its
// flat start, meta[2B] = the total.
template <class LenFn>
__device__ inline void flat_publish(int B, int K, int l0, LenFn len_of, int32_t* meta) {
  const int lane = threadIdx.x & 63;
  int run = 0;
  for (int i0 = 0; i0 < B; i0 += 64) {
    const int i = i0 + lane;
    const int L = chunk_length(B, i0, l0, len_of);
    const int incl = wave_incl_scan(K * pad32(L));
    if (i < B) {
      meta[i] = L;
      meta[B + i] = run + incl - K * pad32(L);
    }
    run += uniform(__shfl(incl, 63));
  }
  if (lane == 0) meta[2 * B] = run;
}

// Walks the segments of workgroup w: calls seg(b, k, t0, t1, L_b, slot) for
// every pair (b, k) whose valid positions meet the workgroup's range, in
// flat order.  len_of(b) must give the same lengths in every workgroup.
template <class LenFn, class SegFn>
__device__ inline void flat_for_each_segment(int w, int B, int K, int total, int R, int l0,
                                             LenFn len_of, SegFn seg) {
  int pos = w * R;
  const int end = min(pos + R, total);
  if (pos >= end) return;
  int b, start_b, L_b;
  flat_find(B, K, pos, l0, len_of, b, start_b, L_b);
  int Lp = pad32(L_b);
  int k = (pos - start_b) / Lp;
  int base = start_b + k * Lp;  // flat start of pair (b, k)
  for (;;) {
    const int t0 = pos - base;
    const int t1 = min(end - base, L_b);
    if (t0 < t1) seg(b, k, t0, t1, L_b, w + b * K + k);
    pos = base + Lp;  // start of the next pair
    if (pos >= end) break;
    if (++k == K) {
      k = 0;
      do {  // sequences of length 0 take no flat positions
        ++b;
        L_b = b >= B ? 1 : (b < 64 ? uniform(__shfl(l0, b)) : len_of(b));
      } while (L_b == 0);
      if (b >= B) break;
      Lp = pad32(L_b);
    }
    base = pos;
  }
}

}  // namespace gqa
