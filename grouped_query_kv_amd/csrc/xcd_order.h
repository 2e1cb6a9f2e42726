// Workgroup numbering for gfx950's eight XCDs (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

namespace gqa {
// gfx950 deals the workgroups of a launch to its eight XCDs round-robin by
// linear id, and each XCD has an L2 of its own.  xcd_block_id(wid, n)
// renumbers linear id wid of an n-workgroup launch so that each XCD runs one
// contiguous block of the new order (XCD x: the ids x + 8 m, numbered from
// x * floor(n / 8) + min(x, n % 8) on): workgroups that are neighbours in
// the new order share an L2.  A permutation of [0, n) for every n >= 1.
constexpr int kXcds = 8;
__host__ __device__ inline int xcd_block_id(int wid, int n) {
  const int per = n / kXcds, rem = n - per * kXcds;
  const int x = wid % kXcds, m = wid / kXcds;
  return x * per + (x < rem ? x : rem) + m;
}

}  // namespace gqa
