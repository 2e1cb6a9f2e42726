// Cache append: one new K row and one new V row per (sequence, KV head) are
// written at position seq_lens[b], then seq_lens[b] grows by one.
//
// compassingai.com "分組查詢注意力", section 技術原理 (technical principle): a
// generated token writes a [batch, 1, K, d_k] K and V row (K KV heads, not
// H).  pinghaoyang.com.cn "GQA 完全拆解", section 解码推理的内存账本 (decode
// memory ledger): the new row joins the cache at every decode step.
//
// One workgroup per sequence b.  Every thread reads seq_lens[b] before the
// barrier and only thread 0 writes it after the barrier, so no thread can
// see the incremented value.  Rows are moved as raw 16-byte words (bit
// exact for any element type).  A full cache (L == S_max) is left as is.
#include "gqa_internal.h"

namespace gqa {
namespace {

constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int32_t* __restrict__ seq_lens,
    int K, int S_max, int row_words) {
  const int b = blockIdx.x;
  const int L = seq_lens[b];
  __syncthreads();
  if (L < 0 || L >= S_max) return;  // full (or corrupt) entry: write nothing
  const int words = K * row_words;
  for (int w = threadIdx.x; w < words; w += kAppendThreads) {
    const int k = w / row_words;
    const int o = w - k * row_words;
    const size_t src = (size_t)(b * K + k) * row_words + o;
    const size_t dst = ((size_t)(b * K + k) * S_max + L) * row_words + o;
    k_cache[dst] = k_new[src];
    v_cache[dst] = v_new[src];
  }
  if (threadIdx.x == 0) seq_lens[b] = L + 1;
}

// Paged variant: position L of sequence b lives in physical block
// block_table[b][L / block_size], row L % block_size of each KV head.  An
// invalid block id (outside [0, num_blocks)) or a full table leaves the
// sequence untouched.
__global__ __launch_bounds__(kAppendThreads) void kv_append_paged_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    uint4* __restrict__ k_pool, uint4* __restrict__ v_pool, const int32_t* __restrict__ block_table,
    int32_t* __restrict__ seq_lens, int K, int block_size, int max_blocks, int num_blocks,
    int row_words) {
  const int b = blockIdx.x;
  const int L = seq_lens[b];
  const int blk = (L >= 0 && L < max_blocks * block_size)
                      ? block_table[(size_t)b * max_blocks + L / block_size] : -1;
  __syncthreads();
  if (blk < 0 || blk >= num_blocks) return;
  const int row = L - (L / block_size) * block_size;
  const int words = K * row_words;
  for (int w = threadIdx.x; w < words; w += kAppendThreads) {
    const int k = w / row_words;
    const int o = w - k * row_words;
    const size_t src = (size_t)(b * K + k) * row_words + o;
    const size_t dst = (((size_t)blk * K + k) * block_size + row) * row_words + o;
    k_pool[dst] = k_new[src];
    v_pool[dst] = v_new[src];
  }
  if (threadIdx.x == 0) seq_lens[b] = L + 1;
}

// Multi-row variant: T rows per (sequence, KV head) go to positions
// [L, L + T); a sequence without room for all T rows is left untouched.
// With `publish` (one workgroup per sequence) the workgroup also writes the
// new length after its barrier; otherwise a separate launch does.
__global__ __launch_bounds__(kAppendThreads) void kv_append_rows_kernel(
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, int32_t* __restrict__ seq_lens,
    int K, int T, int S_max, int row_words, bool publish) {
  const int b = blockIdx.x;
  const int L = seq_lens[b];
  __syncthreads();
  if (L < 0 || L > S_max - T) return;
  const int words = T * row_words;  // per KV head: T consecutive rows in both layouts
  for (int k = blockIdx.y; k < K; k += gridDim.y) {
    const size_t src0 = ((size_t)b * K + k) * words;
    const size_t dst0 = (((size_t)b * K + k) * S_max + L) * row_words;
    for (int w = threadIdx.x; w < words; w += kAppendThreads) {
      k_cache[dst0 + w] = k_new[src0 + w];
      v_cache[dst0 + w] = v_new[src0 + w];
    }
  }
  if (publish && threadIdx.x == 0) seq_lens[b] = L + T;
}

// Publishes the new lengths once every workgroup of the writing launch has
// read the old ones (a separate launch orders the two).
__global__ void bump_lens_kernel(int32_t* __restrict__ seq_lens, int B, int T, int S_max) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    const int L = seq_lens[b];
    if (L >= 0 && L <= S_max - T) seq_lens[b] = L + T;
  }
}

}  // namespace

hipError_t launch_kv_append_rows(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 int32_t* seq_lens, int B, int K, int T, int S_max, int row_bytes,
                                 hipStream_t stream) {
  // a few rows per sequence (a decode step): one workgroup per sequence,
  // which also publishes the length; else up to 8 per sequence and a
  // separate length update
  const long long words = (long long)K * T * (row_bytes / 16);
  const int ky = words <= 8192 ? 1 : (K < 8 ? K : 8);
  hipLaunchKernelGGL(kv_append_rows_kernel, dim3(B, ky), dim3(kAppendThreads), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), seq_lens, K, T,
                     S_max, row_bytes / 16, ky == 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ky == 1) return e;
  return launch_bump_lens(seq_lens, B, T, S_max, stream);
}

hipError_t launch_bump_lens(int32_t* seq_lens, int B, int T, int S_max, hipStream_t stream) {
  hipLaunchKernelGGL(bump_lens_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, seq_lens, B, T,
                     S_max);
  return hipGetLastError();
}

hipError_t launch_kv_append_paged(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                  const PagedArgs& pg, int32_t* seq_lens, int B, int K,
                                  int row_bytes, hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_paged_kernel, dim3(B), dim3(kAppendThreads), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), pg.block_table,
                     seq_lens, K, pg.block_size, pg.max_blocks, pg.num_blocks, row_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            int32_t* seq_lens, int B, int K, int S_max, int row_bytes,
                            hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_kernel, dim3(B), dim3(kAppendThreads), 0, stream,
                     static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new),
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), seq_lens, K,
                     S_max, row_bytes / 16);
  return hipGetLastError();
}

}  // namespace gqa
