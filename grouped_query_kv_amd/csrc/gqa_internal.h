// Internal declarations shared by the HIP translation units of libgqa.
// Not part of the public ABI (include/gqa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "decode_flat.h"

namespace gqa {

constexpr float kLog2eHost = 1.4426950408889634f;  // 1 / ln(2)

// Split plan of one decode call: the flat split of decode_flat.h.  The
// partition pass runs fa.n_wg workgroups; the workspace holds `slots`
// partial states of G head rows each (slot w + b K + k for workgroup w's
// segment of pair (b, k), so at most n_wg + B K slots).
enum class PassKind { kBf16, kInt8, kF32 };

struct DecodePlan {
  FlatArgs fa;
  int G;          // query heads per KV head (rows of a slot)
  int head_blocks;  // ceil(G / 16): waves of the wide passes
  long long slots;  // slots the workspace holds
};

// kind: the partition pass that will run; r_max: largest range (paged:
// 63 block_size rounded down to 32; else 0 = none).  ws_n_wg: the
// workgroup count the workspace is sized for (the largest of any kind for
// these sizes, so one workspace size serves every decode entry point).
DecodePlan plan_decode(int B, int H, int K, int max_seq_len, int d, PassKind kind, int r_max = 0);
size_t decode_workspace_bytes(int B, int H, int K, int max_seq_len, int d, int r_max = 0);

// Workspace layout of a decode call:
//   part_acc [slots][G][d]      fp32 un-normalised partial outputs
//   part_ml  [slots][G][2]      fp32 running max (log2 units) and running sum
//   meta     [2B + 1]           int32: the lengths attended over, the flat
//                               starts of the sequences and the total (the
//                               split, recorded by the partition pass)
struct DecodeWorkspace {
  float* part_acc;
  float* part_ml;
  int32_t* meta;
};
// (each region 256-byte aligned; sized for the plan's slots)
DecodeWorkspace carve_decode_workspace(void* base, const DecodePlan& p, int B, int K, int d);

// ---- launchers (each returns the hipGetLastError() of its launch) ----

hipError_t launch_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            int32_t* seq_lens, int B, int K, int S_max, int row_bytes,
                            hipStream_t stream);

// Paged KV cache: pools [num_blocks, K, block_size, d]; block_table
// [B, max_blocks] int32 maps logical block j / block_size of a sequence to a
// physical block.
struct PagedArgs {
  const int32_t* block_table;
  int block_size;  // positions per block, a multiple of 16
  int max_blocks;  // block-table entries per sequence
  int num_blocks;  // physical blocks in each pool
};

// Partition pass, bf16 inputs, matrix-core (MFMA) contraction.  With
// k_new/v_new non-null the step's append is fused in (caches are written);
// with `paged` non-null the caches are block pools (with or without the
// fused append).  Groups of more than 16 query heads go to the wide pass.
hipError_t launch_decode_split_bf16(const void* q, void* k_cache, void* v_cache,
                                    const int32_t* seq_lens, const DecodeWorkspace& ws,
                                    const DecodePlan& plan, int B, int H, int K, int S_max, int d,
                                    float scale_log2, const void* k_new, const void* v_new,
                                    const PagedArgs* paged, hipStream_t stream);

// Partition pass for groups of 2 to 8 blocks of 16 query heads (bf16): one
// workgroup per (partition, KV head, sequence), one wave per head block,
// copies each K/V chunk once into LDS for all of the group's heads.  Same
// arguments and partial state as launch_decode_split_bf16, which routes such
// groups here.
bool decode_wide_supported(int head_blocks);
hipError_t launch_decode_wide_bf16(const void* q, void* k_cache, void* v_cache,
                                   const int32_t* seq_lens, const DecodeWorkspace& ws,
                                   const DecodePlan& plan, int B, int H, int K, int S_max, int d,
                                   float scale_log2, const void* k_new, const void* v_new,
                                   const PagedArgs* paged, hipStream_t stream);

// Append into a paged cache: row seq_lens[b] goes to block
// block_table[b][L / block_size], row L % block_size.
hipError_t launch_kv_append_paged(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                  const PagedArgs& pg, int32_t* seq_lens, int B, int K,
                                  int row_bytes, hipStream_t stream);

// Partition pass, fp32 inputs, vector-ALU contraction (same append option).
hipError_t launch_decode_split_f32(const void* q, void* k_cache, void* v_cache,
                                   const int32_t* seq_lens, const DecodeWorkspace& ws,
                                   const DecodePlan& plan, int B, int H, int K, int S_max, int d,
                                   float scale_log2, const void* k_new, const void* v_new,
                                   hipStream_t stream);

// int8 KV cache (codes [.., d] int8 plus one fp32 scale per row).
hipError_t launch_quantize_rows_int8(const void* src, void* codes, float* scales, int64_t rows,
                                     int d, bool bf16, hipStream_t stream);
hipError_t launch_kv_append_int8(const void* k_new, const void* v_new, void* k_codes, void* v_codes,
                                 float* k_scales, float* v_scales, int32_t* seq_lens, int B, int K,
                                 int S_max, int d, bool bf16, hipStream_t stream);
// Partition pass over an int8 cache (bf16 queries; S_max a multiple of 4).
// With k_new/v_new (bf16) non-null the quantising append is fused in.
hipError_t launch_decode_split_int8(const void* q, void* k_codes, void* v_codes, float* k_scales,
                                    float* v_scales, const int32_t* seq_lens,
                                    const DecodeWorkspace& ws, const DecodePlan& plan, int B, int H,
                                    int K, int S_max, int d, float scale_log2, const void* k_new,
                                    const void* v_new, hipStream_t stream);

// The int8 partition pass for groups of 2 to 8 blocks of 16 query heads:
// one workgroup per (partition, KV head, sequence), one wave per head block,
// codes and scales copied once into LDS for all of the group's heads.  Same
// arguments and partial state as launch_decode_split_int8, which routes such
// groups here.
hipError_t launch_decode_wide_int8(const void* q, void* k_codes, void* v_codes, float* k_scales,
                                   float* v_scales, const int32_t* seq_lens,
                                   const DecodeWorkspace& ws, const DecodePlan& plan, int B, int H,
                                   int K, int S_max, int d, float scale_log2, const void* k_new,
                                   const void* v_new, hipStream_t stream);

// Combine pass: partials -> out (fp32 or bf16).
// publish_lens: write the lengths the partition pass attended over (after a
// fused append) to seq_lens.
hipError_t launch_decode_combine(const DecodeWorkspace& ws, int32_t* seq_lens, void* out,
                                 const DecodePlan& plan, int B, int H, int K, int d, bool out_bf16,
                                 bool publish_lens, hipStream_t stream);

// Prefill family (bf16 in): S queries per sequence over L_b keys
// (kv_lens[b], or S_kv when kv_lens is null); causal: key j visible to query
// i iff j <= L_b - S + i.
hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, void* out,
                               const int32_t* kv_lens, int B, int H, int K, int S, int S_kv,
                               int S_max, int d, float scale_log2, bool out_bf16, bool causal,
                               hipStream_t stream);

// The same family for fp32 inputs and outputs (vector ALUs, fp32 throughout).
hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, void* out,
                              const int32_t* kv_lens, int B, int H, int K, int S, int S_kv, int S_max,
                              int d, float scale_log2, bool causal, hipStream_t stream);

// seq_lens[b] += T where L + T <= S_max (run after the launch that wrote the rows).
hipError_t launch_bump_lens(int32_t* seq_lens, int B, int T, int S_max, hipStream_t stream);

// K/V projection of B*T tokens x [B, T, d_model] by W_KV [K, 2d, d_model]
// (bf16) into rows k_out, v_out [B, K, T, d].
hipError_t launch_kv_project(const void* x, const void* w_kv, void* k_out, void* v_out, int B, int T,
                             int d_model, int K, int d, hipStream_t stream);

// Append T rows per (sequence, KV head) at seq_lens[b] (two launches).
hipError_t launch_kv_append_rows(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                                 int32_t* seq_lens, int B, int K, int T, int S_max, int row_bytes,
                                 hipStream_t stream);

hipError_t launch_meanpool(const void* src, void* dst, int64_t outer, int H, int K, int64_t inner,
                           bool bf16, hipStream_t stream);

}  // namespace gqa
