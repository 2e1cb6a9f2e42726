/*
 * gqa.h -- C ABI of the MI355X (gfx950) grouped-query-attention library.
 *
 * Grouped-query attention (GQA) splits H query heads into K groups of
 * G = H / K consecutive heads; every head of group g attends to the one
 * shared key head K_g and value head V_g with softmax(q K_g^T * scale) V_g.
 *   - compassingai.com "分組查詢注意力", section 技術原理 (technical principle):
 *     Q is regrouped [.., H, d] -> [.., K, H/K, d]; each generated token
 *     writes one [batch, 1, K, d_k] K and V row.
 *   - pinghaoyang.com.cn/aigc/posts/gqa "GQA 完全拆解", section
 *     GQA：插值在 MHA 与 MQA 之间的分组共享 (GQA): group g is the consecutive
 *     query heads (g-1)H/K+1 .. gH/K; K = 1 is MQA and K = H is MHA.
 *   - same page, section 解码推理的内存账本 (decode memory ledger): at decode
 *     step t the new query attends to all cached rows 1..t and the new K/V
 *     row joins the cache; prefill processes the whole prefix at once.
 *   - same page, section 工程实现 (engineering): the cache is laid out
 *     layer x KV head x position and a group-aware kernel loads each shared
 *     KV block once for all query heads of its group.
 *
 * Conventions for every entry point
 *   - Layouts are contiguous row-major:
 *       q (decode)        [B, H, d]
 *       k_cache, v_cache  [B, K, S_max, d]      (position rows, d innermost)
 *       k_new, v_new      [B, K, d]
 *       seq_lens          [B] int32             (valid rows per sequence)
 *       q, out (prefill)  [B, H, S, d]
 *     Query head h uses KV head h / G (integer division).
 *   - All pointers are device memory owned by the caller (hipMalloc or a
 *     framework allocator); the library never frees or retains them after
 *     the call returns.  Base pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work and never synchronises the device.
 *   - Element types: GQA_F32 (float) and GQA_BF16 (bfloat16, RNE on output).
 *     Supported head dimensions: d = 64 and d = 128.
 *   - Return value: GQA_OK, or a negative code.  Argument errors are found
 *     on the host before anything is enqueued; the text of the last error of
 *     the calling thread is returned by gqa_last_error().
 *   - Device-side contract (cannot be checked without a synchronisation):
 *     0 <= seq_lens[b] <= S_max, and for decode seq_lens[b] <= max_seq_len.
 *     Cache rows at positions >= seq_lens[b] are never read.
 */
#ifndef GQA_H_
#define GQA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { GQA_F32 = 0, GQA_BF16 = 1 };

enum {
  GQA_OK = 0,
  GQA_ERR_INVALID = -1,     /* null pointer, bad size, H % K != 0, misalignment */
  GQA_ERR_UNSUPPORTED = -2, /* d not in {64, 128}, unsupported dtype pair       */
  GQA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required      */
  GQA_ERR_HIP = -4          /* a HIP runtime call or launch failed             */
};

/* Version of this ABI (bumped on any incompatible change). */
int gqa_abi_version(void);

/*
 * Identity of the code this library was built from: the lowercase hex
 * SHA-256 of its sources (every kernel and header source and this header,
 * with comments removed and whitespace runs collapsed), fixed at build time.
 * A caller compares it with the hash of the sources it expects, so that a
 * library built from other sources is never used.  The string is static.
 */
const char* gqa_build_id(void);

/*
 * Append one token per sequence: for every b with L = seq_lens[b] < S_max
 *   k_cache[b, k, L, :] = k_new[b, k, :],  v_cache[b, k, L, :] = v_new[b, k, :]
 * for all k, then seq_lens[b] = L + 1.  A sequence whose cache is full
 * (L == S_max) is left untouched, so nothing is ever written out of bounds.
 * The copy is bit-exact.  (compassingai.com, technical principle: a token
 * writes a [batch, 1, K, d_k] row; pinghaoyang.com.cn, decode memory ledger.)
 * Arguments: B, K >= 1; S_max >= 1; d in {64, 128}; dtype GQA_F32 or GQA_BF16.
 */
int gqa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  int32_t* seq_lens, int B, int K, int S_max, int d, int dtype,
                  void* stream);

/*
 * Bytes of device workspace gqa_decode needs for these sizes (0 on invalid
 * sizes).  The workspace holds per-partition partial results and is fully
 * overwritten by every call; its content on entry does not matter.
 */
size_t gqa_decode_workspace_bytes(int B, int H, int K, int max_seq_len, int d);

/*
 * One decode step of GQA over the KV cache:
 *   out[b, h, :] = sum_{j < L_b} p_j v_cache[b, h/G, j, :],
 *   p = softmax_j(scale * q[b, h, :] . k_cache[b, h/G, j, :]),  L_b = seq_lens[b]
 * and out[b, h, :] = 0 when L_b == 0.  Call gqa_kv_append first to attend
 * to the new token as well (pinghaoyang.com.cn, decode memory ledger: the
 * step-t query sees rows 1..t).
 *
 * The cache is split along positions into partitions that are reduced with
 * an online softmax (fp32 running max and sum) and combined in a second
 * pass; each partition streams its K/V rows once for all G heads.
 *
 * max_seq_len: host-side upper bound of every seq_lens[b] (sizes the split).
 * dtype: element type of q and the caches; out_dtype: GQA_F32, or GQA_BF16
 * when dtype is GQA_BF16.  scale: finite and > 0, usually 1/sqrt(d).
 * workspace: device buffer of at least gqa_decode_workspace_bytes(...) bytes.
 */
int gqa_decode(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* seq_lens, void* out, void* workspace, size_t workspace_bytes,
               int B, int H, int K, int S_max, int max_seq_len, int d, float scale,
               int dtype, int out_dtype, void* stream);

/*
 * One decode step with the cache append fused in: the same result as
 * gqa_kv_append(k_new, v_new, k_cache, v_cache, seq_lens, ...) followed by
 * gqa_decode(q, k_cache, v_cache, seq_lens, out, ...) -- caches and
 * seq_lens end up bit-identical, out within the decode tolerance -- in two
 * kernel launches instead of three: the partition holding the new position
 * takes that row from k_new/v_new and writes it into the cache.  A sequence
 * whose cache is full (seq_lens[b] == S_max) gets no append and attends over
 * its S_max rows.  max_seq_len bounds the lengths *after* the append.
 * (pinghaoyang.com.cn, decode memory ledger: each step appends the new K/V
 * row and the new query attends to every cached row including it.)
 * Arguments as gqa_kv_append and gqa_decode; workspace sized by
 * gqa_decode_workspace_bytes(B, H, K, max_seq_len, d).
 */
int gqa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                      void* v_cache, int32_t* seq_lens, void* out, void* workspace,
                      size_t workspace_bytes, int B, int H, int K, int S_max, int max_seq_len,
                      int d, float scale, int dtype, int out_dtype, void* stream);

/*
 * gqa_decode_append without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, results and
 * kernels as gqa_decode_append; the partial results go to a static device
 * array inside the library of 64 MiB (67,108,864 bytes) per GPU, held from
 * the first call on that GPU until the process ends.  Sizes whose
 * gqa_decode_workspace_bytes(B, H, K, max_seq_len, d) exceeds that return
 * GQA_ERR_WORKSPACE before anything is enqueued.  The call allocates and
 * frees nothing.  Every call on one GPU uses the same array: calls that
 * overlap in time on one GPU (different streams, or different host threads)
 * race and must be serialised by the caller.  The first call on a device
 * looks up the array's address on the current device (hipGetDevice), so the
 * stream must belong to the current device.
 */
int gqa_decode_append_noalloc(const void* q, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, int32_t* seq_lens, void* out, int B, int H, int K,
                              int S_max, int max_seq_len, int d, float scale, int dtype,
                              int out_dtype, void* stream);

/*
 * Paged KV cache.  The K and V pools are [num_blocks, K, block_size, d]:
 * physical block n holds block_size consecutive positions of every KV head,
 * one row of d elements per (head, position).  block_table is [B, max_blocks]
 * int32 (row-major): logical position j of sequence b lives in physical block
 * block_table[b, j / block_size], row j % block_size.  Blocks may be shared
 * between sequences and appear in any order.  Each block is K * block_size
 * rows (not H * block_size), broadcast inside the kernel to the G query heads
 * of its group.  (compassingai.com "分組查詢注意力", section 下游 (downstream
 * schedulers): paged blocks hold K * s rows and are broadcast to the H/K
 * query heads; pinghaoyang.com.cn "GQA 完全拆解", section 工程实现
 * (engineering): paged blocks are organised by KV head and the kernel
 * broadcasts inside the group; same page, decode memory ledger: paging
 * removes allocation waste and is orthogonal to GQA.)
 *
 * Paged caches are bf16 only; block_size is a multiple of 16; num_blocks,
 * max_blocks >= 1; max_blocks * block_size <= 2^30.  Device-side contract:
 * 0 <= seq_lens[b] <= max_blocks * block_size and every block id a kernel
 * reads lies in [0, num_blocks) (ids outside it are clamped on read, so a
 * bad table yields wrong values, never an out-of-bounds access).
 */

/*
 * Append one token per sequence into a paged cache: for every b with
 * L = seq_lens[b] < max_blocks * block_size and n = block_table[b, L /
 * block_size] in [0, num_blocks):
 *   k_pool[n, k, L % block_size, :] = k_new[b, k, :]   (and v likewise)
 * then seq_lens[b] = L + 1.  Otherwise the sequence is left untouched.
 * The copy is bit-exact.  dtype GQA_F32 or GQA_BF16; d in {64, 128}.
 */
int gqa_kv_append_paged(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                        const int32_t* block_table, int32_t* seq_lens, int B, int K,
                        int num_blocks, int block_size, int max_blocks, int d, int dtype,
                        void* stream);

/*
 * Bytes of device workspace gqa_decode_paged needs (0 on invalid sizes).
 */
size_t gqa_decode_paged_workspace_bytes(int B, int H, int K, int max_seq_len, int d,
                                        int block_size);

/*
 * One decode step over a paged cache: the result of gqa_decode on the
 * contiguous cache whose row j of (b, k) is k_pool[block_table[b, j /
 * block_size], k, j % block_size, :] (and v likewise).  L_b = seq_lens[b];
 * out[b, h, :] = 0 when L_b == 0.  max_seq_len bounds every seq_lens[b]
 * and is at most max_blocks * block_size.  dtype GQA_BF16; out_dtype
 * GQA_BF16 or GQA_F32; workspace of gqa_decode_paged_workspace_bytes(...).
 */
int gqa_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const int32_t* seq_lens, void* out,
                     void* workspace, size_t workspace_bytes, int B, int H, int K,
                     int num_blocks, int block_size, int max_blocks, int max_seq_len, int d,
                     float scale, int dtype, int out_dtype, void* stream);

/*
 * One paged decode step with the append fused in: the result of
 * gqa_kv_append_paged(k_new, v_new, ...) followed by gqa_decode_paged(q, ...)
 * on the grown cache -- the same pools, lengths and output bits -- in one
 * partition pass and one combine pass.  The append rule is the standalone
 * one: a sequence with L = seq_lens[b] < max_blocks * block_size whose block
 * id block_table[b, L / block_size] lies in [0, num_blocks) gets the row at
 * L and L + 1; any other sequence is attended as it is.  (pinghaoyang.com.cn
 * "GQA 完全拆解", decode memory ledger: each step appends one K and V row per
 * KV head and reads the cache; compassingai.com "分組查詢注意力", downstream
 * schedulers: paged blocks hold K * s rows.)  q, k_new, v_new bf16 ([B, H,
 * d] and [B, K, d]; dtype must be GQA_BF16); max_seq_len bounds the lengths
 * *after* the append.  Other arguments, alignment and workspace
 * (gqa_decode_paged_workspace_bytes) as gqa_decode_paged.
 */
int gqa_decode_append_paged(const void* q, const void* k_new, const void* v_new, void* k_pool,
                            void* v_pool, const int32_t* block_table, int32_t* seq_lens, void* out,
                            void* workspace, size_t workspace_bytes, int B, int H, int K,
                            int num_blocks, int block_size, int max_blocks, int max_seq_len, int d,
                            float scale, int dtype, int out_dtype, void* stream);

/*
 * int8 KV cache.  Codes k_codes, v_codes are int8 [B, K, S_max, d]; scales
 * k_scales, v_scales are float [B, K, S_max], one per cached row; row
 * (b, k, j) reads back as codes[b, k, j, i] * scales[b, k, j].  The pages
 * give no quantisation rule; this library quantises each row of d elements
 * symmetrically by its absolute maximum, in IEEE fp32 with correctly rounded
 * division: amax = max |x_i|, c_i = clamp(rint(x_i * (127 / amax)), -127,
 * 127), scale = amax / 127 (a zero row: codes 0, scale 0).  Rows must be
 * finite.  (pinghaoyang.com.cn "GQA 完全拆解", the related-work list after the
 * KV ledger: INT8 / INT4 KV quantisation is orthogonal to GQA and the savings
 * multiply; aicoding.csdn.net "LLaMa3与DeepSeek采用的GQA技术", section 3
 * (deployment tips): 8-bit KV quantisation halves the cache.)  An int8
 * cache holds 2 (d + 4) bytes per position and KV head against 4 d in bf16.
 */

/*
 * Quantise `rows` rows of d elements (src: GQA_F32 or GQA_BF16, [rows, d])
 * into codes [rows, d] and scales [rows] by the rule above, bit-exactly.
 * src 16-byte aligned, codes 8-byte aligned, scales 4-byte aligned.
 */
int gqa_kv_quantize_int8(const void* src, void* codes, float* scales, int64_t rows, int d,
                         int dtype, void* stream);

/*
 * Append one token per sequence into an int8 cache: for every b with
 * L = seq_lens[b] < S_max, quantise k_new[b, k, :] and v_new[b, k, :]
 * (dtype GQA_F32 or GQA_BF16) and store codes and scales at position L of
 * every KV head k, then seq_lens[b] = L + 1.  A full cache is left untouched.
 */
int gqa_kv_append_int8(const void* k_new, const void* v_new, void* k_codes, void* v_codes,
                       float* k_scales, float* v_scales, int32_t* seq_lens, int B, int K,
                       int S_max, int d, int dtype, void* stream);

/*
 * One decode step over an int8 cache: gqa_decode's result on the cache
 * whose rows are the dequantised codes * scales.  q is bf16 [B, H, d]
 * (q_dtype must be GQA_BF16); out_dtype GQA_BF16 or GQA_F32.  S_max must be
 * a multiple of 4 (scale rows are read 16 bytes at a time) and every
 * pointer 16-byte aligned.  Workspace: gqa_decode_workspace_bytes(B, H, K,
 * max_seq_len, d) bytes.
 */
int gqa_decode_int8(const void* q, const void* k_codes, const void* v_codes, const float* k_scales,
                    const float* v_scales, const int32_t* seq_lens, void* out, void* workspace,
                    size_t workspace_bytes, int B, int H, int K, int S_max, int max_seq_len, int d,
                    float scale, int q_dtype, int out_dtype, void* stream);

/*
 * One decode step with the quantising append fused in: the result of
 * gqa_kv_append_int8(k_new, v_new, ...) followed by gqa_decode_int8(q, ...)
 * on the grown cache -- the same codes, scales, lengths and output bits --
 * in one partition pass and one combine pass.  (pinghaoyang.com.cn "GQA
 * 完全拆解", decode memory ledger: each step writes the new token's K and V
 * once per KV head and reads the cache; the int8 rule is the one above.)
 * q, k_new, v_new are bf16 [B, H, d] / [B, K, d] (dtype must be GQA_BF16);
 * max_seq_len bounds the lengths *after* the append.  Other arguments,
 * alignment and workspace as gqa_decode_int8.
 */
int gqa_decode_append_int8(const void* q, const void* k_new, const void* v_new, void* k_codes,
                           void* v_codes, float* k_scales, float* v_scales, int32_t* seq_lens,
                           void* out, void* workspace, size_t workspace_bytes, int B, int H, int K,
                           int S_max, int max_seq_len, int d, float scale, int dtype, int out_dtype,
                           void* stream);

/*
 * Causal GQA attention over a whole prefix (prefill):
 *   out[b, h, i, :] = sum_{j <= i} softmax_j(scale q[b,h,i,:] . k[b,h/G,j,:]) v[b,h/G,j,:]
 * for i in [0, S).  k and v are [B, K, S_max, d] with S <= S_max; rows >= S
 * are never read.  (pinghaoyang.com.cn, decode memory ledger: prefill
 * computes the whole prefix in parallel; row i equals decode step i.)
 * dtype GQA_BF16 (bf16 matrix-core path, fp32 accumulation; out_dtype
 * GQA_BF16 or GQA_F32) or GQA_F32 (vector-ALU path, fp32 throughout;
 * out_dtype GQA_F32); scale finite and > 0.  Any other pair returns
 * GQA_ERR_UNSUPPORTED.
 */
int gqa_prefill_causal(const void* q, const void* k, const void* v, void* out,
                       int B, int H, int K, int S, int S_max, int d, float scale,
                       int dtype, int out_dtype, void* stream);

/*
 * Prefill of a chunk over a cache: q, out [B, H, S, d]; the caches
 * [B, K, S_max, d] already hold the chunk's K/V rows as their last S rows,
 * L_b = seq_lens[b] rows in all (device int32 [B]).  Query i of sequence b
 * sits at position L_b - S + i and attends causally:
 *   out[b, h, i, :] = sum_{j <= L_b - S + i} softmax_j(scale q . k_j) v_j.
 * (pinghaoyang.com.cn "GQA 完全拆解", decode memory ledger: the query at
 * position t attends to cached rows 1..t; prefill computes a run of
 * positions at once -- a chunk is such a run continuing a cache.)
 * gqa_prefill_causal is the case L_b = S.  Device-side contract:
 * S <= seq_lens[b] <= S_max (a query with no visible row gets zeros).
 * Types as gqa_prefill_causal; scale finite and > 0.
 */
int gqa_prefill_chunk(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seq_lens, void* out, int B, int H, int K, int S, int S_max,
                      int d, float scale, int dtype, int out_dtype, void* stream);

/*
 * Non-causal GQA attention (cross-attention): q, out [B, H, S_q, d] over rows
 * [0, L_b) of k, v [B, K, S_max, d], L_b = kv_lens[b] (device int32 [B],
 * 0 <= L_b <= S_max):
 *   out[b, h, i, :] = sum_{j < L_b} softmax_j(scale q[b,h,i,:] . k[b,h/G,j,:]) v[b,h/G,j,:]
 * and zeros when L_b = 0.  (pinghaoyang.com.cn "GQA 完全拆解", GQA section:
 * grouped KV heads are used in decoder self-attention and in
 * cross-attention, not in encoder self-attention.)  Types as prefill.
 */
int gqa_cross_attention(const void* q, const void* k, const void* v, const int32_t* kv_lens,
                        void* out, int B, int H, int K, int S_q, int S_max, int d, float scale,
                        int dtype, int out_dtype, void* stream);

/*
 * Append T rows per sequence: for every b with L = seq_lens[b] and
 * L + T <= S_max, k_cache[b, k, L + t, :] = k_new[b, k, t, :] (and v) for
 * t < T and every k, then seq_lens[b] = L + T; a sequence without room for
 * all T rows is left untouched.  k_new, v_new [B, K, T, d]; bit-exact copy;
 * dtype GQA_F32 or GQA_BF16.  Two kernel launches (copy, then lengths).
 */
int gqa_kv_append_rows(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       int32_t* seq_lens, int B, int K, int T, int S_max, int d, int dtype,
                       void* stream);

/*
 * Fused K/V projection.  x [B, T, d_model] holds the hidden states of T new
 * tokens per sequence; w_kv [K, 2d, d_model] is the merged key/value
 * projection (rows [0, d) of head k are W_K[k], rows [d, 2d) are W_V[k]):
 *   k_out[b, k, t, :] = W_KV[k, 0:d, :] x[b, t, :],   v_out[b, k, t, :] = W_KV[k, d:2d, :] x[b, t, :]
 * with fp32 accumulation rounded to bf16; k_out, v_out are [B, K, T, d], the
 * layout gqa_kv_append_rows takes (and, for T = 1, the k_new / v_new of
 * gqa_decode_append, which appends them inside the attention pass).
 * (pinghaoyang.com.cn "GQA 完全拆解", section 工程实现 (engineering): W_K, W_V
 * are [G, d_k, d_model] with G KV heads, and frameworks merge them into one
 * W_KV [G, 2 d_k, d_model] so that one GEMM yields K and V.)  No bias and
 * no positional rotation.  bf16 only; d_model a multiple of 32; d in
 * {64, 128}; x and w_kv 16-byte aligned.  One kernel launch; each W_KV
 * byte is read once per 16 tokens.
 */
int gqa_kv_project(const void* x, const void* w_kv, void* k_out, void* v_out, int B, int T,
                   int d_model, int K, int d, int dtype, void* stream);

/*
 * gqa_kv_project followed by gqa_kv_append_rows: the projected rows are
 * written at positions [L_b, L_b + T) of k_cache, v_cache [B, K, S_max, d]
 * and seq_lens[b] += T (a sequence without room for T rows is left
 * untouched).  workspace: device buffer of at least
 * gqa_kv_project_workspace_bytes(B, T, d_model, K, d) bytes (the projected
 * rows; content on entry does not matter).  Two kernel launches (three when
 * a sequence's T rows exceed 8192 16-byte words).
 */
size_t gqa_kv_project_workspace_bytes(int B, int T, int d_model, int K, int d);
int gqa_kv_project_append(const void* x, const void* w_kv, void* k_cache, void* v_cache,
                          int32_t* seq_lens, void* workspace, size_t workspace_bytes, int B, int T,
                          int d_model, int K, int S_max, int d, int dtype, void* stream);

/*
 * Mean-pool conversion of per-head weights into group weights:
 *   dst[o, g, i] = (sum_{r < G} src[o, g*G + r, i]) / G
 * with src [outer, H, inner] and dst [outer, K, inner], both of `dtype`.
 * The sum runs in fp32 in head order and is divided once by G (IEEE
 * division), then rounded to dtype.  (pinghaoyang.com.cn, section
 * Uptraining：把现成 MHA 检查点改造成 GQA (mean-pooling conversion);
 * compassingai.com, technical principle.)
 */
int gqa_meanpool_convert(const void* src, void* dst, int64_t outer, int H, int K,
                         int64_t inner, int dtype, void* stream);

/*
 * KV-cache size in bytes: 2 * layers * K * d * elem_bytes * tokens
 * (pinghaoyang.com.cn, decode memory ledger and GQA section).  Host only.
 * Returns 0 if any argument is negative.
 */
uint64_t gqa_kv_cache_bytes(int layers, int K, int d, int elem_bytes, uint64_t tokens);

/*
 * Benchmark timing hook.  While set (both non-NULL), the decode entry
 * points (around their partition pass), the prefill family, the projection
 * entry points and the mean-pool conversion record `begin_event` on their
 * stream immediately before launching that kernel and `end_event`
 * immediately after it; the events are hipEvent_t handles passed as void*,
 * owned by the caller.  The append-only entry points record nothing.
 * Applies to calls from the calling thread only; pass NULLs to clear.
 */
int gqa_set_timing_events(void* begin_event, void* end_event);

/* Text of the last error returned on the calling thread ("" if none). */
const char* gqa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H_ */
