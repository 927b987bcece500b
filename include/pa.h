/*
 * pa.h - C ABI of the paged decode-attention library (libpa.so) for AMD
 * Instinct MI355X (gfx950).
 *
 * The library implements the GPU hot path of PagedAttention decode:
 *   - pa_reshape_and_cache: append new tokens' key/value rows into the slots
 *     the block manager assigned them (the KV cache grows by one row per
 *     generated token; blocks are allocated on demand):
 *       "Paged Attention and Memory Efficiency in Production LLM Serving",
 *       sections "Why KV cache memory was the bottleneck ..." and "How
 *       PagedAttention borrows OS paging ...";
 *       "PagedAttention in Production", section "Core Principle".
 *   - pa_decode: one query token per sequence attends over that sequence's
 *     keys/values, which live in fixed-size physical blocks found through the
 *     sequence's block table at run time; the result is ordinary softmax
 *     attention:
 *       "Paged Attention and Memory Efficiency ...", section "How
 *       PagedAttention borrows OS paging ...";
 *       "PagedAttention in Production", section "Relationship with Continuous
 *       Batching" (flow figure: the attention kernel reads blocks by block
 *       table);
 *       "PagedAttention - The KV Cache Problem", section "How It Works".
 *   - pa_decode_append: one decode step in one call (append, then attend).
 *   - pa_bm_*: the host block manager that hands out the slots, tables and
 *     copy pairs the calls above take (pool, on-demand growth, sharing,
 *     copy-on-write, sink + window eviction).
 *   - pa_copy_blocks: copy-on-write duplication of a shared block once a
 *     sequence diverges from a shared prefix:
 *       "Paged Attention and Memory Efficiency ...", section "How
 *       PagedAttention borrows OS paging ..." (sharing and copy-on-write);
 *       "PagedAttention - The KV Cache Problem", section "Why This Matters for
 *       Production" (copy-on-write for parallel sampling and beam search).
 *
 * Conventions shared by every call
 *   - KV cache layout (one tensor for K, one for V, per layer):
 *       [num_blocks, num_kv_heads, block_size, head_dim], row-major, so one
 *       (block, kv head) chunk is block_size*head_dim contiguous elements.
 *   - Slot of a token = physical_block * block_size + row within the block.
 *   - Query head i reads KV head i / gqa_group (consecutive grouping).
 *   - Element dtypes: PA_F16 / PA_BF16 are IEEE half / bfloat16;
 *     PA_FP8_E4M3 is the OCP E4M3FN 8-bit format (bias 7, max 448, no
 *     infinities, S.1111.111 = NaN) with one fp32 scale per tensor:
 *     value = decode(code) * scale, or one per row (the *_scaled calls);
 *     PA_FP4_E2M1 is OCP E2M1 (max 6), only with a scale per row.
 *   - Ownership: the caller allocates and owns every buffer.  All pointers
 *     are device pointers except where stated; each must be 16-byte aligned.
 *     The library never allocates, frees or synchronises device memory and
 *     never changes the current device.  Work is enqueued asynchronously on
 *     `stream` (NULL = the default stream).
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued, so a call that returns an error has no effect.  A failed
 *     kernel launch returns PA_ERR_HIP.  pa_last_error_message() gives a
 *     thread-local description of the last error.
 *   - Device-side contract (not checked on the host, since checking would
 *     need the device data): block ids in block tables and copy pairs lie in
 *     [0, num_blocks); slots are unique within one call; copy pairs have
 *     distinct destinations and no destination is also a source in the same
 *     call; 0 <= context_lens[s] <= max_context_len; for pa_decode_append,
 *     the block that receives a sequence's new row (its block of position
 *     L - 1) is read by no other table entry of the call.  The kernels never read
 *     or write outside the buffers when these are violated (out-of-range ids
 *     and slots are skipped, lengths are clamped), but results are then
 *     unspecified.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* pa_stream_t; /* a hipStream_t */

typedef enum {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E4M3 = 3,
  PA_FP4_E2M1 = 4 /* OCP E2M1, two per byte (element 2i in the low nibble); row-scaled caches only */
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned pointer */
  PA_ERR_UNSUPPORTED = -2, /* valid but not built: dtype combination, head_dim, block size */
  PA_ERR_WORKSPACE = -3,   /* workspace smaller than pa_decode_workspace_size() */
  PA_ERR_HIP = -4,         /* the HIP runtime refused a launch */
  PA_ERR_NO_BLOCKS = -5,   /* block manager: the pool has too few free blocks */
  PA_ERR_CONTRACT = -6     /* checked build only: the device-side contract is violated */
} pa_status;

/*
 * Checked build.  libpa_checked.so (the same sources built with PA_CHECKED)
 * checks the device-side contract above on the device: before a call
 * enqueues its work it runs small kernels over the device arrays the
 * contract bounds, waits for the stream, and returns PA_ERR_CONTRACT (with
 * pa_last_error_message() naming each violation) without enqueueing
 * anything else, so a rejected call has no effect.  It is for debugging:
 * every call waits for its stream.  Under stream capture the checks are
 * captured with the work and a violation is reported by the next call made
 * outside a capture.  The bits of what was found:
 */
#define PA_VIOLATION_BLOCK_ID 0x01u          /* a table entry a sequence reads lies outside [0, num_blocks) */
#define PA_VIOLATION_CONTEXT_LEN 0x02u       /* context_lens[s] outside [0, max_context_len] */
#define PA_VIOLATION_SLOT 0x04u              /* a slot >= num_blocks * block_size */
#define PA_VIOLATION_SLOT_REPEATED 0x08u     /* a non-negative slot given twice in one call */
#define PA_VIOLATION_COPY_ID 0x10u           /* a copy pair id outside [0, num_blocks) */
#define PA_VIOLATION_COPY_DST_REPEATED 0x20u /* two copy pairs with one destination */
#define PA_VIOLATION_COPY_DST_IS_SRC 0x40u   /* a copy destination that is another pair's source */
#define PA_VIOLATION_QUERY_START 0x80u       /* query_start not as pa_decode_multi requires */
#define PA_VIOLATION_APPEND_BLOCK_SHARED 0x100u /* pa_decode_append: a sequence's block of position L - 1
                                                   is also read by another table entry of the call */
#define PA_VIOLATION_PREFIX_GROUP 0x200u        /* pa_decode_shared_prefix: group_start or prefix_lens
                                                   not as the call requires */

/* 1 in libpa_checked.so, 0 in libpa.so. */
int32_t pa_is_checked_build(void);

/*
 * Append rows: for every token n in [0, T) with slot = slot_mapping[n] >= 0,
 *   k_cache[slot / block_size, h, slot % block_size, :] = enc(key[n, h, :])
 *   v_cache[...same...]                                  = enc(value[n, h, :])
 * for every kv head h.  enc is a bit copy when cache_dtype == src_dtype; for
 * an FP8 cache it is the E4M3FN code of fp32(x) / k_scale (v_scale for V)
 * with IEEE fp32 division, round-to-nearest-even, magnitudes beyond 448
 * saturating to 448 and a NaN input stored as the NaN code of its sign
 * (0x7F or 0xFF).
 *   key, value     [T, num_kv_heads, head_dim], src_dtype (PA_F16 | PA_BF16)
 *   k_cache, v_cache [num_blocks, num_kv_heads, block_size, head_dim], cache_dtype
 *                  (== src_dtype, or PA_FP8_E4M3)
 *   slot_mapping   [T] int64; a negative slot skips the token (padding)
 *   head_dim in {64, 128}; block_size in {8, 16, 32}; T >= 0 (T == 0 is a no-op).
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int32_t T, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int64_t num_blocks,
                               pa_dtype src_dtype, pa_dtype cache_dtype, float k_scale,
                               float v_scale, pa_stream_t stream);

/*
 * Bytes of device workspace pa_decode needs for these sizes (split-K
 * partial results and the work list).  A function of its arguments alone:
 * it covers every kernel choice on any gfx950 device (the split is planned
 * for at most 256 compute units and 8 waves on each), so a workspace sized
 * once serves every device of the process.  max_context_len is the length
 * bound the decode call plans with: for a call given max_context_len <= 0,
 * pass max_blocks_per_seq * block_size here.  Returns 0 for B <= 0,
 * max_context_len <= 0 or sizes the calls refuse.
 */
size_t pa_decode_workspace_size(int32_t B, int32_t num_kv_heads, int32_t gqa_group,
                                int32_t head_dim, int32_t block_size, int32_t max_context_len);

/*
 * Paged decode attention.  For each sequence s < B and query head
 * i < num_kv_heads * gqa_group, with h = i / gqa_group and L = context_lens[s]:
 *   score[t] = scale * dot(q[s, i, :], K[t, h, :])                 for t < L
 *   out[s, i, :] = sum_t softmax(score)[t] * V[t, h, :]
 * where K[t, h, :] = k_scale * k_cache[block_tables[s][t / bs], h, t % bs, :]
 * (k_scale/v_scale apply to FP8 caches only; they are ignored otherwise).
 * L == 0 gives an all-zero row.  The result does not depend on where the
 * blocks sit in the pool: reduction order depends only on logical positions.
 *   out            [B, num_kv_heads*gqa_group, head_dim], out_dtype (F32 | F16 | BF16);
 *                  16-bit outputs are the fp32 result rounded to nearest even
 *   q              [B, num_kv_heads*gqa_group, head_dim], q_dtype (F16 | BF16)
 *   k_cache, v_cache [num_blocks, num_kv_heads, block_size, head_dim], cache_dtype
 *                  (== q_dtype, or PA_FP8_E4M3 with either q dtype)
 *   block_tables   [B, max_blocks_per_seq] int32; entries past a sequence's
 *                  last block are never read
 *   context_lens   [B] int32
 *   max_context_len host-side upper bound of context_lens (<= 0 means
 *                  max_blocks_per_seq * block_size); sizes the split-K plan
 *   workspace      device buffer of at least pa_decode_workspace_size(B,
 *                  num_kv_heads, gqa_group, head_dim, block_size,
 *                  max_context_len) bytes; its contents need no
 *                  initialisation and are scratch after the call.
 * Environment: PA_DECODE_VARIANT=valu|mfma forces one of the two kernel
 * families (default: MFMA for every group size; the VALU/DPP kernel is built
 * for groups 1 and 2, and forcing it at another group gives
 * PA_ERR_UNSUPPORTED).
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                    int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim, int32_t block_size,
                    int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                    float scale, float k_scale, float v_scale, pa_dtype q_dtype,
                    pa_dtype cache_dtype, pa_dtype out_dtype, void* workspace,
                    size_t workspace_bytes, pa_stream_t stream);

/*
 * Decode over shared prefixes, each read once per group ("Paged Attention
 * and Memory Efficiency ...", section "How PagedAttention borrows OS paging
 * ...": requests that share a prefix point at the same physical blocks;
 * "PagedAttention - The KV Cache Problem", section "Why This Matters for
 * Production": parallel sampling and beam search).  The result is pa_decode's
 * for the same arguments; only the reading differs.  Group p is sequences
 * group_start[p] .. group_start[p + 1] - 1, which share their first
 * prefix_lens[p] positions: each member's K/V rows at those positions equal
 * the group's first member's (the same blocks, or copy-on-write copies of
 * them).  The call attends the members' queries over that prefix together,
 * reading it once per group through the first member's block table, then
 * attends each sequence over its own positions from prefix_lens[p] on and
 * combines the two, exactly as softmax over all positions.
 *   group_start    [num_groups + 1] int32, device: non-decreasing from 0 to B
 *   prefix_lens    [num_groups] int32, device: 0 <= prefix_lens[p] <=
 *                  L_s - 1 for every member s (the newest position is its own)
 *   num_groups     1 .. B; max_group_size: host bound of members per group,
 *                  1 .. 1024; B <= 3072 (one launch per pass)
 *   workspace      at least pa_decode_shared_prefix_workspace_size(B,
 *                  num_groups, max_group_size, num_kv_heads, gqa_group,
 *                  head_dim, block_size, max_context_len) bytes (with
 *                  max_context_len <= 0 read as max_blocks_per_seq * block_size)
 * Caches: 16-bit with a query of the same dtype, or FP8 with a scale per
 * tensor.  group_start and prefix_lens outside these rules are part of the
 * device-side contract (PA_VIOLATION_PREFIX_GROUP in the checked build).
 * Every other argument and error is pa_decode's.
 */
size_t pa_decode_shared_prefix_workspace_size(int32_t B, int32_t num_groups, int32_t max_group_size,
                                              int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                                              int32_t block_size, int32_t max_context_len);
pa_status pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* group_start, const int32_t* prefix_lens, int32_t B,
                                  int32_t num_groups, int32_t max_group_size, int32_t num_kv_heads,
                                  int32_t gqa_group, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len, float scale, float k_scale,
                                  float v_scale, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                                  void* workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * Attention sinks plus a sliding window, token-exact ("Paged Attention and
 * Memory Efficiency ...", section "Eviction, compression, and the challenge
 * of fitting more KV cache into less memory": StreamingLLM keeps the first
 * few tokens as attention sinks next to a window of recent ones).  pa_decode
 * where sequence s (L = context_lens[s], clamped as pa_decode clamps it)
 * attends only to its positions t < sink_tokens and t >= L - window_tokens:
 *   out[s, i, :] = sum over those t of softmax(score)[t] * V[t, h, :]
 * The kernel reads only the blocks of the chunks of 32 positions that hold
 * such positions (the sink's and the window's), so a long sequence costs
 * about (sink + window) positions of K/V traffic, not L.  Over a table that
 * pa_bm_evict shortened with the same sink and window (whole blocks gone,
 * positions renumbered), the result is the same attention: the kept blocks
 * hold the first positions first and the last positions last.
 *   sink_tokens >= 0, window_tokens >= 1 (the newest position is always
 *   seen, so no row is empty for L > 0); L == 0 gives an all-zero row.
 * Every other argument, the workspace (pa_decode_workspace_size) and the
 * errors are those of pa_decode; the kernel is the MFMA one.
 */
pa_status pa_decode_window(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                           int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                           int32_t sink_tokens, int32_t window_tokens, float scale, float k_scale, float v_scale,
                           pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype, void* workspace,
                           size_t workspace_bytes, pa_stream_t stream);

/*
 * One decode step in one call: each sequence's new token row is appended
 * and the sequence then attends over all of its positions, the new one
 * included (the cache grows by one row per generated token: "Paged Attention
 * and Memory Efficiency ...", section "Why KV cache memory was the
 * bottleneck ...").  The result, out and both caches, equals
 *   pa_reshape_and_cache(key, value, slots) followed by pa_decode(...)
 * with slots[s] = block_tables[s][(L - 1) / bs] * bs + (L - 1) % bs for the
 * clamped length L = min(context_lens[s], max_context_len, M * bs) of each
 * sequence; a sequence with L == 0, or whose last block id lies outside the
 * pool, appends nothing.  The block of position L - 1 must be private to the
 * sequence (copy it first with pa_copy_blocks if it is shared).
 *   key, value     [B, num_kv_heads, head_dim] rows of position L - 1, src_dtype:
 *                  == cache_dtype for 16-bit caches, PA_F16 or PA_BF16 for
 *                  an FP8 cache (encoded as pa_reshape_and_cache does)
 *   every other argument as for pa_decode; the caches are written.
 * For 16-bit caches the decode kernel stores the rows itself and reads them
 * from key/value, so the call launches no scatter; for FP8 caches a scatter
 * runs first.  Errors are those of pa_decode and pa_reshape_and_cache; every
 * check that can refuse the call (arguments, workspace, kernel choice) runs
 * before anything is enqueued, so such a call has no effect.  Only a launch
 * the HIP runtime itself refuses (PA_ERR_HIP) can come after the FP8
 * scatter was enqueued; the appended rows may then be written.
 */
/*
 * FP8 or FP4 cache with one scale per (slot, kv head) row ("PagedAttention -
 * The KV Cache Problem", section "What's Still Unsolved": FP8/FP4 quantized
 * KV caches).  pa_reshape_and_cache_scaled writes each (token, head) row as
 * codes of fp32(x) / s with s = (largest |x| of the row, NaN left out) / qmax
 * in fp32 -- 1 for a row of zeros or one holding an infinity -- and stores s
 * at the row's place in the scale pools.
 *   PA_FP8_E4M3: qmax = 448, the encoder of pa_reshape_and_cache; a row is
 *                  head_dim bytes.
 *   PA_FP4_E2M1: qmax = 6; OCP E2M1 codes (0, 0.5, 1, 1.5, 2, 3, 4, 6 and
 *                  negatives; the element type of the OCP Microscaling
 *                  formats), nearest with ties to the even code, saturating
 *                  at 6, a NaN element stored as +0; two codes per byte,
 *                  element 2i in the low nibble, so a row is head_dim / 2
 *                  bytes and the caches are [num_blocks, num_kv_heads,
 *                  block_size, head_dim / 2].
 * A row's scale is fixed when the row is written, so appending one token at
 * a time never re-encodes earlier rows, and rows of very different
 * magnitudes keep their own precision.
 *   k_scales, v_scales [num_blocks, num_kv_heads, block_size] fp32 (device;
 *                  4 bytes per 128-byte FP8 row at head_dim 128, per 64-byte
 *                  FP4 row)
 *   cache_dtype    PA_FP8_E4M3 or PA_FP4_E2M1; key, value f16 or bf16;
 *                  slot_mapping as for pa_reshape_and_cache.
 * pa_decode_scaled is pa_decode over such a cache: K[t, h, :] =
 * k_scales[b, h, t % bs] * decode(k_cache[b, h, t % bs, :]) with
 * b = block_tables[s][t / bs], V likewise; the workspace is pa_decode's.
 * The kernel is the MFMA one for every group size.  pa_copy_blocks_scaled
 * is pa_copy_blocks for such a cache: it copies the blocks' rows and their
 * scales.
 */
pa_status pa_reshape_and_cache_scaled(const void* key, const void* value, void* k_cache, void* v_cache,
                                      float* k_scales, float* v_scales, const int64_t* slot_mapping, int32_t T,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                      pa_dtype src_dtype, pa_dtype cache_dtype, pa_stream_t stream);
pa_status pa_copy_blocks_scaled(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                                const int64_t* block_mapping, int32_t N, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int64_t num_blocks, pa_dtype cache_dtype, pa_stream_t stream);
pa_status pa_decode_scaled(void* out, const void* q, const void* k_cache, const void* v_cache, const float* k_scales,
                           const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
                           int32_t B, int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_context_len, float scale, pa_dtype q_dtype, pa_dtype cache_dtype,
                           pa_dtype out_dtype, void* workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * Several query tokens per sequence over the same paged cache: the tokens of
 * a chunked prefill, or the draft tokens a speculative decoder verifies
 * ("Paged Attention and Memory Efficiency ...", section "How vLLM turned
 * PagedAttention into a production serving engine": batched speculative
 * decoding and prefill next to decode; "PagedAttention in Production",
 * section "Deployment Architecture", "Inference Service Layer": a scheduling
 * strategy for the prefill and decode phases).  The n = query_start[s + 1] - query_start[s] queries of sequence s
 * are its last n positions (their K/V rows are in the cache already, with
 * context_lens[s] = L counting them), and query j of them sees positions
 * 0 .. L - n + j (causal within the chunk):
 *   out[query_start[s] + j, i, :] = sum_{t <= L-n+j} softmax_t(scale * q.K[t]) V[t]
 * with the head mapping, dtypes and scales of pa_decode.
 *   q, out         [total_queries, num_kv_heads*gqa_group, head_dim]
 *   query_start    [B + 1] int32 device array, non-decreasing, query_start[0] = 0,
 *                  query_start[B] = total_queries; 0 <= n <= min(max_queries, L)
 *                  (n larger than that is cut to it; a range outside the rows
 *                  is dropped: device-side contract)
 *   max_queries    host-side bound of n, 1 .. 1024; n = 1 everywhere is pa_decode
 *   workspace      at least pa_decode_multi_workspace_size(B, num_kv_heads,
 *                  gqa_group, head_dim, block_size, max_context_len, max_queries) bytes
 * The kernel is the MFMA one, its 16 columns being (query, head) pairs, for
 * every group size.
 */
size_t pa_decode_multi_workspace_size(int32_t B, int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                                      int32_t block_size, int32_t max_context_len, int32_t max_queries);
pa_status pa_decode_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                          int32_t B, int32_t total_queries, int32_t max_queries, int32_t num_kv_heads,
                          int32_t gqa_group, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t max_context_len, float scale, float k_scale,
                          float v_scale, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                          void* workspace, size_t workspace_bytes, pa_stream_t stream);

pa_status pa_decode_append(void* out, const void* q, void* k_cache, void* v_cache, const void* key,
                           const void* value, pa_dtype src_dtype, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t B, int32_t num_kv_heads, int32_t gqa_group,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_context_len, float scale, float k_scale,
                           float v_scale, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                           void* workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * pa_decode_append for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops that never call hipMalloc,
 * harnesses that forbid allocation.  It takes no workspace: the split-K
 * partials live in a scratch array the library holds in device memory,
 * 64 MiB on each device it runs on (set aside when the library's code is
 * loaded there, kept until the process ends; its address is looked up once
 * per device, on the first call there).  The call itself allocates and
 * frees nothing.  Sizes whose pa_decode_workspace_size(B, num_kv_heads,
 * gqa_group, head_dim, block_size, max_context_len) exceeds 64 MiB (with
 * max_context_len <= 0 read as max_blocks_per_seq * block_size) return
 * PA_ERR_WORKSPACE before anything is enqueued.  Every call on one device
 * shares that device's array: calls whose work may overlap on one device
 * (streams with no ordering between them) race and give unspecified
 * results; calls ordered on one stream, or by events, do not.  The array
 * needs no clearing: each call writes every part of it that it reads.
 * Otherwise, arguments, results and errors are those of pa_decode_append.
 */
pa_status pa_decode_append_noalloc(void* out, const void* q, void* k_cache, void* v_cache, const void* key,
                                   const void* value, pa_dtype src_dtype, const int32_t* block_tables,
                                   const int32_t* context_lens, int32_t B, int32_t num_kv_heads, int32_t gqa_group,
                                   int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                   int32_t max_blocks_per_seq, int32_t max_context_len, float scale, float k_scale,
                                   float v_scale, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                                   pa_stream_t stream);

/*
 * Copy-on-write: for each n < N with (src, dst) = block_mapping[n],
 *   k_cache[dst] = k_cache[src] and v_cache[dst] = v_cache[src]
 * byte for byte (whole [num_kv_heads, block_size, head_dim] chunks; an
 * FP4 chunk is [num_kv_heads, block_size, head_dim / 2] bytes).
 *   block_mapping  [N, 2] int64, device; pairs with an id outside
 *                  [0, num_blocks) or src == dst are skipped.
 * N == 0 is a no-op.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int32_t N,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, pa_dtype cache_dtype, pa_stream_t stream);

/*
 * Host block manager: the memory-management side of the paged cache.
 *   "Paged Attention and Memory Efficiency ...", section "How PagedAttention
 *   borrows OS paging ..." (block tables resolved at run time, blocks
 *   allocated on demand, waste only in the tail of the last block, shared
 *   prefixes, copy-on-write); "PagedAttention in Production", section "Core
 *   Principle" (blocks allocated on demand and returned to the pool when a
 *   request finishes); "PagedAttention - The KV Cache Problem", sections "How
 *   It Works" and "Why This Matters for Production" (copy-on-write for
 *   parallel sampling and beam search).
 * A fixed pool of num_blocks physical blocks of block_size tokens.  Each
 * sequence (any int64 id) has a block table that grows as tokens are
 * appended; forking shares all of a sequence's blocks (reference counts);
 * appending into a shared, partially filled last block first moves the
 * sequence onto a copy of it, reported as a (src, dst) pair that the caller
 * copies with pa_copy_blocks before writing the new rows; freeing a sequence
 * returns the blocks no other sequence references.  Free blocks are handed
 * out last-freed-first (a fresh pool hands out 0, 1, 2, ...).  Every call is
 * host-only, synchronous and not thread-safe; the manager owns its host
 * memory.  A call that fails changes nothing.
 */
typedef struct pa_block_manager pa_block_manager;

typedef struct {
  int64_t blocks_in_use;  /* physical blocks referenced by some table */
  int64_t blocks_free;
  int64_t shared_blocks;  /* blocks referenced by more than one table */
  int64_t slots_held;     /* sum over sequences of table length * block_size */
  int64_t tokens;         /* sum over sequences of their length */
  int64_t sequences;
} pa_bm_stats;

/* NULL on bad sizes (num_blocks outside [0, 2^31), block_size < 1) or no memory. */
pa_block_manager* pa_bm_create(int64_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* bm);
/* new empty sequence; PA_ERR_INVALID_ARG if the id exists */
pa_status pa_bm_add(pa_block_manager* bm, int64_t seq);
/* child shares every block of parent (and its length) */
pa_status pa_bm_fork(pa_block_manager* bm, int64_t parent, int64_t child);
/*
 * Reserve n >= 0 token slots at the end of seq: slots[0..n) receive the slot
 * ids (block * block_size + row).  *copied is 1 when a copy-on-write was
 * needed, with copy_pair[0..2) = (src, dst); else 0.  PA_ERR_NO_BLOCKS when
 * the pool cannot supply every block the append needs.
 */
pa_status pa_bm_append(pa_block_manager* bm, int64_t seq, int32_t n, int64_t* slots, int64_t* copy_pair,
                       int32_t* copied);
/*
 * Append n_tokens[i] tokens to seqs[i] for i < count, in order (each id at
 * most once): slots get the sum of n_tokens slot ids, sequence after
 * sequence; copy_pairs[0 .. 2 * *n_pairs) the copy-on-write pairs (at most one
 * per sequence, so room for 2 * count).  All or nothing: the blocks needed,
 * counted before any of the batch is applied, must be free, or the call
 * returns PA_ERR_NO_BLOCKS and changes nothing.
 */
pa_status pa_bm_append_batch(pa_block_manager* bm, const int64_t* seqs, int32_t count, const int32_t* n_tokens,
                             int64_t* slots, int64_t* copy_pairs, int32_t* n_pairs);
/*
 * Block-wise sliding-window eviction with attention sinks: keep the blocks
 * that hold the first sink_tokens positions and those that hold the last
 * window_tokens positions of seq, release the whole blocks in between (a
 * shared block loses one reference) and close the gap in the table.  The
 * sequence then holds its kept positions in order, renumbered from 0, so a
 * plain pa_decode over the new table attends exactly to the sink and the
 * recent window; its length shrinks by *dropped (a multiple of block_size,
 * 0 when nothing lies between).  Whole blocks only: at least sink_tokens
 * and window_tokens positions stay, at most block_size - 1 more of each,
 * and the block holding the newest position always stays (window 0 keeps
 * the block the next token goes into).
 * ("Paged Attention and Memory Efficiency ...", section "Eviction,
 * compression, and the challenge of fitting more KV cache into less
 * memory": initial sink tokens plus a window of recent ones, and eviction
 * of whole blocks of the paged layout without changing the kernel.)
 * PA_ERR_INVALID_ARG for an unknown id or a negative count.
 */
pa_status pa_bm_evict(pa_block_manager* bm, int64_t seq, int64_t sink_tokens, int64_t window_tokens,
                      int64_t* dropped);
/* return seq's blocks to the pool (those no other sequence references) */
pa_status pa_bm_free(pa_block_manager* bm, int64_t seq);
/* number of blocks of seq (-1 if unknown); writes min(that, capacity) ids to table if non-NULL */
int32_t pa_bm_table(const pa_block_manager* bm, int64_t seq, int32_t* table, int32_t capacity);
/*
 * Block tables of seqs[0..count) as rows of a [count, width] int32 matrix
 * (the layout pa_decode reads), and their lengths into context_lens[count] if
 * non-NULL.  pad != 0 writes -1 into every entry past a sequence's blocks;
 * pad == 0 leaves those entries as they were, so a caller that keeps one
 * matrix across decode steps writes only the block ids (pa_decode never reads
 * an entry past a sequence's ceil(length / block_size) blocks).
 * PA_ERR_INVALID_ARG for an unknown id or a table longer than width (then
 * nothing is written).
 */
pa_status pa_bm_tables(const pa_block_manager* bm, const int64_t* seqs, int32_t count, int32_t* tables,
                       int32_t width, int32_t* context_lens, int32_t pad);
/* length of seq in tokens, -1 if unknown */
int64_t pa_bm_length(const pa_block_manager* bm, int64_t seq);
pa_status pa_bm_get_stats(const pa_block_manager* bm, pa_bm_stats* out);

/*
 * Kernel timing, for benchmarks.  start_event and stop_event are hipEvent_t
 * handles the caller created (either may be NULL).  The next pa_decode,
 * pa_decode_append, pa_decode_scaled, pa_decode_multi, pa_decode_window or
 * pa_decode_shared_prefix call on this thread that launches its kernels
 * records start_event when its first attention kernel begins and stop_event
 * when its last attention kernel ends, on the call's stream (the start and
 * stop events of hipExtLaunchKernel), and the pair is then forgotten.  The
 * elapsed time between them is the attention kernel alone (for
 * pa_decode_shared_prefix: its prefix pass through its suffix pass, the
 * merge between them included): the split merge and an FP8 append lie
 * outside it unless a batch runs as several launches (more sequences than
 * one launch takes: 4,096 for decode, 3,072 with several queries per
 * sequence, 2,048 for FP4 and for fp8 at block size 8, 512 for long query
 * chunks on the prefill kernel).
 * Always PA_OK.
 */
pa_status pa_time_next_attention_kernel(void* start_event, void* stop_event);

/*
 * Read-bandwidth probe, for benchmarks: the rate at which the device streams
 * bytes from HBM with the decode kernels' loads (16-byte nontemporal, 256
 * workgroups of eight waves, each wave with two batches of eight 1 KiB
 * loads in flight and whole chunks of chunk_bytes to itself), the measured
 * ceiling that decode bytes per second are set against.  No attention
 * arithmetic.
 *   buf          device buffer (16-byte aligned); its first
 *                floor(bytes / chunk_bytes) chunks are read once each
 *   chunk_bytes  a positive multiple of 1024
 *   sink         device buffer of at least 1024 bytes; it receives a fold of
 *                the bytes read (one word per workgroup: the XOR of the
 *                32-bit words it read), which keeps the loads from being
 *                optimised away
 * Asynchronous on stream; time it with events.  PA_ERR_INVALID_ARG for a
 * null or misaligned buffer, a bad chunk size or a small sink.
 */
pa_status pa_read_probe(const void* buf, size_t bytes, int32_t chunk_bytes, void* sink, size_t sink_bytes,
                        pa_stream_t stream);

/* Static description of a status code. */
const char* pa_status_string(pa_status s);

/* Thread-local description of the last error returned on this thread ("" if none). */
const char* pa_last_error_message(void);

/* Library version string. */
const char* pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
