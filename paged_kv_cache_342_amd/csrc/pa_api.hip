// C entry points of libpa.so: argument validation and dispatch.  Every
// check runs before anything is enqueued, so a call that fails has no effect.
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "pa_internal.h"

namespace pa {

static thread_local char g_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
}

static pa_status fail(pa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return s;
}

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
static bool known_dtype(int d) { return d >= PA_F32 && d <= PA_FP4_E2M1; }
// bytes of one cache row of head_dim elements
static int64_t row_bytes(int head_dim, int d) {
  return d == PA_FP4_E2M1 ? head_dim / 2 : (int64_t)head_dim * (d == PA_FP8_E4M3 ? 1 : (d == PA_F32 ? 4 : 2));
}

#define PA_CHECK_SHAPE(fn, Hkv, D, bs, num_blocks)                                                  \
  do {                                                                                              \
    if ((Hkv) < 1) return fail(PA_ERR_INVALID_ARG, fn ": num_kv_heads must be >= 1 (got %d)", (Hkv)); \
    if ((num_blocks) < 1) return fail(PA_ERR_INVALID_ARG, fn ": num_blocks must be >= 1");          \
    if ((D) != 64 && (D) != 128) return fail(PA_ERR_UNSUPPORTED, fn ": head_dim must be 64 or 128 (got %d)", (D)); \
    if ((bs) != 8 && (bs) != 16 && (bs) != 32)                                                      \
      return fail(PA_ERR_UNSUPPORTED, fn ": block_size must be 8, 16 or 32 (got %d)", (bs));        \
  } while (0)

}  // namespace pa

using namespace pa;

extern "C" {

const char* pa_version(void) { return "pa-mi355x 0.1 (gfx950)"; }

const char* pa_last_error_message(void) { return g_error; }

int32_t pa_is_checked_build(void) {
#ifdef PA_CHECKED
  return 1;
#else
  return 0;
#endif
}

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks";
    case PA_ERR_CONTRACT: return "device-side contract violated";
  }
  return "unknown status";
}

pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                               const int64_t* slot_mapping, int32_t T, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int64_t num_blocks,
                               pa_dtype src_dtype, pa_dtype cache_dtype, float k_scale,
                               float v_scale, pa_stream_t stream) {
  g_error[0] = 0;
  const char* fn = "pa_reshape_and_cache";
  if (T < 0) return fail(PA_ERR_INVALID_ARG, "%s: T must be >= 0", fn);
  PA_CHECK_SHAPE("pa_reshape_and_cache", num_kv_heads, head_dim, block_size, num_blocks);
  if (!known_dtype(src_dtype) || !known_dtype(cache_dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype", fn);
  if (src_dtype != PA_F16 && src_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: source rows must be f16 or bf16", fn);
  if (cache_dtype == PA_FP4_E2M1)
    return fail(PA_ERR_UNSUPPORTED, "%s: fp4 caches take a scale per row (pa_reshape_and_cache_scaled)", fn);
  if (cache_dtype != src_dtype && cache_dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "%s: cache dtype must equal the source dtype or be fp8-e4m3", fn);
  if (cache_dtype == PA_FP8_E4M3 && !(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(PA_ERR_INVALID_ARG, "%s: fp8 scales must be finite and > 0", fn);
  if (!k_cache || !v_cache) return fail(PA_ERR_INVALID_ARG, "%s: null cache pointer", fn);
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16)) return fail(PA_ERR_INVALID_ARG, "%s: cache pointers must be 16-byte aligned", fn);
  if (T == 0) return PA_OK;
  if (!key || !value || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "%s: null key/value/slot_mapping", fn);
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID_ARG, "%s: misaligned key/value/slot_mapping", fn);
  PA_CONTRACT(check_slots_contract(fn, slot_mapping, T, num_blocks * block_size, reinterpret_cast<hipStream_t>(stream)));
  return scatter_launch(key, value, k_cache, v_cache, slot_mapping, T, num_kv_heads, head_dim, block_size,
                        num_blocks, src_dtype, cache_dtype, k_scale, v_scale, reinterpret_cast<hipStream_t>(stream));
}

pa_status pa_time_next_attention_kernel(void* start_event, void* stop_event) {
  g_error[0] = 0;
  set_timing_events(reinterpret_cast<hipEvent_t>(start_event), reinterpret_cast<hipEvent_t>(stop_event));
  return PA_OK;
}

size_t pa_decode_workspace_size(int32_t B, int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                                int32_t block_size, int32_t max_context_len) {
  if (B <= 0 || num_kv_heads <= 0 || gqa_group <= 0 || max_context_len <= 0) return 0;
  if ((head_dim != 64 && head_dim != 128) || (block_size != 8 && block_size != 16 && block_size != 32)) return 0;
  // one query-head tile per KV head gives the most slices of any kernel choice
  return decode_workspace_bound(B, num_kv_heads, gqa_group, head_dim, block_size, max_context_len, 1, false);
}

}  // extern "C"

namespace pa {

// Checks shared by pa_decode and pa_decode_append; fills r on success.
pa_status decode_request(const char* fn, void* out, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                int32_t B, int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                                int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                                int32_t max_context_len, float scale, float k_scale, float v_scale,
                                pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype, void* workspace,
                                size_t workspace_bytes, int nq, bool multi_query, bool row_scales,
                                DecodeRequest& r) {
  if (B < 0) return fail(PA_ERR_INVALID_ARG, "%s: B must be >= 0", fn);
  if (B > 65535) return fail(PA_ERR_UNSUPPORTED, "%s: at most 65535 sequences per call", fn);
  if (num_kv_heads < 1) return fail(PA_ERR_INVALID_ARG, "%s: num_kv_heads must be >= 1 (got %d)", fn, num_kv_heads);
  if (num_blocks < 1) return fail(PA_ERR_INVALID_ARG, "%s: num_blocks must be >= 1", fn);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim must be 64 or 128 (got %d)", fn, head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size must be 8, 16 or 32 (got %d)", fn, block_size);
  if (gqa_group < 1) return fail(PA_ERR_INVALID_ARG, "%s: gqa_group must be >= 1", fn);
  if ((int64_t)num_kv_heads * gqa_group > 65536) return fail(PA_ERR_UNSUPPORTED, "%s: too many query heads", fn);
  if (max_blocks_per_seq < 1) return fail(PA_ERR_INVALID_ARG, "%s: max_blocks_per_seq must be >= 1", fn);
  if ((int64_t)max_blocks_per_seq * block_size > (1 << 30)) return fail(PA_ERR_UNSUPPORTED, "%s: block table too long", fn);
  if (!known_dtype(q_dtype) || !known_dtype(cache_dtype) || !known_dtype(out_dtype))
    return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype", fn);
  if (q_dtype != PA_F16 && q_dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "%s: q must be f16 or bf16", fn);
  if (cache_dtype == PA_FP4_E2M1 && !row_scales)
    return fail(PA_ERR_UNSUPPORTED, "%s: fp4 caches take a scale per row (pa_decode_scaled)", fn);
  if (cache_dtype != q_dtype && cache_dtype != PA_FP8_E4M3 && cache_dtype != PA_FP4_E2M1)
    return fail(PA_ERR_UNSUPPORTED, "%s: cache dtype must equal the q dtype or be fp8-e4m3 (or fp4-e2m1)", fn);
  if (out_dtype != PA_F32 && out_dtype != PA_F16 && out_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: out must be f32, f16 or bf16", fn);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "%s: scale must be finite", fn);
  if (cache_dtype == PA_FP8_E4M3 && !(std::isfinite(k_scale) && k_scale > 0.f && std::isfinite(v_scale) && v_scale > 0.f))
    return fail(PA_ERR_INVALID_ARG, "%s: fp8 scales must be finite and > 0", fn);
  r = DecodeRequest{};
  r.B = B;
  if (B == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "%s: misaligned pointer argument", fn);
  const int full = max_blocks_per_seq * block_size;
  const int plan_ctx = max_context_len > 0 ? max_context_len : full;
  r.out = out;
  r.q = q;
  r.k_cache = k_cache;
  r.v_cache = v_cache;
  r.block_tables = block_tables;
  r.context_lens = context_lens;
  r.Hkv = num_kv_heads;
  r.G = gqa_group;
  r.D = head_dim;
  r.bs = block_size;
  r.M = max_blocks_per_seq;
  r.plan_ctx = plan_ctx;
  r.max_ctx = plan_ctx < full ? plan_ctx : full;
  r.num_blocks = num_blocks;
  r.scale = scale;
  r.k_scale = k_scale;
  r.v_scale = v_scale;
  r.q_dtype = q_dtype;
  r.cache_dtype = cache_dtype;
  r.out_dtype = out_dtype;
  r.workspace = workspace;
  r.workspace_bytes = workspace_bytes;
  // last: a call whose every other argument is valid gets PA_ERR_WORKSPACE
  // with r filled (the shared-prefix call sizes its own workspace from it)
  const size_t need = decode_workspace_bound(B, num_kv_heads, gqa_group, head_dim, block_size, plan_ctx, nq,
                                             multi_query);
  if (!workspace || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(PA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  return PA_OK;
}

// The checks pa_decode_append adds to pa_decode's: the new rows' dtype and pointers.
pa_status append_rows_check(const char* fn, pa_dtype src_dtype, pa_dtype cache_dtype, const void* key,
                            const void* value, int32_t B) {
  if (!known_dtype(src_dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype", fn);
  if (cache_dtype == PA_FP8_E4M3 ? (src_dtype != PA_F16 && src_dtype != PA_BF16) : src_dtype != cache_dtype)
    return fail(PA_ERR_UNSUPPORTED, "%s: new rows must have the cache dtype (f16 or bf16 for an fp8 cache)", fn);
  if (B == 0) return PA_OK;
  if (!key || !value) return fail(PA_ERR_INVALID_ARG, "%s: null key/value", fn);
  if (!aligned(key, 16) || !aligned(value, 16)) return fail(PA_ERR_INVALID_ARG, "%s: misaligned key/value", fn);
  return PA_OK;
}

}  // namespace pa

extern "C" {

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                    int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim, int32_t block_size,
                    int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                    float scale, float k_scale, float v_scale, pa_dtype q_dtype,
                    pa_dtype cache_dtype, pa_dtype out_dtype, void* workspace,
                    size_t workspace_bytes, pa_stream_t stream) {
  g_error[0] = 0;
  DecodeRequest r;
  const pa_status st = decode_request("pa_decode", out, q, k_cache, v_cache, block_tables, context_lens, B,
                                      num_kv_heads, gqa_group, head_dim, block_size, num_blocks,
                                      max_blocks_per_seq, max_context_len, scale, k_scale, v_scale, q_dtype,
                                      cache_dtype, out_dtype, workspace, workspace_bytes, 1, false, false, r);
  if (st != PA_OK || B == 0) return st;
  PA_CONTRACT(check_decode_contract("pa_decode", r, reinterpret_cast<hipStream_t>(stream)));
  return decode_launch(r, reinterpret_cast<hipStream_t>(stream));
}

pa_status pa_decode_window(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                           int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                           int32_t sink_tokens, int32_t window_tokens, float scale, float k_scale, float v_scale,
                           pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype, void* workspace,
                           size_t workspace_bytes, pa_stream_t stream) {
  g_error[0] = 0;
  const char* fn = "pa_decode_window";
  if (sink_tokens < 0) return fail(PA_ERR_INVALID_ARG, "%s: sink_tokens must be >= 0 (got %d)", fn, sink_tokens);
  if (window_tokens < 1)
    return fail(PA_ERR_INVALID_ARG, "%s: window_tokens must be >= 1 (got %d)", fn, window_tokens);
  DecodeRequest r;
  const pa_status st = decode_request(fn, out, q, k_cache, v_cache, block_tables, context_lens, B, num_kv_heads,
                                      gqa_group, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                      max_context_len, scale, k_scale, v_scale, q_dtype, cache_dtype, out_dtype,
                                      workspace, workspace_bytes, 1, false, false, r);
  if (st != PA_OK || B == 0) return st;
  // lengths are at most 2^30 (max_blocks_per_seq * block_size), so larger
  // counts mean the same and are clamped to keep the index math in range
  r.sink = sink_tokens > (1 << 30) ? (1 << 30) : sink_tokens;
  r.window = window_tokens > (1 << 30) ? (1 << 30) : window_tokens;
  PA_CONTRACT(check_decode_contract(fn, r, reinterpret_cast<hipStream_t>(stream)));
  return decode_launch(r, reinterpret_cast<hipStream_t>(stream));
}

size_t pa_decode_shared_prefix_workspace_size(int32_t B, int32_t num_groups, int32_t max_group_size,
                                              int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                                              int32_t block_size, int32_t max_context_len) {
  if (B <= 0 || num_groups <= 0 || num_groups > B || max_group_size <= 0 || num_kv_heads <= 0 || gqa_group <= 0 ||
      max_context_len <= 0)
    return 0;
  if ((head_dim != 64 && head_dim != 128) || (block_size != 8 && block_size != 16 && block_size != 32)) return 0;
  if (max_group_size > kMaxQueries || B > cascade_max_sequences()) return 0;
  return cascade_workspace_bound(B, num_groups, max_group_size, num_kv_heads, gqa_group, head_dim, block_size,
                                 max_context_len);
}

pa_status pa_decode_shared_prefix(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* group_start, const int32_t* prefix_lens, int32_t B,
                                  int32_t num_groups, int32_t max_group_size, int32_t num_kv_heads,
                                  int32_t gqa_group, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                  int32_t max_blocks_per_seq, int32_t max_context_len, float scale, float k_scale,
                                  float v_scale, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                                  void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  g_error[0] = 0;
  const char* fn = "pa_decode_shared_prefix";
  if (max_group_size < 1 || max_group_size > kMaxQueries)
    return fail(PA_ERR_UNSUPPORTED, "%s: max_group_size must be in [1, %d] (got %d)", fn, kMaxQueries, max_group_size);
  DecodeRequest r;
  // every check of pa_decode but the workspace, which is this call's own
  pa_status st = decode_request(fn, out, q, k_cache, v_cache, block_tables, context_lens, B, num_kv_heads, gqa_group,
                                head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, k_scale,
                                v_scale, q_dtype, cache_dtype, out_dtype, nullptr, 0, 1, false, false, r);
  if (st != PA_ERR_WORKSPACE) return st;  // an invalid argument, or OK for B == 0
  if (num_groups < 1 || num_groups > B)
    return fail(PA_ERR_INVALID_ARG, "%s: num_groups must be in [1, B] (got %d)", fn, num_groups);
  if (B > cascade_max_sequences())
    return fail(PA_ERR_UNSUPPORTED, "%s: at most %d sequences per call", fn, cascade_max_sequences());
  if (!group_start || !prefix_lens || !aligned(group_start, 4) || !aligned(prefix_lens, 4))
    return fail(PA_ERR_INVALID_ARG, "%s: null or misaligned group_start / prefix_lens", fn);
  const size_t need = cascade_workspace_bound(B, num_groups, max_group_size, num_kv_heads, gqa_group, head_dim,
                                              block_size, r.plan_ctx);
  if (!workspace || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 256)) return fail(PA_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
  r.workspace = workspace;
  r.workspace_bytes = workspace_bytes;
  r.group_start = group_start;
  r.prefix_lens = prefix_lens;
  r.n_groups = num_groups;
  r.nq = max_group_size;
  PA_CONTRACT(check_decode_contract(fn, r, reinterpret_cast<hipStream_t>(stream)));
  return cascade_launch(r, reinterpret_cast<hipStream_t>(stream));
}

pa_status pa_decode_append(void* out, const void* q, void* k_cache, void* v_cache, const void* key,
                           const void* value, pa_dtype src_dtype, const int32_t* block_tables,
                           const int32_t* context_lens, int32_t B, int32_t num_kv_heads, int32_t gqa_group,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_context_len, float scale, float k_scale,
                           float v_scale, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                           void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  g_error[0] = 0;
  const char* fn = "pa_decode_append";
  DecodeRequest r;
  const pa_status st = decode_request(fn, out, q, k_cache, v_cache, block_tables, context_lens, B, num_kv_heads,
                                      gqa_group, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                      max_context_len, scale, k_scale, v_scale, q_dtype, cache_dtype, out_dtype,
                                      workspace, workspace_bytes, 1, false, false, r);
  if (st != PA_OK) return st;
  const pa_status sa = append_rows_check(fn, src_dtype, cache_dtype, key, value, B);
  if (sa != PA_OK || B == 0) return sa;
  r.new_k = key;
  r.new_v = value;
  r.src_dtype = src_dtype;
  PA_CONTRACT(check_decode_contract(fn, r, reinterpret_cast<hipStream_t>(stream)));
  return decode_launch(r, reinterpret_cast<hipStream_t>(stream));
}

pa_status pa_reshape_and_cache_scaled(const void* key, const void* value, void* k_cache, void* v_cache,
                                      float* k_scales, float* v_scales, const int64_t* slot_mapping, int32_t T,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                      pa_dtype src_dtype, pa_dtype cache_dtype, pa_stream_t stream) {
  g_error[0] = 0;
  const char* fn = "pa_reshape_and_cache_scaled";
  if (T < 0) return fail(PA_ERR_INVALID_ARG, "%s: T must be >= 0", fn);
  PA_CHECK_SHAPE("pa_reshape_and_cache_scaled", num_kv_heads, head_dim, block_size, num_blocks);
  if (!known_dtype(src_dtype) || !known_dtype(cache_dtype)) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype", fn);
  if (src_dtype != PA_F16 && src_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: source rows must be f16 or bf16", fn);
  if (cache_dtype != PA_FP8_E4M3 && cache_dtype != PA_FP4_E2M1)
    return fail(PA_ERR_UNSUPPORTED, "%s: row scales are for fp8-e4m3 and fp4-e2m1 caches", fn);
  if (!k_cache || !v_cache || !k_scales || !v_scales) return fail(PA_ERR_INVALID_ARG, "%s: null cache or scale pointer", fn);
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_scales, 16) || !aligned(v_scales, 16))
    return fail(PA_ERR_INVALID_ARG, "%s: cache and scale pointers must be 16-byte aligned", fn);
  if (T == 0) return PA_OK;
  if (!key || !value || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "%s: null key/value/slot_mapping", fn);
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID_ARG, "%s: misaligned key/value/slot_mapping", fn);
  PA_CONTRACT(check_slots_contract(fn, slot_mapping, T, num_blocks * block_size, reinterpret_cast<hipStream_t>(stream)));
  return scatter_rows_launch(key, value, k_cache, v_cache, k_scales, v_scales, slot_mapping, T, num_kv_heads,
                             head_dim, block_size, num_blocks, src_dtype, cache_dtype,
                             reinterpret_cast<hipStream_t>(stream));
}

pa_status pa_decode_scaled(void* out, const void* q, const void* k_cache, const void* v_cache, const float* k_scales,
                           const float* v_scales, const int32_t* block_tables, const int32_t* context_lens,
                           int32_t B, int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                           int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                           int32_t max_context_len, float scale, pa_dtype q_dtype, pa_dtype cache_dtype,
                           pa_dtype out_dtype, void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  g_error[0] = 0;
  const char* fn = "pa_decode_scaled";
  if (cache_dtype != PA_FP8_E4M3 && cache_dtype != PA_FP4_E2M1)
    return fail(PA_ERR_UNSUPPORTED, "%s: row scales are for fp8-e4m3 and fp4-e2m1 caches", fn);
  DecodeRequest r;
  const pa_status st = decode_request(fn, out, q, k_cache, v_cache, block_tables, context_lens, B, num_kv_heads,
                                      gqa_group, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                      max_context_len, scale, 1.f, 1.f, q_dtype, cache_dtype, out_dtype, workspace,
                                      workspace_bytes, 1, false, true, r);
  if (st != PA_OK || B == 0) return st;
  if (!k_scales || !v_scales || !aligned(k_scales, 16) || !aligned(v_scales, 16))
    return fail(PA_ERR_INVALID_ARG, "%s: null or misaligned scale pools", fn);
  r.k_row_scale = k_scales;
  r.v_row_scale = v_scales;
  PA_CONTRACT(check_decode_contract(fn, r, reinterpret_cast<hipStream_t>(stream)));
  return decode_launch(r, reinterpret_cast<hipStream_t>(stream));
}

size_t pa_decode_multi_workspace_size(int32_t B, int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                                      int32_t block_size, int32_t max_context_len, int32_t max_queries) {
  if (B <= 0 || num_kv_heads <= 0 || gqa_group <= 0 || max_context_len <= 0 || max_queries <= 0) return 0;
  if ((head_dim != 64 && head_dim != 128) || (block_size != 8 && block_size != 16 && block_size != 32)) return 0;
  if (max_queries > kMaxQueries) return 0;
  return decode_workspace_bound(B, num_kv_heads, gqa_group, head_dim, block_size, max_context_len, max_queries,
                                true);
}

pa_status pa_decode_multi(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                          int32_t B, int32_t total_queries, int32_t max_queries, int32_t num_kv_heads,
                          int32_t gqa_group, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t max_context_len, float scale, float k_scale,
                          float v_scale, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                          void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  g_error[0] = 0;
  const char* fn = "pa_decode_multi";
  if (max_queries < 1 || max_queries > kMaxQueries)
    return fail(PA_ERR_UNSUPPORTED, "%s: max_queries must be in [1, %d] (got %d)", fn, kMaxQueries, max_queries);
  if (total_queries < 0) return fail(PA_ERR_INVALID_ARG, "%s: total_queries must be >= 0", fn);
  if ((int64_t)total_queries * num_kv_heads * gqa_group > ((int64_t)1 << 31))
    return fail(PA_ERR_UNSUPPORTED, "%s: too many query rows", fn);
  DecodeRequest r;
  const pa_status st = decode_request(fn, out, q, k_cache, v_cache, block_tables, context_lens, B, num_kv_heads,
                                      gqa_group, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                      max_context_len, scale, k_scale, v_scale, q_dtype, cache_dtype, out_dtype,
                                      workspace, workspace_bytes, max_queries, true, false, r);
  if (st != PA_OK) return st;
  if (B == 0 || total_queries == 0) return PA_OK;
  if (!query_start || !aligned(query_start, 4)) return fail(PA_ERR_INVALID_ARG, "%s: null or misaligned query_start", fn);
  r.q_start = query_start;
  r.nq = max_queries;
  r.q_rows = total_queries;
  PA_CONTRACT(check_decode_contract(fn, r, reinterpret_cast<hipStream_t>(stream)));
  return decode_launch(r, reinterpret_cast<hipStream_t>(stream));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int32_t N,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, pa_dtype cache_dtype, pa_stream_t stream) {
  g_error[0] = 0;
  const char* fn = "pa_copy_blocks";
  if (N < 0) return fail(PA_ERR_INVALID_ARG, "%s: N must be >= 0", fn);
  PA_CHECK_SHAPE("pa_copy_blocks", num_kv_heads, head_dim, block_size, num_blocks);
  if (!known_dtype(cache_dtype) || cache_dtype == PA_F32)
    return fail(PA_ERR_UNSUPPORTED, "%s: cache dtype must be f16, bf16 or fp8-e4m3", fn);
  if (!k_cache || !v_cache) return fail(PA_ERR_INVALID_ARG, "%s: null cache pointer", fn);
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16)) return fail(PA_ERR_INVALID_ARG, "%s: cache pointers must be 16-byte aligned", fn);
  if (N == 0) return PA_OK;
  if (!block_mapping || !aligned(block_mapping, 8)) return fail(PA_ERR_INVALID_ARG, "%s: null or misaligned block_mapping", fn);
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * row_bytes(head_dim, cache_dtype);
  PA_CONTRACT(check_pairs_contract(fn, block_mapping, N, num_blocks, reinterpret_cast<hipStream_t>(stream)));
  return copy_blocks_launch(k_cache, v_cache, block_mapping, N, block_bytes, num_blocks,
                            reinterpret_cast<hipStream_t>(stream));
}

pa_status pa_copy_blocks_scaled(void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                                const int64_t* block_mapping, int32_t N, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int64_t num_blocks, pa_dtype cache_dtype, pa_stream_t stream) {
  g_error[0] = 0;
  const char* fn = "pa_copy_blocks_scaled";
  if (N < 0) return fail(PA_ERR_INVALID_ARG, "%s: N must be >= 0", fn);
  PA_CHECK_SHAPE("pa_copy_blocks_scaled", num_kv_heads, head_dim, block_size, num_blocks);
  if (cache_dtype != PA_FP8_E4M3 && cache_dtype != PA_FP4_E2M1)
    return fail(PA_ERR_UNSUPPORTED, "%s: row scales are for fp8-e4m3 and fp4-e2m1 caches", fn);
  if (!k_cache || !v_cache || !k_scales || !v_scales) return fail(PA_ERR_INVALID_ARG, "%s: null cache or scale pointer", fn);
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_scales, 16) || !aligned(v_scales, 16))
    return fail(PA_ERR_INVALID_ARG, "%s: cache and scale pointers must be 16-byte aligned", fn);
  if (N == 0) return PA_OK;
  if (!block_mapping || !aligned(block_mapping, 8)) return fail(PA_ERR_INVALID_ARG, "%s: null or misaligned block_mapping", fn);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  PA_CONTRACT(check_pairs_contract(fn, block_mapping, N, num_blocks, st));
  const pa_status s1 = copy_blocks_launch(k_cache, v_cache, block_mapping, N,
                                          (int64_t)num_kv_heads * block_size * row_bytes(head_dim, cache_dtype),
                                          num_blocks, st);
  if (s1 != PA_OK) return s1;
  return copy_blocks_launch(k_scales, v_scales, block_mapping, N, (int64_t)num_kv_heads * block_size * 4, num_blocks,
                            st);
}

}  // extern "C"
