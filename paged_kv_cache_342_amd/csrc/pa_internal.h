// Host-side interfaces between the C entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// thread-local error text behind pa_last_error_message()
void set_error(const char* fmt, ...);

struct DecodePlan {
  int nslices;    // slices per (KV head, head tile): one wave each
  int min_slice;  // fewest chunks per slice
  int seg_cost;   // virtual chunks charged per non-empty sequence
  int sub_batch;  // sequences per launch
  size_t meta_off, ml_off, acc_off, bytes;  // workspace layout
};

// most queries per sequence pa_decode_multi takes
constexpr int kMaxQueries = 1024;
// A launch plans for at most this many compute units (every gfx950 part has
// 256; a device with more would use 256 of them for the split) and at most
// kMaxWavesPerCU waves on each, so that workspace sizes are a function of the
// call's arguments alone.
constexpr int kPlanMaxCUs = 256;
constexpr int kMaxWavesPerCU = 8;

// compute units of the current device (cached per device)
int device_cu_count();

// waves: slices are planned for this many waves in the grid.
// nq: queries per sequence at most (1 for decode); partial rows scale with it.
// multi_query: the launch uses the several-queries kernel (fewer sequences per launch).
// two_waves: the kernel runs two waves per SIMD (twice the slices, half the
// sequences per launch: mfma_two_waves()).
// scan_cap: sequences one launch takes at most (0: scan_capacity()).
// charge: chunks each sequence is charged on the line for its fixed costs
// (PA_DECODE_SEGMENT_COST overrides it); a larger charge never enlarges the
// workspace.
DecodePlan plan_decode(int B, int Hkv, int G, int D, int bs, int max_ctx, int head_tiles, int64_t waves, int nq,
                       bool multi_query, bool two_waves, int scan_cap = 0, int charge = 2);
// Workspace bytes that cover every kernel choice and device for these sizes
// (the most slices a launch can have, either occupancy).
size_t decode_workspace_bound(int B, int Hkv, int G, int D, int bs, int max_ctx, int nq, bool multi_query);

// Events an attention-kernel launch records (hipExtLaunchKernel's start and
// stop events; null = not recorded).
struct LaunchEvents {
  hipEvent_t start;
  hipEvent_t stop;
};
// The pair the next decode call on this thread records around its attention
// kernels (pa_time_next_attention_kernel).
void set_timing_events(hipEvent_t start, hipEvent_t stop);

struct DecodeRequest {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int B, Hkv, G, D, bs, M;
  int max_ctx;   // lengths are clamped to this: min(plan_ctx, M * bs)
  int plan_ctx;  // the caller's max_context_len (M * bs when not given); sizes the plan
  int64_t num_blocks;
  float scale, k_scale, v_scale;
  int q_dtype, cache_dtype, out_dtype;
  void* workspace;
  size_t workspace_bytes;
  // appending the row of position L - 1 of every sequence in the same call
  // ([B, Hkv, D], src_dtype); null = plain decode
  const void* new_k;
  const void* new_v;
  int src_dtype;
  // several queries per sequence: rows q_start[s] .. q_start[s+1]-1 of q and
  // out ([q_rows, Hq, D]), at most nq per sequence; null = one per sequence
  const int32_t* q_start;
  int nq;
  int q_rows;
  // FP8 cache with a scale per (slot, kv head) row ([num_blocks, Hkv, bs]
  // fp32 each); null = one scale per tensor
  const float* k_row_scale;
  const float* v_row_scale;
  // attention sinks plus a sliding window (pa_decode_window): each sequence
  // attends to t < sink and t >= L - window; window == 0 = every position
  int sink;
  int window;
  // shared prefixes (pa_decode_shared_prefix): group p is sequences
  // group_start[p] .. group_start[p + 1] - 1 (device, [n_groups + 1]), which
  // share their first prefix_lens[p] positions (device, [n_groups]); nq is
  // then the largest group
  const int32_t* group_start;
  const int32_t* prefix_lens;
  int n_groups;
};

// Workspace bytes of pa_decode_shared_prefix: the prefix pass's plan over
// the groups, the suffix pass's plan over the sequences and the members'
// states, for any device (as decode_workspace_bound).
size_t cascade_workspace_bound(int B, int n_groups, int max_group, int Hkv, int G, int D, int bs, int max_ctx);
// Most sequences (and groups) one pa_decode_shared_prefix call takes: each
// pass runs as a single launch.
int cascade_max_sequences();
pa_status cascade_launch(const DecodeRequest& r, hipStream_t stream);

// 0 = default choice, 1 = VALU/DPP kernel, 2 = MFMA kernel
int decode_variant_override();
bool decode_uses_valu(int variant, int G);

pa_status decode_launch(const DecodeRequest& r, hipStream_t stream);

// Host checks of the decode calls (pa_api.hip): decode_request validates
// everything pa_decode takes and fills r, the workspace last (so a call with
// no workspace that passes every other check gives PA_ERR_WORKSPACE);
// append_rows_check adds pa_decode_append's checks of the new rows.
pa_status decode_request(const char* fn, void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens, int32_t B, int32_t num_kv_heads,
                         int32_t gqa_group, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                         int32_t max_blocks_per_seq, int32_t max_context_len, float scale, float k_scale,
                         float v_scale, pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype, void* workspace,
                         size_t workspace_bytes, int nq, bool multi_query, bool row_scales, DecodeRequest& r);
pa_status append_rows_check(const char* fn, pa_dtype src_dtype, pa_dtype cache_dtype, const void* key,
                            const void* value, int32_t B);

pa_status scatter_launch(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slots, int T, int Hkv, int D, int bs, int64_t num_blocks,
                         int src_dtype, int cache_dtype, float k_scale, float v_scale,
                         hipStream_t stream);

pa_status scatter_rows_launch(const void* key, const void* value, void* k_cache, void* v_cache, float* k_scales,
                              float* v_scales, const int64_t* slots, int T, int Hkv, int D, int bs,
                              int64_t num_blocks, int src_dtype, int cache_dtype, hipStream_t stream);

pa_status append_last_launch(const void* key, const void* value, void* k_cache, void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens, int B, int M,
                             int max_ctx, int Hkv, int D, int bs, int64_t num_blocks, int src_dtype,
                             int cache_dtype, float k_scale, float v_scale, hipStream_t stream);

pa_status copy_blocks_launch(void* k_cache, void* v_cache, const int64_t* pairs, int N,
                             int64_t block_bytes, int64_t num_blocks, hipStream_t stream);

// Checked build (PA_CHECKED): device-side contract checks run before a
// call's work; PA_ERR_CONTRACT when violated (contract_check.hip).
pa_status check_decode_contract(const char* fn, const DecodeRequest& r, hipStream_t stream);
pa_status check_slots_contract(const char* fn, const int64_t* slots, int T, int64_t num_slots, hipStream_t stream);
pa_status check_pairs_contract(const char* fn, const int64_t* pairs, int N, int64_t num_blocks, hipStream_t stream);

#ifdef PA_CHECKED
#define PA_CONTRACT(call)              \
  do {                                 \
    const pa_status cst_ = (call);     \
    if (cst_ != PA_OK) return cst_;    \
  } while (0)
#else
#define PA_CONTRACT(call) \
  do {                    \
  } while (0)
#endif

}  // namespace pa
