// pa_decode_append_noalloc: one decode step with the split-K partials in a
// scratch array the library holds in device memory, for callers that cannot
// allocate (see include/pa.h).
//
// The array is a file-scope __device__ array: each device the library runs
// on gets its own copy, at its own address, when the code object is loaded
// there, and keeps it until the process ends.  Host code never uses the
// array's name as an address (on the host it is only a stand-in for the
// symbol): the first call on a device asks the runtime for that device's
// address with hipGetSymbolAddress and keeps it, and kernels receive that
// address as their workspace.
#include <mutex>

#include "pa_internal.h"

namespace pa {

constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch`, looked up once per device.
static pa_status scratch_address(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("pa_decode_append_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
    return PA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("pa_decode_append_noalloc: device %d is beyond the %d the library keeps scratch for", dev, kMaxDevices);
    return PA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess || p == nullptr) {
      set_error("pa_decode_append_noalloc: hipGetSymbolAddress of the scratch array failed on device %d: %s", dev,
                hipGetErrorString(g));
      return PA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_decode_append_noalloc(void* out, const void* q, void* k_cache, void* v_cache,
                                              const void* key, const void* value, pa_dtype src_dtype,
                                              const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                              int32_t num_kv_heads, int32_t gqa_group, int32_t head_dim,
                                              int32_t block_size, int64_t num_blocks, int32_t max_blocks_per_seq,
                                              int32_t max_context_len, float scale, float k_scale, float v_scale,
                                              pa_dtype q_dtype, pa_dtype cache_dtype, pa_dtype out_dtype,
                                              pa_stream_t stream) {
  // Every argument check first (the workspace check comes last in
  // decode_request, so with none given a valid call stops there), then the
  // partials against the array, then the array's address.
  const char* fn = "pa_decode_append_noalloc";
  DecodeRequest r;
  pa_status st = decode_request(fn, out, q, k_cache, v_cache, block_tables, context_lens, B, num_kv_heads, gqa_group,
                                head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, k_scale,
                                v_scale, q_dtype, cache_dtype, out_dtype, nullptr, 0, 1, false, false, r);
  if (st != PA_OK && st != PA_ERR_WORKSPACE) return st;
  st = append_rows_check(fn, src_dtype, cache_dtype, key, value, B);
  if (st != PA_OK || B == 0) return st;
  const int32_t plan_ctx = max_context_len > 0 ? max_context_len : max_blocks_per_seq * block_size;
  const size_t need = pa_decode_workspace_size(B, num_kv_heads, gqa_group, head_dim, block_size, plan_ctx);
  if (need > kScratchBytes) {
    set_error("%s: these sizes need %zu bytes of scratch; the library holds %zu per device", fn, need,
              kScratchBytes);
    return PA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != PA_OK) return st;
  return pa_decode_append(out, q, k_cache, v_cache, key, value, src_dtype, block_tables, context_lens, B,
                          num_kv_heads, gqa_group, head_dim, block_size, num_blocks, max_blocks_per_seq,
                          max_context_len, scale, k_scale, v_scale, q_dtype, cache_dtype, out_dtype, ws,
                          kScratchBytes, stream);
}
