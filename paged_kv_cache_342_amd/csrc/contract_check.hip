// Device-side contract checks of the checked build (libpa_checked.so, built
// with PA_CHECKED).  The contract of include/pa.h constrains device arrays
// the host never reads: block ids, context lengths, slots, copy pairs and
// query ranges.  In the checked build every entry point first runs the
// kernels below over those arrays; each sets bits (PA_VIOLATION_*) in one
// device-resident word.  The entry point then waits for its stream, reads and
// clears the word, and rejects the call with PA_ERR_CONTRACT before anything
// else is enqueued, so a rejected call has no effect.  Under stream capture
// it cannot wait: the check kernels are captured with the work and a
// violation is reported by the next call made outside a capture.
//
// The checks read only what the contract bounds by host-known sizes (rows
// [0, ceil(clamped L / bs)) of each table row, B + 1 query starts, T slots,
// N pairs), so they are safe to run on arrays that violate the contract.
#include <cstdio>

#include "pa_internal.h"

namespace pa {

static __device__ uint32_t g_violations = 0;

// The word's device address on the current device (one copy per device).
static uint32_t* violation_word() {
  static uint32_t* cache[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (cache[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_violations)) != hipSuccess) return nullptr;
    cache[dev] = reinterpret_cast<uint32_t*>(p);
  }
  return cache[dev];
}

__device__ __forceinline__ void flag(uint32_t* word, uint32_t bits) { atomicOr(word, bits); }

// One wave per sequence: its length, the table entries it reads and, with
// several queries per sequence, its query range.
__global__ __launch_bounds__(64) void check_tables_kernel(const int32_t* tables, const int32_t* lens,
                                                          const int32_t* q_start, int B, int M, int bs,
                                                          int max_ctx, int64_t num_blocks, int nq, int q_rows,
                                                          uint32_t* word) {
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  if (s >= B) return;
  const int L = lens[s];
  uint32_t bits = 0;
  if (lane == 0 && (L < 0 || L > max_ctx)) bits |= PA_VIOLATION_CONTEXT_LEN;
  const int Lc = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
  const int nblk = (Lc + bs - 1) / bs;  // <= M, since max_ctx <= M * bs
  for (int j = lane; j < nblk; j += 64) {
    const int id = tables[(int64_t)s * M + j];
    if (id < 0 || (int64_t)id >= num_blocks) bits |= PA_VIOLATION_BLOCK_ID;
  }
  if (q_start != nullptr && lane == 0) {
    const int a = q_start[s], b = q_start[s + 1];
    if (b < a || b - a > nq || b - a > Lc || a < 0 || b > q_rows) bits |= PA_VIOLATION_QUERY_START;
    if ((s == 0 && a != 0) || (s == B - 1 && b != q_rows)) bits |= PA_VIOLATION_QUERY_START;
  }
  if (bits) flag(word, bits);
}

constexpr int kTile = 256;

// pa_decode_append: the block that receives a sequence's new row (its block
// of position L - 1) must be read by no other sequence of the call, nor
// twice by its own table, since the decode kernel stores the row while
// other waves of the launch read.  One wave per sequence s compares every
// table entry s reads with the tail block of every sequence t, 64 tails at a
// time from LDS; the entry that is t's own tail (t == s, at its index) is
// the one allowed match.
__global__ __launch_bounds__(64) void check_append_kernel(const int32_t* tables, const int32_t* lens, int B, int M,
                                                          int bs, int max_ctx, uint32_t* word) {
  __shared__ int tail_id[64];
  __shared__ int tail_j[64];
  const int s = blockIdx.x;
  const int lane = threadIdx.x;
  if (s >= B) return;
  auto blocks_of = [&](int t) {
    const int L = lens[t];
    const int Lc = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
    return (Lc + bs - 1) / bs;  // <= M, since max_ctx <= M * bs
  };
  const int nblk = blocks_of(s);
  bool shared = false;
  for (int t0 = 0; t0 < B; t0 += 64) {
    __syncthreads();
    const int t = t0 + lane;
    const int nb = t < B ? blocks_of(t) : 0;
    tail_j[lane] = nb - 1;
    tail_id[lane] = nb > 0 ? tables[(int64_t)t * M + nb - 1] : -1;
    __syncthreads();
    const int n = B - t0 < 64 ? B - t0 : 64;
    for (int j = lane; j < nblk; j += 64) {
      const int id = tables[(int64_t)s * M + j];
      for (int u = 0; u < n; ++u)
        if (tail_j[u] >= 0 && tail_id[u] == id && !(t0 + u == s && j == tail_j[u])) shared = true;
    }
  }
  if (shared) flag(word, PA_VIOLATION_APPEND_BLOCK_SHARED);
}

// pa_decode_shared_prefix: group_start rises from 0 to B, each group has at
// most max_group members, and its prefix length is at least 0 and below the
// (clamped) length of each member.  One thread per group.
__global__ __launch_bounds__(kTile) void check_groups_kernel(const int32_t* group_start, const int32_t* prefix_lens,
                                                             const int32_t* lens, int P, int B, int max_group,
                                                             int max_ctx, uint32_t* word) {
  const int p = blockIdx.x * kTile + threadIdx.x;
  if (p >= P) return;
  const int a = group_start[p], b = group_start[p + 1], pl = prefix_lens[p];
  bool bad = b < a || b - a > max_group || a < 0 || b > B || pl < 0;
  if ((p == 0 && a != 0) || (p == P - 1 && b != B)) bad = true;
  for (int s = a < 0 ? 0 : a; !bad && s < (b > B ? B : b); ++s) {
    const int L = lens[s];
    const int Lc = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
    if (pl > Lc - 1) bad = true;
  }
  if (bad) flag(word, PA_VIOLATION_PREFIX_GROUP);
}

// Slots: each non-negative slot lies below num_slots and appears once.  Thread
// i compares its slot with every later one, a tile of 256 at a time from LDS.
__global__ __launch_bounds__(kTile) void check_slots_kernel(const int64_t* slots, int T, int64_t num_slots,
                                                            uint32_t* word) {
  __shared__ int64_t tile[kTile];
  const int i = blockIdx.x * kTile + threadIdx.x;
  const int64_t mine = i < T ? slots[i] : -1;
  uint32_t bits = 0;
  if (mine >= num_slots) bits |= PA_VIOLATION_SLOT;
  for (int j0 = blockIdx.x * kTile; j0 < T; j0 += kTile) {
    __syncthreads();
    const int j = j0 + threadIdx.x;
    tile[threadIdx.x] = j < T ? slots[j] : -1;
    __syncthreads();
    if (mine >= 0) {
      const int n = T - j0 < kTile ? T - j0 : kTile;
      for (int u = 0; u < n; ++u)
        if (j0 + u > i && tile[u] == mine) bits |= PA_VIOLATION_SLOT_REPEATED;
    }
  }
  if (bits) flag(word, bits);
}

// Copy pairs: ids inside the pool, distinct destinations, and no destination
// that is the source of another pair (a pair with src == dst is a no-op).
__global__ __launch_bounds__(kTile) void check_pairs_kernel(const int64_t* pairs, int N, int64_t num_blocks,
                                                            uint32_t* word) {
  __shared__ int64_t src_t[kTile], dst_t[kTile];
  const int i = blockIdx.x * kTile + threadIdx.x;
  const int64_t src = i < N ? pairs[2 * (int64_t)i] : -1;
  const int64_t dst = i < N ? pairs[2 * (int64_t)i + 1] : -1;
  uint32_t bits = 0;
  if (i < N && (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks)) bits |= PA_VIOLATION_COPY_ID;
  for (int j0 = 0; j0 < N; j0 += kTile) {
    __syncthreads();
    const int j = j0 + threadIdx.x;
    src_t[threadIdx.x] = j < N ? pairs[2 * (int64_t)j] : -2;
    dst_t[threadIdx.x] = j < N ? pairs[2 * (int64_t)j + 1] : -2;
    __syncthreads();
    if (i < N) {
      const int n = N - j0 < kTile ? N - j0 : kTile;
      for (int u = 0; u < n; ++u) {
        if (j0 + u == i) continue;
        if (dst_t[u] == dst) bits |= PA_VIOLATION_COPY_DST_REPEATED;
        if (src_t[u] == dst && src_t[u] != dst_t[u]) bits |= PA_VIOLATION_COPY_DST_IS_SRC;
      }
    }
  }
  if (bits) flag(word, bits);
}

static void describe(uint32_t bits, char* buf, size_t n) {
  static const struct {
    uint32_t bit;
    const char* what;
  } names[] = {
      {PA_VIOLATION_BLOCK_ID, "a block table entry outside [0, num_blocks)"},
      {PA_VIOLATION_CONTEXT_LEN, "a context length outside [0, max_context_len]"},
      {PA_VIOLATION_SLOT, "a slot at or beyond num_blocks * block_size"},
      {PA_VIOLATION_SLOT_REPEATED, "a slot given twice"},
      {PA_VIOLATION_COPY_ID, "a copy pair id outside [0, num_blocks)"},
      {PA_VIOLATION_COPY_DST_REPEATED, "a copy destination given twice"},
      {PA_VIOLATION_COPY_DST_IS_SRC, "a copy destination that is another pair's source"},
      {PA_VIOLATION_QUERY_START, "a query range outside the contract"},
      {PA_VIOLATION_APPEND_BLOCK_SHARED, "a block receiving a new row that another table entry of the call reads"},
      {PA_VIOLATION_PREFIX_GROUP, "a prefix group or prefix length outside the contract"},
  };
  size_t used = 0;
  buf[0] = 0;
  for (const auto& e : names) {
    if (!(bits & e.bit) || used + 4 >= n) continue;
    used += std::snprintf(buf + used, n - used, "%s%s", used ? "; " : "", e.what);
  }
}

// Waits for the stream and turns the word into a status (and clears it).
static pa_status collect(const char* fn, uint32_t* word, hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess) {
    set_error("%s: contract check: hipStreamIsCapturing failed", fn);
    return PA_ERR_HIP;
  }
  if (cap != hipStreamCaptureStatusNone) return PA_OK;  // reported by a later call
  uint32_t bits = 0;
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(&bits, word, sizeof(bits), hipMemcpyDeviceToHost) != hipSuccess) {
    set_error("%s: contract check: reading the violation word failed", fn);
    return PA_ERR_HIP;
  }
  if (bits == 0) return PA_OK;
  const uint32_t zero = 0;
  if (hipMemcpy(word, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) {
    set_error("%s: contract check: clearing the violation word failed", fn);
    return PA_ERR_HIP;
  }
  char what[400];
  describe(bits, what, sizeof(what));
  set_error("%s: device-side contract violated (bits 0x%x): %s", fn, bits, what);
  return PA_ERR_CONTRACT;
}

static pa_status launched(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return PA_OK;
  set_error("%s: contract check launch failed: %s", fn, hipGetErrorString(e));
  return PA_ERR_HIP;
}

pa_status check_decode_contract(const char* fn, const DecodeRequest& r, hipStream_t stream) {
  uint32_t* word = violation_word();
  if (word == nullptr) {
    set_error("%s: contract check: no violation word on this device", fn);
    return PA_ERR_HIP;
  }
  hipLaunchKernelGGL(check_tables_kernel, dim3((unsigned)r.B), dim3(64), 0, stream, r.block_tables, r.context_lens,
                     r.q_start, r.B, r.M, r.bs, r.max_ctx, r.num_blocks, r.q_start ? r.nq : 1, r.q_rows, word);
  if (r.new_k != nullptr)
    hipLaunchKernelGGL(check_append_kernel, dim3((unsigned)r.B), dim3(64), 0, stream, r.block_tables, r.context_lens,
                       r.B, r.M, r.bs, r.max_ctx, word);
  if (r.group_start != nullptr)
    hipLaunchKernelGGL(check_groups_kernel, dim3((unsigned)((r.n_groups + kTile - 1) / kTile)), dim3(kTile), 0, stream,
                       r.group_start, r.prefix_lens, r.context_lens, r.n_groups, r.B, r.nq, r.max_ctx, word);
  const pa_status st = launched(fn);
  return st != PA_OK ? st : collect(fn, word, stream);
}

pa_status check_slots_contract(const char* fn, const int64_t* slots, int T, int64_t num_slots, hipStream_t stream) {
  uint32_t* word = violation_word();
  if (word == nullptr) {
    set_error("%s: contract check: no violation word on this device", fn);
    return PA_ERR_HIP;
  }
  hipLaunchKernelGGL(check_slots_kernel, dim3((unsigned)((T + kTile - 1) / kTile)), dim3(kTile), 0, stream, slots, T,
                     num_slots, word);
  const pa_status st = launched(fn);
  return st != PA_OK ? st : collect(fn, word, stream);
}

pa_status check_pairs_contract(const char* fn, const int64_t* pairs, int N, int64_t num_blocks, hipStream_t stream) {
  uint32_t* word = violation_word();
  if (word == nullptr) {
    set_error("%s: contract check: no violation word on this device", fn);
    return PA_ERR_HIP;
  }
  hipLaunchKernelGGL(check_pairs_kernel, dim3((unsigned)((N + kTile - 1) / kTile)), dim3(kTile), 0, stream, pairs, N,
                     num_blocks, word);
  const pa_status st = launched(fn);
  return st != PA_OK ? st : collect(fn, word, stream);
}

}  // namespace pa
