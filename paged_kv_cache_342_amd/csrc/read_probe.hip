// Read-bandwidth probe for the benchmarks: the rate at which this device
// streams bytes from HBM with 16-byte nontemporal loads (the decode kernels'
// loads), two waves per SIMD and 8 to 16 KiB in flight per wave, each wave
// streaming whole chunks of the buffer.  It is
// the measured ceiling the decode's bytes per second are set against; it
// does no attention arithmetic.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kProbeWorkgroups = 256;
constexpr int kProbeThreads = 512;  // eight waves, two per SIMD
constexpr int kProbeBatch = 8;      // 1 KiB units a wave has in flight per batch (two batches)

// Wave w of the grid reads chunks w, w + W, w + 2 W, ... of chunk_bytes
// (W waves), each front to back in 1 KiB units (its v-th unit is unit
// v % upc of its (v / upc)-th chunk), in batches of kProbeBatch units, the
// next batch loaded before the current one is folded.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint8_t* __restrict__ buf,
                                                                  int64_t nchunks, int32_t chunk_bytes,
                                                                  uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kProbeThreads + threadIdx.x) >> 6;
  const int64_t W = ((int64_t)gridDim.x * kProbeThreads) >> 6;
  const int upc = chunk_bytes / 1024;
  const int64_t mine = wave < nchunks ? (nchunks - 1 - wave) / W + 1 : 0;  // chunks of this wave
  const int64_t vend = mine * upc;
  auto load = [&](int64_t v) -> i32x4 {
    if (v >= vend) return i32x4{0, 0, 0, 0};
    const int64_t c = wave + (v / upc) * W;
    return ld16_stream(buf + c * chunk_bytes + (v % upc) * 1024 + 16 * lane);
  };
  uint32_t x = 0;
  i32x4 cur[kProbeBatch];
  int64_t v0 = 0;
#pragma unroll
  for (int k = 0; k < kProbeBatch; ++k) cur[k] = load(v0 + k);
  while (v0 < vend) {
    const int64_t v1 = v0 + kProbeBatch;
    i32x4 nxt[kProbeBatch];
#pragma unroll
    for (int k = 0; k < kProbeBatch; ++k) nxt[k] = load(v1 + k);
#pragma unroll
    for (int k = 0; k < kProbeBatch; ++k) {
      x ^= (uint32_t)(cur[k][0] ^ cur[k][1] ^ cur[k][2] ^ cur[k][3]);
      cur[k] = nxt[k];
    }
    v0 = v1;
  }
  // fold the workgroup's lanes so the loads stay live
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x ^= (uint32_t)__shfl_xor((int)x, m);
  __shared__ uint32_t fold[kProbeThreads / 64];
  if (lane == 0) fold[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) y ^= fold[w];
    sink[blockIdx.x] = y;
  }
}

}  // namespace pa

extern "C" pa_status pa_read_probe(const void* buf, size_t bytes, int32_t chunk_bytes, void* sink, size_t sink_bytes,
                                   pa_stream_t stream) {
  using namespace pa;
  if (!buf || !sink) {
    set_error("pa_read_probe: null buffer or sink");
    return PA_ERR_INVALID_ARG;
  }
  if (chunk_bytes < 1024 || chunk_bytes % 1024 != 0 || (uintptr_t)buf % 16 != 0) {
    set_error("pa_read_probe: chunk_bytes must be a positive multiple of 1024 and buf 16-byte aligned");
    return PA_ERR_INVALID_ARG;
  }
  if (sink_bytes < (size_t)kProbeWorkgroups * sizeof(uint32_t)) {
    set_error("pa_read_probe: the sink takes %d bytes", (int)(kProbeWorkgroups * sizeof(uint32_t)));
    return PA_ERR_INVALID_ARG;
  }
  const int64_t nchunks = (int64_t)(bytes / (size_t)chunk_bytes);  // none: the sink still gets its zero folds
  hipLaunchKernelGGL(read_probe_kernel, dim3(kProbeWorkgroups), dim3(kProbeThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint8_t*>(buf), nchunks, chunk_bytes,
                     reinterpret_cast<uint32_t*>(sink));
  if (hipGetLastError() != hipSuccess) {
    set_error("pa_read_probe: launch failed");
    return PA_ERR_HIP;
  }
  return PA_OK;
}
