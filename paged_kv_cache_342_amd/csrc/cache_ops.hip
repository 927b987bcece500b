// Slot scatter (appending new tokens' K/V rows) and copy-on-write block copy.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// E4M3FN code of fp32(x) / scale: IEEE division, round to nearest even in
// the hardware convert, magnitudes beyond 448 saturate, NaN stays NaN.
__device__ __forceinline__ float fp8_prescale(float x, float scale) {
  const float y = x / scale;
  return y != y ? y : fminf(fmaxf(y, -448.0f), 448.0f);
}

// The hardware convert writes every NaN as the negative NaN code (0xFF);
// E4M3FN has a NaN of each sign (S.1111.111), so the input's sign is put
// back for NaN inputs.
__device__ __forceinline__ uint32_t keep_nan_sign(uint32_t w, const float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (x[i] != x[i]) {
      const uint32_t code = 0x7Fu | ((__float_as_uint(x[i]) >> 24) & 0x80u);
      w = (w & ~(0xFFu << (8 * i))) | (code << (8 * i));
    }
  }
  return w;
}

__device__ __forceinline__ i32x2 encode8_fp8(const float* x, float scale) {
  int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_prescale(x[0], scale), fp8_prescale(x[1], scale), 0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_prescale(x[2], scale), fp8_prescale(x[3], scale), w0, true);
  int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_prescale(x[4], scale), fp8_prescale(x[5], scale), 0, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(fp8_prescale(x[6], scale), fp8_prescale(x[7], scale), w1, true);
  return i32x2{(int)keep_nan_sign((uint32_t)w0, x), (int)keep_nan_sign((uint32_t)w1, x + 4)};
}

// 8 elements of a K and a V row into the caches at element offset dst_elem.
template <class ST, bool kFp8>
__device__ __forceinline__ void store_row8(i32x4 kx, i32x4 vx, uint8_t* __restrict__ k_cache,
                                           uint8_t* __restrict__ v_cache, int64_t dst_elem, float k_scale,
                                           float v_scale) {
  if constexpr (!kFp8) {
    *reinterpret_cast<i32x4*>(k_cache + dst_elem * 2) = kx;
    *reinterpret_cast<i32x4*>(v_cache + dst_elem * 2) = vx;
  } else {
    float kf[8], vf[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      unpack2<ST>((uint32_t)kx[w], kf[2 * w], kf[2 * w + 1]);
      unpack2<ST>((uint32_t)vx[w], vf[2 * w], vf[2 * w + 1]);
    }
    *reinterpret_cast<i32x2*>(k_cache + dst_elem) = encode8_fp8(kf, k_scale);
    *reinterpret_cast<i32x2*>(v_cache + dst_elem) = encode8_fp8(vf, v_scale);
  }
}

// One thread per 8 elements of one (token, kv head) row.
template <class ST, bool kFp8>
__global__ __launch_bounds__(256) void scatter_kernel(const uint8_t* __restrict__ key,
                                                      const uint8_t* __restrict__ value,
                                                      uint8_t* __restrict__ k_cache,
                                                      uint8_t* __restrict__ v_cache,
                                                      const int64_t* __restrict__ slots, int T,
                                                      int Hkv, int D, int bs, int64_t num_blocks,
                                                      float k_scale, float v_scale) {
  const int per_row = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / per_row;  // token * Hkv + head
  const int chunk = (int)(gid - row * per_row);
  if (row >= (int64_t)T * Hkv) return;
  const int64_t n = row / Hkv;
  const int h = (int)(row - n * Hkv);
  // the rows do not depend on the slot: request all three at once (the empty
  // asm keeps the compiler from sinking the row loads below the slot test)
  const int64_t src = (row * D + chunk * 8) * 2;
  const int64_t slot = slots[n];
  const i32x4 kx = ld16(key + src);
  const i32x4 vx = ld16(value + src);
  asm volatile("" : : "v"(kx), "v"(vx));
  if (slot < 0 || slot >= num_blocks * bs) return;
  const int64_t b = slot / bs;
  const int o = (int)(slot - b * bs);
  const int64_t dst_elem = ((b * Hkv + h) * bs + o) * D + chunk * 8;
  store_row8<ST, kFp8>(kx, vx, k_cache, v_cache, dst_elem, k_scale, v_scale);
}

// Scale of one row for a cache with a scale per (slot, kv head) row: the
// row's largest magnitude maps to qmax, the largest finite code (448 for
// E4M3FN, 6 for E2M1); a row of zeros, or one holding an infinity, keeps
// scale 1.
__device__ __forceinline__ float row_scale(float amax, float qmax) {
  return amax > 0.f && amax <= 3.402823466e38f ? amax / qmax : 1.0f;
}

// E2M1 code of fp32(x) / scale (IEEE division): the nearest of 0, 0.5, 1,
// 1.5, 2, 3, 4, 6 with ties to the code whose mantissa bit is 0 (the
// thresholds below are the midpoints; a tie takes the side of the even
// code), magnitudes beyond 6 saturating, the sign kept (-0 too).  E2M1 has
// no NaN: a NaN element is stored as +0.
__device__ __forceinline__ uint32_t e2m1_code(float x, float scale) {
  const float y = x / scale;
  if (y != y) return 0u;
  const float a = fabsf(y);
  const uint32_t m = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return m | ((__float_as_uint(y) >> 28) & 0x8u);
}

// eight elements -> eight E2M1 codes in one dword, element 2i in the low
// nibble of byte i
__device__ __forceinline__ uint32_t encode8_fp4(const float* x, float scale) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) w |= e2m1_code(x[i], scale) << (4 * i);
  return w;
}

// One thread per 8 elements of one (token, kv head) row, the D / 8 threads
// of a row being adjacent lanes: they share the row's largest magnitude
// (NaN elements do not count), then write their codes (8 bytes of E4M3FN,
// or 4 bytes of E2M1 with kFp4); the first writes the row's K and V scales.
template <class ST, bool kFp4>
__global__ __launch_bounds__(256) void scatter_rows_kernel(const uint8_t* __restrict__ key,
                                                           const uint8_t* __restrict__ value,
                                                           uint8_t* __restrict__ k_cache,
                                                           uint8_t* __restrict__ v_cache,
                                                           float* __restrict__ k_scales,
                                                           float* __restrict__ v_scales,
                                                           const int64_t* __restrict__ slots, int T, int Hkv,
                                                           int D, int bs, int64_t num_blocks) {
  const int per_row = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / per_row;  // token * Hkv + head
  const int chunk = (int)(gid - row * per_row);
  if (row >= (int64_t)T * Hkv) return;  // whole rows leave together
  const int64_t n = row / Hkv;
  const int h = (int)(row - n * Hkv);
  const int64_t src = (row * D + chunk * 8) * 2;
  const int64_t slot = slots[n];
  const i32x4 kx = ld16(key + src);
  const i32x4 vx = ld16(value + src);
  float kf[8], vf[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    unpack2<ST>((uint32_t)kx[w], kf[2 * w], kf[2 * w + 1]);
    unpack2<ST>((uint32_t)vx[w], vf[2 * w], vf[2 * w + 1]);
  }
  float ka = 0.f, va = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ka = fmaxf(ka, fabsf(kf[i]));
    va = fmaxf(va, fabsf(vf[i]));
  }
  for (int m = 1; m < per_row; m <<= 1) {  // stays inside the row's lanes
    ka = fmaxf(ka, shfl_xor(ka, m));
    va = fmaxf(va, shfl_xor(va, m));
  }
  if (slot < 0 || slot >= num_blocks * bs) return;
  constexpr float qmax = kFp4 ? 6.0f : 448.0f;
  const float ks = row_scale(ka, qmax), vs = row_scale(va, qmax);
  const int64_t b = slot / bs;
  const int o = (int)(slot - b * bs);
  const int64_t srow = (b * Hkv + h) * bs + o;
  const int64_t dst_elem = srow * D + chunk * 8;
  if constexpr (kFp4) {
    *reinterpret_cast<uint32_t*>(k_cache + dst_elem / 2) = encode8_fp4(kf, ks);
    *reinterpret_cast<uint32_t*>(v_cache + dst_elem / 2) = encode8_fp4(vf, vs);
  } else {
    *reinterpret_cast<i32x2*>(k_cache + dst_elem) = encode8_fp8(kf, ks);
    *reinterpret_cast<i32x2*>(v_cache + dst_elem) = encode8_fp8(vf, vs);
  }
  if (chunk == 0) {
    k_scales[srow] = ks;
    v_scales[srow] = vs;
  }
}

pa_status scatter_rows_launch(const void* key, const void* value, void* k_cache, void* v_cache, float* k_scales,
                              float* v_scales, const int64_t* slots, int T, int Hkv, int D, int bs,
                              int64_t num_blocks, int src_dtype, int cache_dtype, hipStream_t stream) {
  if (T == 0) return PA_OK;
  const int64_t threads = (int64_t)T * Hkv * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  auto K = reinterpret_cast<const uint8_t*>(key);
  auto V = reinterpret_cast<const uint8_t*>(value);
  auto KC = reinterpret_cast<uint8_t*>(k_cache);
  auto VC = reinterpret_cast<uint8_t*>(v_cache);
  const bool fp4 = cache_dtype == PA_FP4_E2M1;
  if (src_dtype == PA_F16 && fp4)
    hipLaunchKernelGGL((scatter_rows_kernel<F16, true>), grid, block, 0, stream, K, V, KC, VC, k_scales, v_scales,
                       slots, T, Hkv, D, bs, num_blocks);
  else if (src_dtype == PA_F16)
    hipLaunchKernelGGL((scatter_rows_kernel<F16, false>), grid, block, 0, stream, K, V, KC, VC, k_scales, v_scales,
                       slots, T, Hkv, D, bs, num_blocks);
  else if (fp4)
    hipLaunchKernelGGL((scatter_rows_kernel<BF16, true>), grid, block, 0, stream, K, V, KC, VC, k_scales, v_scales,
                       slots, T, Hkv, D, bs, num_blocks);
  else
    hipLaunchKernelGGL((scatter_rows_kernel<BF16, false>), grid, block, 0, stream, K, V, KC, VC, k_scales, v_scales,
                       slots, T, Hkv, D, bs, num_blocks);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error("pa_reshape_and_cache_scaled: launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}

// The row of position L - 1 of every sequence ([B, Hkv, D]) into the slot
// the sequence's block table gives that position (L = context_lens[s]
// clamped to [0, max_ctx]); nothing for L = 0 or a block id outside the
// pool.  One thread per 8 elements of one (sequence, kv head) row.
template <class ST, bool kFp8>
__global__ __launch_bounds__(256) void append_last_kernel(const uint8_t* __restrict__ key,
                                                          const uint8_t* __restrict__ value,
                                                          uint8_t* __restrict__ k_cache,
                                                          uint8_t* __restrict__ v_cache,
                                                          const int32_t* __restrict__ block_tables,
                                                          const int32_t* __restrict__ context_lens, int B,
                                                          int M, int max_ctx, int Hkv, int D, int bs,
                                                          int64_t num_blocks, float k_scale, float v_scale) {
  const int per_row = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / per_row;  // sequence * Hkv + head
  const int chunk = (int)(gid - row * per_row);
  if (row >= (int64_t)B * Hkv) return;
  const int64_t n = row / Hkv;
  const int h = (int)(row - n * Hkv);
  const int64_t src = (row * D + chunk * 8) * 2;
  const i32x4 kx = ld16(key + src);
  const i32x4 vx = ld16(value + src);
  int L = context_lens[n];
  L = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
  if (L == 0) return;
  const int64_t b = block_tables[n * M + (L - 1) / bs];
  if (b < 0 || b >= num_blocks) return;
  const int64_t dst_elem = ((b * Hkv + h) * bs + (L - 1) % bs) * D + chunk * 8;
  store_row8<ST, kFp8>(kx, vx, k_cache, v_cache, dst_elem, k_scale, v_scale);
}

pa_status append_last_launch(const void* key, const void* value, void* k_cache, void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens, int B, int M,
                             int max_ctx, int Hkv, int D, int bs, int64_t num_blocks, int src_dtype,
                             int cache_dtype, float k_scale, float v_scale, hipStream_t stream) {
  if (B == 0) return PA_OK;
  const int64_t threads = (int64_t)B * Hkv * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  auto K = reinterpret_cast<const uint8_t*>(key);
  auto V = reinterpret_cast<const uint8_t*>(value);
  auto KC = reinterpret_cast<uint8_t*>(k_cache);
  auto VC = reinterpret_cast<uint8_t*>(v_cache);
  if (cache_dtype != PA_FP8_E4M3)
    hipLaunchKernelGGL((append_last_kernel<F16, false>), grid, block, 0, stream, K, V, KC, VC, block_tables,
                       context_lens, B, M, max_ctx, Hkv, D, bs, num_blocks, k_scale, v_scale);
  else if (src_dtype == PA_F16)
    hipLaunchKernelGGL((append_last_kernel<F16, true>), grid, block, 0, stream, K, V, KC, VC, block_tables,
                       context_lens, B, M, max_ctx, Hkv, D, bs, num_blocks, k_scale, v_scale);
  else
    hipLaunchKernelGGL((append_last_kernel<BF16, true>), grid, block, 0, stream, K, V, KC, VC, block_tables,
                       context_lens, B, M, max_ctx, Hkv, D, bs, num_blocks, k_scale, v_scale);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error("pa_decode_append: launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}

pa_status scatter_launch(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slots, int T, int Hkv, int D, int bs, int64_t num_blocks,
                         int src_dtype, int cache_dtype, float k_scale, float v_scale,
                         hipStream_t stream) {
  if (T == 0) return PA_OK;
  const int64_t threads = (int64_t)T * Hkv * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  auto K = reinterpret_cast<const uint8_t*>(key);
  auto V = reinterpret_cast<const uint8_t*>(value);
  auto KC = reinterpret_cast<uint8_t*>(k_cache);
  auto VC = reinterpret_cast<uint8_t*>(v_cache);
  if (cache_dtype != PA_FP8_E4M3) {
    hipLaunchKernelGGL((scatter_kernel<F16, false>), grid, block, 0, stream, K, V, KC, VC, slots, T,
                       Hkv, D, bs, num_blocks, k_scale, v_scale);
  } else if (src_dtype == PA_F16) {
    hipLaunchKernelGGL((scatter_kernel<F16, true>), grid, block, 0, stream, K, V, KC, VC, slots, T,
                       Hkv, D, bs, num_blocks, k_scale, v_scale);
  } else {
    hipLaunchKernelGGL((scatter_kernel<BF16, true>), grid, block, 0, stream, K, V, KC, VC, slots, T,
                       Hkv, D, bs, num_blocks, k_scale, v_scale);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error("pa_reshape_and_cache: launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}

// Copy whole blocks, 16 bytes per thread; grid.y = pair.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ k_cache,
                                                          uint8_t* __restrict__ v_cache,
                                                          const int64_t* __restrict__ pairs,
                                                          int64_t units, int64_t num_blocks) {
  const int64_t src = pairs[2 * (int64_t)blockIdx.y];
  const int64_t dst = pairs[2 * (int64_t)blockIdx.y + 1];
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks || src == dst) return;
  const int64_t so = src * units, d0 = dst * units;
  i32x4* kc = reinterpret_cast<i32x4*>(k_cache);
  i32x4* vc = reinterpret_cast<i32x4*>(v_cache);
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units; u += (int64_t)gridDim.x * blockDim.x) {
    kc[d0 + u] = kc[so + u];
    vc[d0 + u] = vc[so + u];
  }
}

pa_status copy_blocks_launch(void* k_cache, void* v_cache, const int64_t* pairs, int N,
                             int64_t block_bytes, int64_t num_blocks, hipStream_t stream) {
  if (N == 0) return PA_OK;
  const int64_t units = block_bytes / 16;
  int64_t gx = (units + 255) / 256;
  if (gx > 16) gx = 16;
  for (int first = 0; first < N; first += 65535) {  // grid.y limit
    const int n = N - first < 65535 ? N - first : 65535;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)gx, (unsigned)n), dim3(256), 0, stream,
                       reinterpret_cast<uint8_t*>(k_cache), reinterpret_cast<uint8_t*>(v_cache),
                       pairs + 2 * (int64_t)first, units, num_blocks);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error("pa_copy_blocks: launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}

}  // namespace pa
