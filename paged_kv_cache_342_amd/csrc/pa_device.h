// Device-side helpers shared by the gfx950 kernels of the paged decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// element-type tags (bits per element; codes are pa_dtype values)
struct F16 { static constexpr int bytes = 2; static constexpr int bits = 16; static constexpr int code = 1; };
struct BF16 { static constexpr int bytes = 2; static constexpr int bits = 16; static constexpr int code = 2; };
struct FP8 { static constexpr int bytes = 1; static constexpr int bits = 8; static constexpr int code = 3; };
// OCP E2M1, two per byte, element 2i in the low nibble
struct FP4 { static constexpr int bits = 4; static constexpr int code = 4; };

constexpr int kWave = 64;
// log2 of the largest factor by which an un-rescaled probability may exceed 1
// before the running maximum is moved (the result is exact either way; this
// only bounds the size of the stored terms).
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// two 16-bit values packed in a dword -> fp32 (lo, hi)
template <class T>
__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi);
template <>
__device__ __forceinline__ void unpack2<BF16>(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void unpack2<F16>(uint32_t w, float& lo, float& hi) {
  lo = f16_bits_to_f32(w & 0xFFFFu);
  hi = f16_bits_to_f32(w >> 16);
}

// four E4M3FN codes in a dword -> four fp32 values (exact)
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = a[0];
  o[1] = a[1];
  o[2] = b[0];
  o[3] = b[1];
}

// four E4M3FN codes -> four 16-bit values (two dwords), exact: every E4M3FN
// value is representable in both fp16 and bf16.
template <class T>
__device__ __forceinline__ i32x2 fp8x4_to_16(uint32_t w);
template <>
__device__ __forceinline__ i32x2 fp8x4_to_16<F16>(uint32_t w) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true);
  i32x2 r;
  r[0] = __builtin_bit_cast(int, a);
  r[1] = __builtin_bit_cast(int, b);
  return r;
}
template <>
__device__ __forceinline__ i32x2 fp8x4_to_16<BF16>(uint32_t w) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true);
  i32x2 r;
  r[0] = __builtin_bit_cast(int, a);
  r[1] = __builtin_bit_cast(int, b);
  return r;
}

// eight E2M1 codes in a dword (element 2i in the low nibble of byte i) ->
// eight 16-bit values (four dwords), exact: every E2M1 value (0, 0.5 .. 6
// and their negatives) is representable in both fp16 and bf16.  The
// hardware converts one byte (two codes) per instruction, low nibble to
// the low half.
template <class T>
__device__ __forceinline__ i32x4 fp4x8_to_16(uint32_t w);
template <>
__device__ __forceinline__ i32x4 fp4x8_to_16<F16>(uint32_t w) {
  return i32x4{__builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)),
               __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)),
               __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)),
               __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3))};
}
template <>
__device__ __forceinline__ i32x4 fp4x8_to_16<BF16>(uint32_t w) {
  return i32x4{__builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0)),
               __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1)),
               __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2)),
               __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3))};
}
// the four codes of the low two bytes -> four 16-bit values (two dwords)
template <class T>
__device__ __forceinline__ i32x2 fp4x4_to_16(uint32_t w) {
  const i32x4 x = fp4x8_to_16<T>(w);
  return i32x2{x[0], x[1]};
}

// fp32 -> 16-bit storage, round to nearest even
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);  // NaN stays NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// ---- cross-lane ----------------------------------------------------------
// DPP controls (GFX9 encoding)
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor2 = 0x122;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- memory --------------------------------------------------------------
__device__ __forceinline__ i32x4 ld16(const void* p) { return *reinterpret_cast<const i32x4*>(p); }
// KV cache rows are read once per call: nontemporal loads keep them from
// displacing reusable lines and stream better from HBM.
__device__ __forceinline__ i32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}
__device__ __forceinline__ i32x2 ld8_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x2*>(p));
}
__device__ __forceinline__ int ld4_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const int*>(p));
}
__device__ __forceinline__ uint32_t ld2_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}
__device__ __forceinline__ i32x2 ld8(const void* p) { return *reinterpret_cast<const i32x2*>(p); }
__device__ __forceinline__ int ld4(const void* p) { return *reinterpret_cast<const int*>(p); }

}  // namespace pa
