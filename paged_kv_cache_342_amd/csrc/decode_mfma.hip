// Launchers of the MFMA decode kernel (decode_mfma_kernel.h) for decode, for
// several queries per sequence and for caches with row scales.
#include "decode_mfma_kernel.h"

namespace pa {

template <class CT, class QT, int D, int BS>
void launch_mfma(const DecodeArgs& a, bool multi_query, int tiles_per_wave, int waves_per_group, dim3 grid,
                 hipStream_t stream, const LaunchEvents& ev) {
  if (!multi_query) {
    if (a.window > 0)
      launch_with_events(decode_mfma_kernel<CT, QT, D, BS, false, false, 1, 1, true>, grid, dim3(64), stream, ev, a);
    else
      launch_with_events(decode_mfma_kernel<CT, QT, D, BS, false, false, 1>, grid, dim3(64), stream, ev, a);
    return;
  }
  if constexpr (CT::bits == 16) {
    if (waves_per_group == kSharedWaves) {
      launch_with_events(decode_mfma_kernel<CT, QT, D, BS, true, false, 2, kSharedWaves>, grid,
                         dim3(64 * kSharedWaves), stream, ev, a);
      return;
    }
    if (waves_per_group == kSharedWaves1) {
      launch_with_events(decode_mfma_kernel<CT, QT, D, BS, true, false, 1, kSharedWaves1>, grid,
                         dim3(64 * kSharedWaves1), stream, ev, a);
      return;
    }
  }
  if (tiles_per_wave == 2)
    launch_with_events(decode_mfma_kernel<CT, QT, D, BS, true, false, 2>, grid, dim3(64), stream, ev, a);
  else
    launch_with_events(decode_mfma_kernel<CT, QT, D, BS, true, false, 1>, grid, dim3(64), stream, ev, a);
}

#define PA_MFMA_CASE(CT, QT, D, BS)                                                                   \
  if (ct == CT::code && qt == QT::code && head_dim == D && bs == BS) {                                \
    launch_mfma<CT, QT, D, BS>(a, multi_query, tiles_per_wave, waves_per_group, grid, stream, ev);    \
    return true;                                                                                      \
  }

#define PA_MFMA_BS(CT, QT, D) \
  PA_MFMA_CASE(CT, QT, D, 8)  \
  PA_MFMA_CASE(CT, QT, D, 16) \
  PA_MFMA_CASE(CT, QT, D, 32)

// FP8 and FP4 caches with a scale per row
#define PA_MFMA_RS_CASE(CT, QT, D, BS)                                                                    \
  if (qt == QT::code && head_dim == D && bs == BS) {                                                      \
    launch_with_events(decode_mfma_kernel<CT, QT, D, BS, false, true, 1>, grid, dim3(64), stream, ev, a); \
    return true;                                                                                          \
  }
#define PA_MFMA_RS_BS(CT, QT, D) \
  PA_MFMA_RS_CASE(CT, QT, D, 8)  \
  PA_MFMA_RS_CASE(CT, QT, D, 16) \
  PA_MFMA_RS_CASE(CT, QT, D, 32)

// Whether launch_decode_mfma has a kernel for these types and sizes (the
// instantiations below): 16-bit caches read with a query of their own dtype,
// FP8 caches with either query dtype (one query per sequence also with sinks
// plus a window), FP8 and FP4 caches with row scales (one query per
// sequence); head_dim 64 or 128; block size 8, 16 or 32.
bool mfma_kernel_built(int ct, int qt, int head_dim, int bs, bool multi_query, bool row_scales) {
  if ((head_dim != 64 && head_dim != 128) || (bs != 8 && bs != 16 && bs != 32)) return false;
  if (qt != F16::code && qt != BF16::code) return false;
  if (row_scales) return !multi_query && (ct == FP8::code || ct == FP4::code);
  return ct == qt || ct == FP8::code;
}

// tiles_per_wave: 16-column tiles one wave computes (1, or 2 for several
// queries per sequence spanning more than one tile); waves_per_group: 1, or
// kSharedWaves / kSharedWaves1 for the kernels whose waves share K/V chunks
// through LDS
bool launch_decode_mfma(const DecodeArgs& a, int ct, int qt, int head_dim, int bs, bool multi_query,
                        int tiles_per_wave, int waves_per_group, dim3 grid, hipStream_t stream,
                        const LaunchEvents& ev) {
  if (a.k_row_scale != nullptr) {
    if (multi_query) return false;
    if (ct == FP8::code) {
      PA_MFMA_RS_BS(FP8, F16, 64)
      PA_MFMA_RS_BS(FP8, F16, 128)
      PA_MFMA_RS_BS(FP8, BF16, 64)
      PA_MFMA_RS_BS(FP8, BF16, 128)
    } else if (ct == FP4::code) {
      PA_MFMA_RS_BS(FP4, F16, 64)
      PA_MFMA_RS_BS(FP4, F16, 128)
      PA_MFMA_RS_BS(FP4, BF16, 64)
      PA_MFMA_RS_BS(FP4, BF16, 128)
    }
    return false;
  }
  PA_MFMA_BS(F16, F16, 64)
  PA_MFMA_BS(F16, F16, 128)
  PA_MFMA_BS(BF16, BF16, 64)
  PA_MFMA_BS(BF16, BF16, 128)
  PA_MFMA_BS(FP8, F16, 64)
  PA_MFMA_BS(FP8, F16, 128)
  PA_MFMA_BS(FP8, BF16, 64)
  PA_MFMA_BS(FP8, BF16, 128)
  return false;
}

}  // namespace pa
