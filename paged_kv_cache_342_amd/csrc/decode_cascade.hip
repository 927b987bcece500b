// Launchers of the two passes of a decode over shared prefixes
// (pa_decode_shared_prefix): the prefix pass, a several-queries launch whose
// columns are the members of a group (two 16-column tiles per wave), and
// the suffix pass, a decode launch that walks each sequence from its first
// private position and starts from the state the prefix pass left (the
// kernel and both passes: decode_mfma_kernel.h).
#include "decode_mfma_kernel.h"

namespace pa {

#define PA_CASCADE_CASE(CT, QT, D, BS)                                                                          \
  if (ct == CT::code && qt == QT::code && head_dim == D && bs == BS) {                                          \
    if (prefix)                                                                                                 \
      launch_with_events(decode_mfma_kernel<CT, QT, D, BS, true, false, 2, 1, false, kPrefixPass>, grid,        \
                         dim3(64), stream, ev, a);                                                              \
    else                                                                                                        \
      launch_with_events(decode_mfma_kernel<CT, QT, D, BS, false, false, 1, 1, true, kSuffixPass>, grid,        \
                         dim3(64), stream, ev, a);                                                              \
    return true;                                                                                                \
  }

#define PA_CASCADE_BS(CT, QT, D) \
  PA_CASCADE_CASE(CT, QT, D, 8)  \
  PA_CASCADE_CASE(CT, QT, D, 16) \
  PA_CASCADE_CASE(CT, QT, D, 32)

// prefix: the prefix pass (else the suffix pass).  Built for 16-bit caches
// read with a query of their dtype and FP8 caches with either query dtype,
// head_dim 64 or 128, block size 8, 16 or 32.
bool launch_cascade_pass(bool prefix, const DecodeArgs& a, int ct, int qt, int head_dim, int bs, dim3 grid,
                         hipStream_t stream, const LaunchEvents& ev) {
  PA_CASCADE_BS(F16, F16, 64)
  PA_CASCADE_BS(F16, F16, 128)
  PA_CASCADE_BS(BF16, BF16, 64)
  PA_CASCADE_BS(BF16, BF16, 128)
  PA_CASCADE_BS(FP8, F16, 64)
  PA_CASCADE_BS(FP8, F16, 128)
  PA_CASCADE_BS(FP8, BF16, 64)
  PA_CASCADE_BS(FP8, BF16, 128)
  return false;
}

}  // namespace pa
