// Paged decode attention on the vector ALUs, for small query groups.
//
// One wavefront handles one (sequence, partition, KV head) item.  A tile is
// 64 / R positions with R = head_dim / 32 lanes per position: each lane holds
// 32 elements of one key row and of one value row.  The element set of a lane
// is chosen so that the R lanes of a row read R adjacent 16-byte pieces per
// load instruction (each K and V row is read in full, once, by one wave).
//
//   QK:  each lane forms the partial dot product of its 32 elements for each
//        query head of the group (fp32 FMAs against the pre-scaled query),
//        then the R lanes of a row add their partials with DPP quad
//        permutes, so every lane of the row holds the full score.
//   softmax: online in fp32, log2 domain; the wave-uniform running maximum of
//        a head moves only when a score exceeds it by more than
//        kRescaleThreshold.
//   PV:  each lane accumulates p * v for its own position and elements; at
//        the end of the partition the 64 / R lanes that hold the same
//        elements are summed (DPP row rotations, then two cross-row
//        exchanges).
#include "decode_common.h"

namespace pa {

template <class CT, int D>
struct TileRaw {
  static constexpr int U = 32 * CT::bytes / 16;  // 16-byte loads per lane per row
  i32x4 k[U];
  i32x4 v[U];
};

// the 32 elements a lane holds, converted to fp32; element order: unit u,
// then position within the 16-byte unit
template <class CT>
__device__ __forceinline__ void widen32(const i32x4* raw, float* o);
template <>
__device__ __forceinline__ void widen32<BF16>(const i32x4* raw, float* o) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) unpack2<BF16>((uint32_t)raw[u][w], o[8 * u + 2 * w], o[8 * u + 2 * w + 1]);
}
template <>
__device__ __forceinline__ void widen32<F16>(const i32x4* raw, float* o) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) unpack2<F16>((uint32_t)raw[u][w], o[8 * u + 2 * w], o[8 * u + 2 * w + 1]);
}
template <>
__device__ __forceinline__ void widen32<FP8>(const i32x4* raw, float* o) {
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) fp8x4_to_f32((uint32_t)raw[u][w], o + 16 * u + 4 * w);
}

template <class CT, class QT, int D, int BS, int G>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeArgs a) {
  constexpr int e = CT::bytes;
  constexpr int R = D / 32;         // lanes per position
  constexpr int TT = 64 / R;        // positions per tile
  constexpr int EPU = 16 / e;       // elements per 16-byte unit
  using Raw = TileRaw<CT, D>;
  constexpr int U = Raw::U;
  constexpr int64_t kChunkBytes = (int64_t)BS * D * e;

  const int lane = threadIdx.x;
  const int row = lane / R;  // position within the tile
  const int c = lane % R;    // element set
  const int Hq = a.Hkv * a.G;
  const int64_t blk_stride = (int64_t)a.Hkv * kChunkBytes;
  const int total = item_count(a) * a.Hkv;

  for (int flat = blockIdx.x; flat < total; flat += gridDim.x) {
    const Item t = item_at(a, flat);
    const int head0 = t.h * G;

    if (t.L == 0) {
      if (row == 0) {
        float z[EPU];
#pragma unroll
        for (int i = 0; i < EPU; ++i) z[i] = 0.f;
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
          for (int u = 0; u < U; ++u) store_out(a, t.s, head0 + i, D, EPU * (c + R * u), z, EPU);
      }
      continue;
    }

    // query, pre-scaled into the log2 domain
    float qf[G][32];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) + ((int64_t)t.s * Hq + head0 + i) * D * 2;
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int half = 0; half < EPU / 8; ++half) {
          const i32x4 x = ld16(qrow + (EPU * (c + R * u) + 8 * half) * 2);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            float lo, hi;
            unpack2<QT>((uint32_t)x[w], lo, hi);
            qf[i][EPU * u + 8 * half + 2 * w] = lo * a.qk_scale_log2;
            qf[i][EPU * u + 8 * half + 2 * w + 1] = hi * a.qk_scale_log2;
          }
        }
      }
    }

    const int ids = load_block_ids(a, t, BS);
    const uint8_t* kbase = a.k_cache + (int64_t)t.h * kChunkBytes;
    const uint8_t* vbase = a.v_cache + (int64_t)t.h * kChunkBytes;
    const int ntiles = (t.tok_end - t.tok0 + TT - 1) / TT;
    const int64_t last_off = last_row_offset(t, ids, BS, blk_stride, D * e);

    auto load_tile = [&](int tile, Raw& raw) {
      const int tc = TT * tile + row;  // position relative to the partition
      const int id = __shfl(ids, tc / BS);
      const bool ok = t.tok0 + tc < t.tok_end;
      const int64_t off = ok ? (int64_t)id * blk_stride + (tc % BS) * D * e : last_off;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int col = 16 * (c + R * u);
        raw.k[u] = ld16_stream(kbase + off + col);
        raw.v[u] = ld16_stream(vbase + off + col);
      }
    };

    float m[G], l[G], acc[G][32];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      m[i] = -INFINITY;
      l[i] = 0.f;
#pragma unroll
      for (int j = 0; j < 32; ++j) acc[i][j] = 0.f;
    }

    auto compute_tile = [&](int tile, const Raw& raw) {
      const bool ok = t.tok0 + TT * tile + row < t.tok_end;
      float kf[32];
      widen32<CT>(raw.k, kf);
      float s[G];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float x = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) x = fmaf(qf[i][j], kf[j], x);
        x += dpp<kQuadXor1>(x);
        if constexpr (R == 4) x += dpp<kQuadXor2>(x);
        s[i] = ok ? x : -INFINITY;
      }
      float vf[32];
      widen32<CT>(raw.v, vf);
#pragma unroll
      for (int i = 0; i < G; ++i) {
        if (wave_any(s[i] > m[i] + kRescaleThreshold)) {
          const float mn = fmaxf(m[i], wave_max(s[i]));
          const float alpha = fast_exp2(m[i] - mn);
#pragma unroll
          for (int j = 0; j < 32; ++j) acc[i][j] *= alpha;
          l[i] *= alpha;
          m[i] = mn;
        }
        const float p = fast_exp2(s[i] - m[i]);
        l[i] += p;
#pragma unroll
        for (int j = 0; j < 32; ++j) acc[i][j] = fmaf(p, vf[j], acc[i][j]);
      }
    };

    // Double-buffered; the next tile is always requested (past the end every
    // lane reads the last row), so no load sits under a branch.
    Raw buf0, buf1;
    load_tile(0, buf0);
    for (int tile = 0; tile < ntiles; tile += 2) {
      load_tile(tile + 1, buf1);
      compute_tile(tile, buf0);
      if (tile + 1 >= ntiles) break;
      load_tile(tile + 2, buf0);
      compute_tile(tile + 1, buf1);
    }

    // sum over the positions (lanes with the same element set)
    auto row_sum = [&](float x) {
      if constexpr (R == 2) x += dpp<kRowRor2>(x);
      x += dpp<kRowRor4>(x);
      x += dpp<kRowRor8>(x);
      x += shfl_xor(x, 16);
      x += shfl_xor(x, 32);
      return x;
    };
    const bool final = t.nparts == 1;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float lt = row_sum(l[i]);
#pragma unroll
      for (int j = 0; j < 32; ++j) acc[i][j] = row_sum(acc[i][j]);
      if (row == 0) {
        const float f = final ? a.v_scale / lt : 1.f;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float v[EPU];
#pragma unroll
          for (int j = 0; j < EPU; ++j) v[j] = acc[i][EPU * u + j] * f;
          if (final)
            store_out(a, t.s, head0 + i, D, EPU * (c + R * u), v, EPU);
          else
            store_partial(a, t.s, head0 + i, t.p, D, EPU * (c + R * u), v, EPU);
        }
        if (!final && c == 0) store_ml(a, t.s, head0 + i, t.p, m[i], lt);
      }
    }
  }
}

#define PA_VALU_CASE(CT, QT, D, BS, G)                                                            \
  if (ct == CT::code && qt == QT::code && head_dim == D && bs == BS && group == G) {              \
    hipLaunchKernelGGL((decode_valu_kernel<CT, QT, D, BS, G>), grid, dim3(64), 0, stream, a);    \
    return true;                                                                                  \
  }

#define PA_VALU_G(CT, QT, D, BS) \
  PA_VALU_CASE(CT, QT, D, BS, 1) \
  PA_VALU_CASE(CT, QT, D, BS, 2)

#define PA_VALU_BS(CT, QT, D) \
  PA_VALU_G(CT, QT, D, 8)     \
  PA_VALU_G(CT, QT, D, 16)    \
  PA_VALU_G(CT, QT, D, 32)

// group 4 is built only for the block size and head_dim of the measured
// grouped-query workloads, to compare against the MFMA kernel
#define PA_VALU_G4(CT, QT) PA_VALU_CASE(CT, QT, 128, 16, 4)

bool launch_decode_valu(const DecodeArgs& a, int ct, int qt, int head_dim, int bs, int group,
                        dim3 grid, hipStream_t stream) {
  PA_VALU_BS(F16, F16, 64)
  PA_VALU_BS(F16, F16, 128)
  PA_VALU_BS(BF16, BF16, 64)
  PA_VALU_BS(BF16, BF16, 128)
  PA_VALU_BS(FP8, F16, 64)
  PA_VALU_BS(FP8, F16, 128)
  PA_VALU_BS(FP8, BF16, 64)
  PA_VALU_BS(FP8, BF16, 128)
  PA_VALU_G4(F16, F16)
  PA_VALU_G4(BF16, BF16)
  PA_VALU_G4(FP8, BF16)
  return false;
}

bool valu_supports(int ct, int qt, int head_dim, int bs, int group) {
  if (group == 1 || group == 2) return true;
  return group == 4 && head_dim == 128 && bs == 16 && (ct == qt || ct == FP8::code);
}

}  // namespace pa
