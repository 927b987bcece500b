// Paged decode attention on the vector ALUs, for small query groups.
//
// One wavefront walks one slice of the batch (decode_common.h) for one KV
// head and all query heads of its group.  A tile is 64 / R positions with
// R = head_dim / 32 lanes per position: each lane holds 32 elements of one
// key row and of one value row.  The element set of a lane is chosen so that
// the R lanes of a row read R adjacent 16-byte pieces per load instruction
// (each K and V row is read in full, once, by one wave).  A step covers one
// 32-position chunk (two tiles at head_dim 128, one at head_dim 64); the
// next chunk's rows are in flight while the current one is computed.
//
//   QK:  each lane forms the partial dot product of its 32 elements for each
//        query head of the group (fp32 FMAs against the pre-scaled query),
//        then the R lanes of a row add their partials with DPP quad
//        permutes, so every lane of the row holds the full score.
//   softmax: online in fp32, log2 domain; the wave-uniform running maximum of
//        a head moves only when a score exceeds it by more than
//        kRescaleThreshold.
//   PV:  each lane accumulates p * v for its own position and elements; at
//        the end of the segment the 64 / R lanes that hold the same
//        elements are summed (DPP row rotations, then two cross-row
//        exchanges).
// When the launch also appends each sequence's new row (16-bit caches), the
// loads of position L - 1 read the caller's row instead of the cache, and
// the wave that owns the sequence's last chunk stores that row into its slot
// at the end of the segment.
#include "decode_common.h"

namespace pa {

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

// id[i] for a lane-dependent i < N (a select chain, no memory)
template <int N>
__device__ __forceinline__ int pick(const int* id, int i) {
  int x = id[0];
#pragma unroll
  for (int j = 1; j < N; ++j) x = i == j ? id[j] : x;
  return x;
}

template <class CT, class QT, int D, int BS, int G>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeArgs a) {
  constexpr int e = CT::bytes;
  constexpr int R = D / 32;         // lanes per position
  constexpr int TT = 64 / R;        // positions per tile
  constexpr int NT = kChunk / TT;   // tiles per chunk
  constexpr int EPU = 16 / e;       // elements per 16-byte unit
  constexpr int U = 32 * e / 16;    // 16-byte loads per lane per row
  constexpr int64_t kChunkBytes = (int64_t)BS * D * e;
  constexpr int NB = kChunk / BS;
  constexpr bool kCanAppend = e == 2;    // new rows are stored as given
  constexpr int kRowLanes = D * e / 16;  // lanes that hold one row, 16 bytes each
  struct Raw {
    i32x4 k[NT][U];
    i32x4 v[NT][U];
  };

  __shared__ int cum[kScanMax + 1];
  __shared__ int lens[kScanMax];

  const int lane = threadIdx.x;
  const int row = lane / R;  // position within the tile
  const int c = lane % R;    // element set
  const int Hq = a.Hkv * a.G;
  const int64_t blk_stride = (int64_t)a.Hkv * kChunkBytes;

  const int h = blockIdx.x % a.Hkv;
  const int k = blockIdx.x / a.Hkv;
  const int head0 = h * G;

  Slice sl;
  if (!slice_setup(a, cum, lens, nullptr, k, sl)) return;

  const uint8_t* kbase = a.k_cache + (int64_t)h * kChunkBytes;
  const uint8_t* vbase = a.v_cache + (int64_t)h * kChunkBytes;

  // empty contexts in this slice: zero rows, written by the slice that owns them
  for (int s = sl.s_first; s < a.B; ++s) {
    const int cs = cum[s], ce = cum[s + 1];
    if (past_slice(sl, cs, ce)) break;
    if (lens[s] == 0 && row == 0) {
      float z[EPU];
#pragma unroll
      for (int i = 0; i < EPU; ++i) z[i] = 0.f;
#pragma unroll
      for (int i = 0; i < G; ++i)
#pragma unroll
        for (int u = 0; u < U; ++u) store_out(a, s, head0 + i, D, EPU * (c + R * u), z, EPU);
    }
  }

  // What a segment needs before its first chunk: the group's query rows (as
  // loaded), its block-id ring and where its last row is read from (by lanes
  // whose position lies past the end, and, when appending, by the last
  // position itself).  Each header is requested one segment ahead with loads
  // that do not depend on whether there is a next segment (past the last one
  // the current header is read again), so segment changes cost no table or
  // query round trips.
  struct Header {
    i32x4 q[G][U][EPU / 8];
    IdRing<BS> ring;
    const uint8_t* last_k;  // row of the last position
    const uint8_t* last_v;
    int lim;                // positions from lim on read last_k / last_v
    int64_t tail_off;       // cache offset the appended row goes to; -1 = none
  };
  auto load_header = [&](const Segment& g, Header& hd) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) + ((int64_t)g.s * Hq + head0 + i) * D * 2;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int half = 0; half < EPU / 8; ++half) hd.q[i][u][half] = ld16(qrow + (EPU * (c + R * u) + 8 * half) * 2);
    }
    const int32_t* trow = a.block_tables + (int64_t)g.s * a.M;
    const int blk0 = g.tok0 / BS;
    hd.ring.start(trow + blk0, (g.tok_end + BS - 1) / BS - blk0);
    int id = uniform(trow[(g.tok_end - 1) / BS]);
    const bool id_ok = id >= 0 && (int64_t)id < a.num_blocks;
    if (!id_ok) id = 0;
    const int64_t off = (int64_t)id * blk_stride + (int64_t)((g.tok_end - 1) % BS) * D * e;
    const bool app = kCanAppend && a.new_k != nullptr && g.tok_end == lens[g.s];
    const int64_t nrow = ((int64_t)g.s * a.Hkv + h) * D * e;
    hd.last_k = app ? a.new_k + nrow : kbase + off;
    hd.last_v = app ? a.new_v + nrow : vbase + off;
    hd.lim = g.tok_end - (app ? 1 : 0);
    hd.tail_off = app && id_ok ? off : -1;
  };

  Segment cur = next_segment(a, sl, cum, lens,sl.s_first);
  if (cur.s < 0) return;
  Header hc, hn;
  load_header(cur, hc);
  Segment nxt = next_segment(a, sl, cum, lens,cur.s + 1);
  load_header(nxt.s >= 0 ? nxt : cur, hn);

  while (true) {
    const int s = cur.s;
    const int cs = cur.cs, ce = cur.ce;
    const int tok0 = cur.tok0, tok_end = cur.tok_end, nchunks = cur.nchunks;
    IdRing<BS>& ring = hc.ring;
    const int lim = hc.lim;
    // the appended row, stored at the end of the segment: lane i < kRowLanes
    // holds 16 bytes of K, the next kRowLanes lanes 16 bytes of V
    i32x4 app_row = {0, 0, 0, 0};
    if (kCanAppend && a.new_k != nullptr)
      app_row = ld16((lane < kRowLanes ? hc.last_k : hc.last_v) + 16 * (lane % kRowLanes));

    // query, widened and pre-scaled into the log2 domain
    float qf[G][32];
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int half = 0; half < EPU / 8; ++half)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            float lo, hi;
            unpack2<QT>((uint32_t)hc.q[i][u][half][w], lo, hi);
            qf[i][EPU * u + 8 * half + 2 * w] = lo * a.qk_scale_log2;
            qf[i][EPU * u + 8 * half + 2 * w + 1] = hi * a.qk_scale_log2;
          }

    auto load_chunk = [&](int ch, Raw& raw) {
      int id[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int x = ring.id(ch, i);
        id[i] = (x < 0 || (int64_t)x >= a.num_blocks) ? 0 : x;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int tc = TT * t + row;  // position within the chunk
        const bool ok = tok0 + kChunk * ch + tc < lim;
        const int64_t off = (int64_t)pick<NB>(id, tc / BS) * blk_stride + (tc % BS) * D * e;
        const uint8_t* krow = ok ? kbase + off : hc.last_k;
        const uint8_t* vrow = ok ? vbase + off : hc.last_v;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int col = 16 * (c + R * u);
          raw.k[t][u] = ld16_stream(krow + col);
          raw.v[t][u] = ld16_stream(vrow + col);
        }
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

    auto compute_chunk = [&](int ch, const Raw& raw) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bool ok = tok0 + kChunk * ch + TT * t + row < tok_end;
        float kf[32];
        widen32<CT>(raw.k[t], kf);
        float sv[G];
#pragma unroll
        for (int i = 0; i < G; ++i) {
          float x = 0.f;
#pragma unroll
          for (int j = 0; j < 32; ++j) x = fmaf(qf[i][j], kf[j], x);
          x += dpp<kQuadXor1>(x);
          if constexpr (R == 4) x += dpp<kQuadXor2>(x);
          sv[i] = ok ? x : -INFINITY;
        }
        float vf[32];
        widen32<CT>(raw.v[t], vf);
#pragma unroll
        for (int i = 0; i < G; ++i) {
          if (wave_any(sv[i] > m[i] + kRescaleThreshold)) {
            const float mn = fmaxf(m[i], wave_max(sv[i]));
            const float alpha = fast_exp2(m[i] - mn);
#pragma unroll
            for (int j = 0; j < 32; ++j) acc[i][j] *= alpha;
            l[i] *= alpha;
            m[i] = mn;
          }
          const float p = fast_exp2(sv[i] - m[i]);
          l[i] += p;
#pragma unroll
          for (int j = 0; j < 32; ++j) acc[i][j] = fmaf(p, vf[j], acc[i][j]);
        }
      }
    };

    // The next chunk is in flight while one is computed; later chunks are
    // always requested (past the end every lane reads the last row), so no
    // load sits under a branch.
    {
      Raw buf0, buf1;
      load_chunk(0, buf0);
      for (int ch = 0; ch < nchunks; ch += 2) {
        ring.advance();
        load_chunk(ch + 1, buf1);
        compute_chunk(ch, buf0);
        if (ch + 1 >= nchunks) break;
        ring.advance();
        load_chunk(ch + 2, buf0);
        compute_chunk(ch + 1, buf1);
      }
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
    const bool whole = whole_sequence(sl, cs, ce);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float lt = row_sum(l[i]);
#pragma unroll
      for (int j = 0; j < 32; ++j) acc[i][j] = row_sum(acc[i][j]);
      if (row == 0) {
        const float f = whole ? a.v_scale / lt : 1.f;
        const int64_t prow = part_row(a, sl.k, s, 0, head0 + i);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float v[EPU];
#pragma unroll
          for (int j = 0; j < EPU; ++j) v[j] = acc[i][EPU * u + j] * f;
          if (whole)
            store_out(a, s, head0 + i, D, EPU * (c + R * u), v, EPU);
          else
            store_partial(a, prow, D, EPU * (c + R * u), v, EPU);
        }
        if (!whole && c == 0) store_ml(a, prow, m[i], lt);
      }
    }
    if (hc.tail_off >= 0 && lane < 2 * kRowLanes) {
      uint8_t* dst = const_cast<uint8_t*>(lane < kRowLanes ? kbase : vbase) + hc.tail_off;
      *reinterpret_cast<i32x4*>(dst + 16 * (lane % kRowLanes)) = app_row;
    }

    if (nxt.s < 0) break;
    cur = nxt;
    hc = hn;
    nxt = next_segment(a, sl, cum, lens,cur.s + 1);
    load_header(nxt.s >= 0 ? nxt : cur, hn);
  }
}

#define PA_VALU_CASE(CT, QT, D, BS, G)                                                            \
  if (ct == CT::code && qt == QT::code && head_dim == D && bs == BS && group == G) {              \
    launch_with_events(decode_valu_kernel<CT, QT, D, BS, G>, grid, dim3(64), stream, ev, a);      \
    return true;                                                                                  \
  }

#define PA_VALU_G(CT, QT, D, BS) \
  PA_VALU_CASE(CT, QT, D, BS, 1) \
  PA_VALU_CASE(CT, QT, D, BS, 2)

#define PA_VALU_BS(CT, QT, D) \
  PA_VALU_G(CT, QT, D, 8)     \
  PA_VALU_G(CT, QT, D, 16)    \
  PA_VALU_G(CT, QT, D, 32)

bool launch_decode_valu(const DecodeArgs& a, int ct, int qt, int head_dim, int bs, int group,
                        dim3 grid, hipStream_t stream, const LaunchEvents& ev) {
  PA_VALU_BS(F16, F16, 64)
  PA_VALU_BS(F16, F16, 128)
  PA_VALU_BS(BF16, BF16, 64)
  PA_VALU_BS(BF16, BF16, 128)
  PA_VALU_BS(FP8, F16, 64)
  PA_VALU_BS(FP8, F16, 128)
  PA_VALU_BS(FP8, BF16, 64)
  PA_VALU_BS(FP8, BF16, 128)
  return false;
}

bool valu_supports(int ct, int qt, int head_dim, int bs, int group) {
  (void)ct, (void)qt, (void)head_dim, (void)bs;
  return group == 1 || group == 2;
}

}  // namespace pa
