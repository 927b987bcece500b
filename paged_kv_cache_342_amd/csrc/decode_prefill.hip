// Several queries per sequence over a 16-bit cache when a sequence's
// (query, head) columns are many (chunked prefill: 64 queries x 4 heads =
// 256 columns per KV head): 32 x 32 matrix tiles and K/V chunks shared by a
// workgroup through LDS.
//
// A workgroup of kPrefillWaves waves (two per SIMD) takes one slice of the
// chunk line (decode_common.h), one KV head and 256 columns, 32 per wave
// (column c of wave w is column 256 * group + 32 * w + c; its query is
// column / G, its head column % G).  Per 32-position chunk:
//   - the chunk's K and V rows are loaded one chunk ahead, 16 bytes at a
//     time, and after the current chunk is computed stored into the other of
//     two LDS stages: K rows as they are by half of the threads, V
//     transposed (d-major) by the other half, each of which loads the same 8
//     d of two consecutive positions and stores their 8 (position, position
//     + 1) pairs as dwords -- 64 lanes writing 64 distinct banks -- so the
//     V^T operand of every wave is read, not rebuilt;
//   - QK: S^T[32 positions x 32 columns] += K[32 x 16 d] . Q^T[16 d x 32]
//     over the D / 16 slices of d (v_mfma_f32_32x32x16), Q in registers;
//   - softmax per column in fp32, log2 domain: each lane holds 16 positions
//     of one column, the other 16 sit in lane ^ 32;
//   - PV: O^T[D x 32 columns] += V^T[32 d x 16 positions] . P^T, where the
//     16 position slots of each product are the 8 positions each lane
//     already holds per half (so P needs no lane exchange) and V^T is read
//     from LDS in the same order.  P is split into two bf16 terms for bf16
//     (about 16 bits of each weight), one fp16 term for fp16.
// The query j of n a column belongs to sees positions up to L - n + j.
// Segments, partial results and the merge are those of the other decode
// kernels (partial rows [slice + sequence, query, head]).
#include "decode_mfma_kernel.h"

namespace pa {

constexpr int kPrefillWaves = 8;    // waves per workgroup: 256 columns
constexpr int kPrefillCols = 32 * kPrefillWaves;

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <class T>
__device__ __forceinline__ f32x16 mfma32x32(i32x4 a, i32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32x32<F16>(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                0);
}
template <>
__device__ __forceinline__ f32x16 mfma32x32<BF16>(i32x4 a, i32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

template <class CT, int D, int BS>
__global__ __launch_bounds__(64 * kPrefillWaves) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_kernel(DecodeArgs a) {
  static_assert(CT::bits == 16, "16-bit caches");
  constexpr bool kBf16 = std::is_same<CT, BF16>::value;
  constexpr int RB = D * 2;                   // bytes per cache row
  constexpr int KS = D / 16;                  // QK products per chunk (16 d each)
  constexpr int DB = D / 32;                  // 32-row blocks of O^T
  constexpr int64_t kChunkBytes = (int64_t)BS * RB;
  constexpr int NB = kChunk / BS;
  constexpr int kPieceRow = RB / 16;          // 16-byte pieces per row
  // loaders: kLoaders threads take two K pieces each (rows r and r + 16),
  // as many take two V pieces each (rows 2 pp and 2 pp + 1, pp = 0..15), all
  // at the same 16-byte column
  constexpr int kLoaders = 16 * kPieceRow;
  static_assert(2 * kLoaders <= 64 * kPrefillWaves, "loaders");
  // LDS stage: K rows at a pitch of RB + 16 bytes, then V^T rows (one per d)
  // of kChunk positions at a pitch of 72 bytes (18 dwords: the 32 rows one
  // V^T read spans fall on distinct even banks)
  constexpr int KP = RB + 16;
  constexpr int VP = 2 * kChunk + 8;
  constexpr int kStage = kChunk * KP + D * VP;

  constexpr int kScan = kScanMaxMQ;
  __shared__ int cum[kScan + 1];
  __shared__ int lens[kScan];
  __shared__ int qrow[kScan + 1];
  __shared__ __attribute__((aligned(16))) uint8_t stage[2 * kStage];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 31;   // column within the wave's tile; row of A operands
  const int g2 = lane >> 5;  // which 8 of each product's 16 k slots the lane holds
  const int Hq = a.Hkv * a.G;
  const int64_t blk_stride = (int64_t)a.Hkv * kChunkBytes;

  // workgroup -> (slice, column group, KV head), the KV head fastest
  const int h = blockIdx.x % a.Hkv;
  const int rest = blockIdx.x / a.Hkv;
  const int grp = rest % a.head_tiles;
  const int k = rest / a.head_tiles;

  if (a.B > kScan) return;
  Slice sl;
  if (!slice_setup(a, cum, lens, qrow, k, sl)) return;

  const int col = kPrefillCols * grp + 32 * wv + j;
  const int cq = col / a.G;                 // query within the sequence
  const bool col_ok = cq < a.nq;
  const int head = h * a.G + (col_ok ? col - cq * a.G : 0);
  const uint8_t* kbase = a.k_cache + (int64_t)h * kChunkBytes;
  const uint8_t* vbase = a.v_cache + (int64_t)h * kChunkBytes;

  Segment cur = next_segment(a, sl, cum, lens, sl.s_first);
  while (cur.s >= 0) {
    const int s = cur.s;
    int row0, nqs;
    query_range(a, qrow, s, lens[s], row0, nqs);
    row0 = uniform(row0);
    nqs = uniform(nqs);
    const bool live = cq < nqs;
    const bool has = kPrefillCols * grp + 32 * wv < nqs * a.G;  // the wave holds a query of s
    const int qlim = lens[s] - nqs + cq;  // last position the column's query sees

    // Q^T operand slices: d = 16 ks + 8 g2 .. + 7 of the column's query row
    i32x4 qop[KS];
    {
      const int64_t qr = live ? row0 + cq : 0;
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(a.q) + (qr * Hq + (live ? head : h * a.G)) * RB;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const i32x4 x = ld16(qp + (16 * ks + 8 * g2) * 2);
        qop[ks] = live ? x : i32x4{0, 0, 0, 0};
      }
    }

    // block ids of the segment and the row read by positions past its end
    const int32_t* trow = a.block_tables + (int64_t)s * a.M;
    const int blk0 = cur.tok0 / BS;
    IdRing<BS> ring;
    ring.start(trow + blk0, (cur.tok_end + BS - 1) / BS - blk0);
    int last_id = uniform(trow[(cur.tok_end - 1) / BS]);
    if (last_id < 0 || (int64_t)last_id >= a.num_blocks) last_id = 0;
    const int64_t last_off = (int64_t)last_id * blk_stride + (int64_t)((cur.tok_end - 1) % BS) * RB;
    const int tok0 = cur.tok0, tok_end = cur.tok_end, nchunks = cur.nchunks;

    // this thread's two pieces of chunk c: V loaders (threads below
    // kLoaders) take rows 2 pp, 2 pp + 1 of V at column c16, K loaders (the
    // next kLoaders threads) rows r and r + 16 of K at column c16 (lanes run
    // over c16 for K, over pp for V)
    const int tid = (int)threadIdx.x;
    const bool vload = tid < kLoaders;
    const bool kload = !vload && tid < 2 * kLoaders;
    const int lt = vload ? tid : tid - kLoaders;
    const int c16 = vload ? lt / 16 : lt % kPieceRow;
    const int r0 = vload ? 2 * (lt % 16) : lt / kPieceRow;  // first row of the two
    const int r1 = vload ? r0 + 1 : r0 + 16;
    auto load = [&](int c, i32x4* piece) {
      const int ctok = tok0 + kChunk * c;
      int id[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int x = ring.id(c, i);
        id[i] = (x < 0 || (int64_t)x >= a.num_blocks) ? 0 : x;
      }
      const uint8_t* base = vload ? vbase : kbase;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int pos = u ? r1 : r0;
        int bid = id[0];
#pragma unroll
        for (int i = 1; i < NB; ++i)
          if (pos / BS == i) bid = id[i];
        const int64_t off = ctok + pos < tok_end ? (int64_t)bid * blk_stride + (pos % BS) * RB : last_off;
        piece[u] = (vload || kload) ? ld16_stream(base + off + 16 * c16) : i32x4{0, 0, 0, 0};
      }
    };
    auto store = [&](int c, const i32x4* piece) {
      uint8_t* sb = stage + (c & 1) * kStage;
      if (kload) {
        *reinterpret_cast<i32x4*>(sb + r0 * KP + 16 * c16) = piece[0];
        *reinterpret_cast<i32x4*>(sb + r1 * KP + 16 * c16) = piece[1];
      } else if (vload) {
        // dword e of a piece holds d = 8 c16 + 2 e (low half) and + 1 (high);
        // V^T row d gets (position r0, position r1) as one dword
        uint8_t* vt = sb + kChunk * KP + (8 * c16) * VP + 2 * r0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x0 = (uint32_t)piece[0][e], x1 = (uint32_t)piece[1][e];
          *reinterpret_cast<uint32_t*>(vt + (2 * e) * VP) = __builtin_amdgcn_perm(x1, x0, 0x05040100u);
          *reinterpret_cast<uint32_t*>(vt + (2 * e + 1) * VP) = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
        }
      }
    };

    float m = -INFINITY, l = 0.f;
    f32x16 acc[DB];
#pragma unroll
    for (int e = 0; e < DB; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[e][r] = 0.f;

    auto compute = [&](int c) {
      const uint8_t* sb = stage + (c & 1) * kStage;
      const int ctok = tok0 + kChunk * c;
      // ---- QK: S^T[pos][col]; lane (j, g2) register r holds position 8 (r / 4) + 4 g2 + r % 4
      f32x16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const i32x4 kop = *reinterpret_cast<const i32x4*>(sb + j * KP + (16 * ks + 8 * g2) * 2);
        sacc = mfma32x32<CT>(kop, qop[ks], sacc);
      }
      // ---- online softmax for the lane's column; a chunk every position of
      // which every column of the wave sees skips the masks
      float sc[16];
      float mx = -INFINITY;
      const int lim_col = min(tok_end, qlim + 1) - ctok;  // this column sees positions below lim_col
      const bool open = !wave_any(lim_col < kChunk);
      if (open) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[r] = sacc[r] * a.qk_scale_log2;
          mx = fmaxf(mx, sc[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bool seen = 8 * (r >> 2) + 4 * g2 + (r & 3) < lim_col;
          sc[r] = seen ? sacc[r] * a.qk_scale_log2 : -INFINITY;
          mx = fmaxf(mx, sc[r]);
        }
      }
      mx = fmaxf(mx, shfl_xor(mx, 32));
      if (wave_any(mx > m + kRescaleThreshold)) {
        const float mn = fmaxf(m, mx);
        const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
#pragma unroll
        for (int e = 0; e < DB; ++e) acc[e] *= alpha;
        l *= alpha;
        m = mn;
      }
      float p[16];
      if (open) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = fast_exp2(sc[r] - m);
          l += p[r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = sc[r] == -INFINITY ? 0.f : fast_exp2(sc[r] - m);
          l += p[r];
        }
      }
      // ---- PV: position slots of product t are the lane's registers 8 t .. 8 t + 7
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        i32x4 phi, plo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = p[8 * t + 2 * e], p1 = p[8 * t + 2 * e + 1];
          if constexpr (kBf16) {
            const uint32_t hi = pack_bf16(p0, p1);
            phi[e] = (int)hi;
            plo[e] = (int)pack_bf16(p0 - __uint_as_float(hi << 16), p1 - __uint_as_float(hi & 0xFFFF0000u));
          } else {
            phi[e] = (int)pack_f16(p0, p1);
          }
        }
        // V^T rows d = 32 e + j; slots 0..3 are positions 16 t + 4 g2 .. + 3,
        // slots 4..7 positions 16 t + 8 + 4 g2 .. + 3
        const uint8_t* vt = sb + kChunk * KP + j * VP + 2 * (16 * t + 4 * g2);
#pragma unroll
        for (int e = 0; e < DB; ++e) {
          const i32x2 v0 = *reinterpret_cast<const i32x2*>(vt + (32 * e) * VP);
          const i32x2 v1 = *reinterpret_cast<const i32x2*>(vt + (32 * e) * VP + 16);
          const i32x4 vop = {v0[0], v0[1], v1[0], v1[1]};
          acc[e] = mfma32x32<CT>(vop, phi, acc[e]);
          if constexpr (kBf16) acc[e] = mfma32x32<CT>(vop, plo, acc[e]);
        }
      }
    };

    i32x4 pieces[2];
    load(0, pieces);
    store(0, pieces);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      const bool more = c + 1 < nchunks;
      if (more) {
        ring.advance();
        load(c + 1, pieces);
      }
      if (has) compute(c);
      if (more) store(c + 1, pieces);
      __syncthreads();
    }

    // ---- epilogue: lane (j, g2) holds d = 32 e + 8 R + 4 g2 + 0..3 of its column
    l += shfl_xor(l, 32);
    if (has && live) {
      const bool whole = whole_sequence(sl, cur.cs, cur.ce);
      const float f = whole ? 1.f / l : 1.f;
      const int64_t prow = whole ? 0 : part_row(a, sl.k, s, cq, head);
#pragma unroll
      for (int e = 0; e < DB; ++e)
#pragma unroll
        for (int R = 0; R < 4; ++R) {
          const int d0 = 32 * e + 8 * R + 4 * g2;
          const float v[4] = {acc[e][4 * R] * f, acc[e][4 * R + 1] * f, acc[e][4 * R + 2] * f, acc[e][4 * R + 3] * f};
          if (whole)
            store_out(a, row0 + cq, head, D, d0, v, 4);
          else
            store_partial(a, prow, D, d0, v, 4);
        }
      if (!whole && g2 == 0) store_ml(a, prow, m, l);
    }

    cur = next_segment(a, sl, cum, lens, s + 1);
  }
}

#define PA_PREFILL_CASE(CT, D, BS)                                                                       \
  if (ct == CT::code && qt == CT::code && head_dim == D && bs == BS) {                                   \
    launch_with_events(prefill_kernel<CT, D, BS>, grid, dim3(64 * kPrefillWaves), stream, ev, a);        \
    return true;                                                                                         \
  }
#define PA_PREFILL_BS(CT, D) \
  PA_PREFILL_CASE(CT, D, 8)  \
  PA_PREFILL_CASE(CT, D, 16) \
  PA_PREFILL_CASE(CT, D, 32)

// Several queries per sequence on a 16-bit cache read with a query of its
// own dtype, head_dim 64 or 128, block size 8, 16 or 32; grid = slices x KV
// heads x a.head_tiles groups of 256 columns.
bool launch_prefill(const DecodeArgs& a, int ct, int qt, int head_dim, int bs, dim3 grid, hipStream_t stream,
                    const LaunchEvents& ev) {
  PA_PREFILL_BS(F16, 64)
  PA_PREFILL_BS(F16, 128)
  PA_PREFILL_BS(BF16, 64)
  PA_PREFILL_BS(BF16, 128)
  return false;
}

}  // namespace pa
