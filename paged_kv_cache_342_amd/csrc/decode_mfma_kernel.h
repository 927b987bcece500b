// Paged decode attention on the matrix cores (v_mfma_f32_16x16x32_{f16,bf16}).
//
// One wavefront walks one slice of the batch (decode_common.h) for one KV
// head and one tile of up to 16 of its query heads, 32 positions (a chunk)
// at a time.  Per chunk:
//   QK:  S^T[tok, head] = K[tok, :] . Q[head, :]  as two 16x16 output tiles,
//        K rows are the A operand (one position per lane row), the group's
//        query heads are the B operand (padded to 16 columns).
//   PV:  O^T[d, head] += V^T[d, tok] . P^T[tok, head] with the probabilities
//        as the B operand straight from the QK accumulator registers.
// Both products sum over an index (head_dim for QK, position for PV) whose
// order inside one MFMA is free as long as A and B agree, which lets every
// lane fetch contiguous 16-byte pieces: K rows give 64 contiguous bytes per
// row per load instruction, and V is fetched as whole rows (16 lanes x 16 B)
// and transposed inside each lane's registers (8 positions x head_dim/16
// values) with byte permutes.  The next chunk's K/V is in flight in
// registers while the current one is computed; loads are nontemporal, and
// none of them sits under a branch (positions past the end of a segment
// re-read its last row and get a score of -inf).
//
// Several queries per sequence (MQ): the columns of a tile are (query, head)
// pairs instead of heads -- column c is query c / G of the sequence and head
// c % G of the group -- and each column masks the positions its query may
// not see (past L - n + j for query j of n).  A tile none of whose columns is
// a query of the sequence skips the segment.  When a sequence's queries span
// several tiles, one wave computes TW = 2 tiles per chunk: the K/V loads,
// their addresses and the V transposes are shared by both, only the
// products and the softmax are per tile.
//
// FP8 and FP4 caches with a scale per (slot, kv head) row (RS): each lane
// also loads the scales of the positions its scores and its V values belong
// to (four consecutive positions per 16-byte load); a score is multiplied by
// its K row's scale, and the probability that weights a V row by that row's
// scale (the denominator takes the probability itself).  An FP4 row is
// head_dim / 2 bytes: a lane takes a quarter of each K row as one load (so
// the k-slot order puts D/4 consecutive elements in each lane group) and
// head_dim / 16 elements of each V row; the hardware converts two E2M1 codes
// per instruction, exactly, to 16 bits.
//
// When the launch also appends each sequence's new row (16-bit caches), the
// loads of position L - 1 read the caller's row instead of the cache, and
// the wave that owns the sequence's last chunk stores that row into its slot
// at the end of the segment.
//
// Softmax runs online in fp32 in the log2 domain.  The running maximum of a
// head only moves when some score exceeds it by more than kRescaleThreshold
// (a wave-uniform branch); otherwise probabilities are 2^(s - m) <= 2^8,
// so the accumulator is rescaled rarely.  The result is exact regardless,
// since numerator and denominator share the same reference.
//
// P for the PV product: fp16 when V is fp16 or fp8 with a scale per tensor
// (fp8 -> fp16 is exact), and a two-term bf16 split (hi + lo) when V is bf16
// or carries row scales, so the weights keep ~16 bits (and, with row scales,
// the range of fp32: p * scale reaches 2^8 * max|V| / 6 for FP4).  Scores use q * k products of the 16-bit inputs, exact in
// the fp32 accumulator; scale * log2(e) is applied in fp32 afterwards.
#pragma once

#include <type_traits>

#include "decode_common.h"

namespace pa {

template <class T>
__device__ __forceinline__ f32x4 mfma32(i32x4 a, i32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma32<F16>(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma32<BF16>(i32x4 a, i32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Registers of one 32-position chunk, as loaded from memory.  A lane takes
// a quarter of each of 16 K rows per tile (KB bytes) and 1/16 of each of 8
// V rows (VB bytes).
template <class CT, int D>
struct ChunkRaw {
  static constexpr int KB = D * CT::bits / 32;          // K bytes per lane per 16-row tile
  static constexpr int VB = D * CT::bits / 128;         // V bytes per lane per position
  static constexpr int KR = KB >= 16 ? KB / 16 : 1;     // 16-byte K loads (FP4 at D = 64: one 8-byte load)
  static constexpr int VD = VB >= 4 ? VB / 4 : 1;       // dwords of V per lane per position
  i32x4 k[2][KR];
  uint32_t v[8][VD];
};

// Row scales of one chunk: positions 16 * tt + 4 * gq .. + 3 for K and V.
struct ChunkScales {
  f32x4 k[2];
  f32x4 v[2];
};
struct NoScales {};

template <int BYTES>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t* o) {
  if constexpr (BYTES == 16) {
    i32x4 x = ld16_stream(p);
    o[0] = x[0]; o[1] = x[1]; o[2] = x[2]; o[3] = x[3];
  } else if constexpr (BYTES == 8) {
    i32x2 x = ld8_stream(p);
    o[0] = x[0]; o[1] = x[1];
  } else if constexpr (BYTES == 4) {
    o[0] = ld4_stream(p);
  } else {
    o[0] = ld2_stream(p);
  }
}

// two fp32 -> packed 16-bit pair, round to nearest even (hardware converts)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <class CT, bool RS, int TW, int NW, int BS, bool PLAIN>
struct MfmaWaves {
  static constexpr int value = (NW == kSharedWaves1 || mfma_two_waves(CT::code, RS, TW, BS, PLAIN)) ? 2 : 1;
};

// NW > 1 (several queries per sequence, 16-bit caches): a workgroup of NW
// waves walks one slice for NW consecutive groups of TW tiles (NW = 4 waves
// of two tiles at one wave per SIMD, or NW = 8 waves of one tile at two per
// SIMD) and shares each K/V chunk through LDS.  Every lane loads a few 16-byte pieces
// of the chunk and stores them into one of two LDS stages; after a barrier
// each wave reads its MFMA operands from the stage in the byte pattern the
// one-wave kernel loads from memory.  All waves of the workgroup walk the
// same segments and chunks, so every barrier is reached by all of them; a
// wave whose tiles hold no query of the sequence loads and waits but does
// not compute.
//
// WIN (one query per sequence, no row scales): attention sinks plus a
// sliding window.  The walk visits the sink chunks and the window chunks of
// each sequence (visit_len), the id ring skips the table entries in between,
// and a position is masked unless it is below the sink or at or past
// L - window; since a segment can then see no position at all, p and the
// rescale are guarded as under MQ.
//
// CAS: the two passes of a decode over shared prefixes (DecodeArgs).
//   kPrefixPass (MQ): the "sequences" are groups, their queries the members'
//     rows, every member seeing the whole prefix through the table row of the
//     group's first member; a segment that is a whole prefix leaves each
//     member's unnormalised state (m, l, acc) in its state rows, a cut one a
//     partial as usual (merged into the state rows afterwards).
//   kSuffixPass (WIN): each sequence attends from its group's prefix length
//     on (LDS qrow holds those first positions) and its first segment starts
//     from the state the prefix pass left, so the usual epilogue and merge
//     give the attention over all of its positions.
constexpr int kPlainPass = 0;
constexpr int kPrefixPass = 1;
constexpr int kSuffixPass = 2;

template <class CT, class QT, int D, int BS, bool MQ, bool RS, int TW, int NW = 1, bool WIN = false,
          int CAS = kPlainPass>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(MfmaWaves<CT, RS, TW, NW, BS, !MQ && CAS == kPlainPass>::value)))
void decode_mfma_kernel(DecodeArgs a) {
  static_assert(!WIN || (!MQ && !RS && NW == 1), "windows: one query per sequence, a scale per tensor");
  static_assert(CAS != kPrefixPass || (MQ && !RS && NW == 1), "the prefix pass is a several-queries launch");
  static_assert(CAS != kSuffixPass || WIN, "the suffix pass walks from each sequence's first position");
  constexpr bool kMasked = MQ || WIN;  // a column may see no position of a chunk or a segment
  constexpr bool kStarts = CAS == kSuffixPass;  // qrow holds first attended positions
  constexpr int RB = D * CT::bits / 8;  // bytes per cache row
  constexpr int KK = D / 32;   // MFMAs per QK tile
  constexpr int W = D / 16;    // V values per lane per position (one output d-run)
  constexpr bool kFp8 = std::is_same<CT, FP8>::value;
  constexpr bool kFp4 = std::is_same<CT, FP4>::value;
  // PV in bf16 with P split in two terms: for bf16 caches, and for caches
  // with row scales, whose weights p * scale can exceed the fp16 range
  constexpr bool kBf16V = std::is_same<CT, BF16>::value || RS;
  using PT = typename std::conditional<kBf16V, BF16, F16>::type;  // PV operand type
  using Raw = ChunkRaw<CT, D>;
  using Scales = typename std::conditional<RS, ChunkScales, NoScales>::type;
  constexpr int VD = Raw::VD;
  constexpr int64_t kChunkBytes = (int64_t)BS * RB;  // one (block, head) chunk
  constexpr int NB = kChunk / BS;
  constexpr bool kCanAppend = !kFp8 && !kFp4;  // new rows are stored as given
  constexpr int kRowLanes = RB / 16;  // lanes that hold one row, 16 bytes each

  constexpr int kScan =
      scan_capacity(MQ || kStarts, MfmaWaves<CT, RS, TW, NW, BS, !MQ && CAS == kPlainPass>::value == 2);
  __shared__ int cum[kScan + 1];
  __shared__ int lens[kScan];
  __shared__ int qrow[(MQ || kStarts) ? kScan + 1 : 1];
  constexpr bool kShared = NW > 1;
  static_assert(!kShared || (MQ && !RS && CT::bits == 16), "shared chunks: several queries, 16-bit caches");
  // LDS stages: [2 stages][K, V][kChunk rows] at a pitch of RB + 16 bytes, so
  // that the 16 rows one K read spans fall on different banks
  constexpr int kPitch = RB + 16;
  constexpr int kPieceRow = RB / 16;                        // 16-byte pieces per row
  constexpr int kPieces = 2 * kChunk * kPieceRow / (64 * NW);  // pieces each lane loads
  static_assert(!kShared || kPieces * 64 * NW == 2 * kChunk * kPieceRow, "pieces per lane");
  __shared__ __attribute__((aligned(16))) uint8_t stage[kShared ? 2 * 2 * kChunk * kPitch : 16];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;  // wave within the workgroup
  const int r = lane & 15;   // A-operand row / B-operand column / C column
  const int gq = lane >> 4;  // k-slot group
  const int Hq = a.Hkv * a.G;
  const int64_t blk_stride = (int64_t)a.Hkv * kChunkBytes;

  // wave -> (slice, head tile, KV head); the KV head varies fastest, so the
  // workgroups of one KV head land on the same XCD
  // (with NW waves per workgroup, head_tiles counts workgroups per slice and
  // KV head, and wave wv takes tile pair NW * that + wv).
  // With row scales the order is XCD-major instead: workgroups go to the
  // XCDs in turn, so workgroup b runs on XCD b % kXcds and takes item
  // (b % kXcds) * (N / kXcds) + b / kXcds, and every XCD takes a contiguous
  // run of items (KV head fastest).  The scale rows of KV heads 2p and
  // 2p + 1 share one 128-byte line, which is then fetched by one XCD's L2
  // rather than two.
  int item = blockIdx.x;
  if constexpr (RS) {
    const int n = (int)gridDim.x;
    if (n % (2 * kXcds) == 0) item = (item % kXcds) * (n / kXcds) + item / kXcds;
  }
  const int h = item % a.Hkv;
  const int rest = item / a.Hkv;
  const int ht = (rest % a.head_tiles) * NW + wv;
  const int k = rest / a.head_tiles;

  // the host sizes every launch to the scan arrays (scan_capacity); a launch
  // that did not fit would write past them
  if (a.B > kScan) return;
  Slice sl;
  if (!slice_setup(a, cum, lens, (MQ || kStarts) ? qrow : nullptr, k, sl)) return;
  const int* starts = kStarts ? qrow : nullptr;  // first attended positions (suffix pass)

  // this lane's column in each of the wave's TW tiles: its query within the
  // sequence (MQ) and its head within the group
  int cq[TW], head[TW];
  bool col_ok[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int col = 16 * (TW * ht + t) + r;
    cq[t] = MQ ? col / a.G : 0;
    const int col_head = MQ ? col - cq[t] * a.G : col;
    col_ok[t] = MQ ? cq[t] < a.nq : col < a.G;
    head[t] = h * a.G + (col_ok[t] ? col_head : 0);
  }
  const uint8_t* kbase = a.k_cache + (int64_t)h * kChunkBytes;
  const uint8_t* vbase = a.v_cache + (int64_t)h * kChunkBytes;

  // empty contexts in this slice: zero rows, written by the slice that owns
  // them (a sequence with no positions has no queries under MQ)
  for (int s = sl.s_first; s < a.B && !MQ; ++s) {
    const int cs = cum[s], ce = cum[s + 1];
    if (past_slice(sl, cs, ce)) break;
    if (lens[s] == 0 && col_ok[0]) {
      float z[4 * W];
#pragma unroll
      for (int i = 0; i < 4 * W; ++i) z[i] = 0.f;
      store_out(a, s, head[0], D, 4 * W * gq, z, 4 * W);
    }
  }

  // What a segment needs before its first chunk: the query (B operand of QK,
  // in the k-slot order the K loads use), its block-id ring and where its
  // last row is read from (by lanes whose position lies past the end, and,
  // when appending, by the last position itself).  Each segment's header is
  // requested one segment ahead, with loads that do not depend on whether
  // there is a next segment (past the last one the current segment's header
  // is read again), so segment changes cost no table or query round trips.
  struct Header {
    i32x4 qop[TW][KK];
    IdRing<BS, WIN> ring;
    const uint8_t* last_k;  // row of the last position
    const uint8_t* last_v;
    int lim;                // positions from lim on read last_k / last_v
    int64_t tail_off;       // cache offset the appended row goes to; -1 = none
    int qrow0;              // row of the sequence's first query
    int nqs;                // its queries (1 for decode)
  };
  auto load_query = [&](const Segment& g, Header& hd) {
    // a column that is no query of the sequence reads a row that exists
    // (row 0) and contributes zeros
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      const bool live = MQ ? cq[t] < hd.nqs : col_ok[t];
      const int64_t qr = MQ ? (live ? hd.qrow0 + cq[t] : 0) : g.s;
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(a.q) + (qr * Hq + (live ? head[t] : h * a.G)) * D * 2;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        // the k-slot order of the K loads: lane group gq holds a quarter of
        // each row (FP4), two 16-byte pieces (fp8) or four (16-bit)
        const int d = kFp4 ? (D / 4) * gq + 8 * kk : kFp8 ? 64 * (kk >> 1) + 16 * gq + 8 * (kk & 1) : 32 * kk + 8 * gq;
        const i32x4 x = ld16(qrow + d * 2);
        hd.qop[t][kk] = live ? x : i32x4{0, 0, 0, 0};
      }
    }
  };
  // The shared-chunk kernel loads a segment's query when the segment starts
  // rather than a segment ahead: a second query buffer would not fit its
  // registers, and its segments (long query chunks) are long.
  constexpr bool kQueryLate = kShared;
  auto load_header = [&](const Segment& g, Header& hd) {
    hd.qrow0 = g.s;
    hd.nqs = 1;
    if constexpr (MQ) {
      int row0, n;
      query_range(a, qrow, g.s, lens[g.s], row0, n, CAS != kPrefixPass);
      hd.qrow0 = uniform(row0);
      hd.nqs = uniform(n);
    }
    if constexpr (!kQueryLate) load_query(g, hd);
    // the prefix pass reads a group's prefix through its first member's table row
    const int32_t* trow = a.block_tables + (int64_t)(CAS == kPrefixPass ? hd.qrow0 : g.s) * a.M;
    const int blk0 = g.tok0 / BS;
    int last_blk = (g.tok_end - 1) / BS;  // visited block of the last position
    if constexpr (WIN) {
      // visited blocks from the end of the sink chunks on lie g.shift / BS
      // table entries further on
      const int sink_blocks = (attend_sink(a) + kChunk - 1) / kChunk * NB;
      const int gap = g.shift / BS;
      hd.ring.start(trow + blk0, (g.tok_end + BS - 1) / BS - blk0, sink_blocks - blk0, gap);
      if (last_blk >= sink_blocks) last_blk += gap;
    } else {
      hd.ring.start(trow + blk0, (g.tok_end + BS - 1) / BS - blk0);
    }
    int id = uniform(trow[last_blk]);
    const bool id_ok = id >= 0 && (int64_t)id < a.num_blocks;
    if (!id_ok) id = 0;
    const int64_t off = (int64_t)id * blk_stride + (int64_t)((g.tok_end - 1) % BS) * RB;
    const bool app = kCanAppend && a.new_k != nullptr && g.tok_end == lens[g.s];
    const int64_t nrow = ((int64_t)g.s * a.Hkv + h) * RB;
    hd.last_k = app ? a.new_k + nrow : kbase + off;
    hd.last_v = app ? a.new_v + nrow : vbase + off;
    hd.lim = g.tok_end - (app ? 1 : 0);
    hd.tail_off = app && id_ok && ht == 0 ? off : -1;
  };

  Segment cur = next_segment(a, sl, cum, lens, sl.s_first, starts);
  if (cur.s < 0) return;
  Header hc, hn;
  load_header(cur, hc);
  if constexpr (kQueryLate) load_query(cur, hc);
  Segment nxt = next_segment(a, sl, cum, lens, cur.s + 1, starts);
  load_header(nxt.s >= 0 ? nxt : cur, hn);

  while (true) {
    const int s = cur.s;
    const int cs = cur.cs, ce = cur.ce;
    const int tok0 = cur.tok0, tok_end = cur.tok_end, nchunks = cur.nchunks;
    IdRing<BS, WIN>& ring = hc.ring;
    const int lim = hc.lim;
    // WIN: a visited position p is seen if p < sink or p + shift >= lo (lo =
    // L - window, or the sequence's first position in the suffix pass; in the
    // sink chunks p + shift stays below lo whenever shift > 0)
    const int win_shift = WIN ? cur.shift : 0;
    const int win_sink = WIN ? attend_sink(a) : 0;
    const int win_lo = WIN ? attend_lo(a, lens[s], kStarts ? min(starts[s], lens[s]) : 0) : 0;
    bool live[TW];
    int qlim[TW];  // last position each column's query sees (MQ)
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      live[t] = MQ ? cq[t] < hc.nqs : col_ok[t];
      // (the prefix pass: every member sees the whole prefix)
      qlim[t] = MQ ? (CAS == kPrefixPass ? lens[s] - 1 : lens[s] - hc.nqs + cq[t]) : 0;
    }
    // the appended row, stored at the end of the segment: lane i < kRowLanes
    // holds 16 bytes of K, the next kRowLanes lanes 16 bytes of V
    i32x4 app_row = {0, 0, 0, 0};
    if (kCanAppend && a.new_k != nullptr)
      app_row = ld16((lane < kRowLanes ? hc.last_k : hc.last_v) + 16 * (lane % kRowLanes));

    auto load_chunk = [&](int c, Raw& raw, Scales& scl) {
      const int ctok = tok0 + kChunk * c;  // first position of the chunk
      int id[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int x = ring.id(c, i);
        id[i] = (x < 0 || (int64_t)x >= a.num_blocks) ? 0 : x;
      }
      // K: rows 16*tt + r
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int tc = 16 * tt + r;
        const int bsel = BS == 32 ? 0 : (BS == 16 ? tt : 2 * tt + (r >> 3));
        const bool ok = ctok + tc < lim;
        const uint8_t* row = ok ? kbase + (int64_t)id[bsel] * blk_stride + (tc % BS) * RB : hc.last_k;
        if constexpr (kFp4 && Raw::KB == 8) {
          const i32x2 x = ld8_stream(row + 8 * gq);
          raw.k[tt][0] = i32x4{x[0], x[1], 0, 0};
        } else {
#pragma unroll
          for (int u = 0; u < Raw::KR; ++u) {
            const int off = kFp4 ? 16 * gq : kFp8 ? 64 * u + 16 * gq : (32 * u + 8 * gq) * 2;
            raw.k[tt][u] = ld16_stream(row + off);
          }
        }
      }
      // V: whole rows, position slot j -> 16*(j>>2) + 4*gq + (j&3)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int tc = 16 * (j >> 2) + 4 * gq + (j & 3);
        const int bsel = BS == 32 ? 0 : (BS == 16 ? (j >> 2) : 2 * (j >> 2) + (gq >> 1));
        const bool ok = ctok + tc < lim;
        const uint8_t* row = ok ? vbase + (int64_t)id[bsel] * blk_stride + (tc % BS) * RB : hc.last_v;
        load_bytes<Raw::VB>(row + Raw::VB * r, raw.v[j]);
      }
      if constexpr (RS) {
        // the scales of positions 16*tt + 4*gq .. + 3 (one block; past the end
        // of the segment the ring's ids stay valid and the scores are masked)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int tc = 16 * tt + 4 * gq;
          const int bsel = BS == 32 ? 0 : (BS == 16 ? tt : 2 * tt + (gq >> 1));
          const int64_t off = ((int64_t)id[bsel] * a.Hkv + h) * BS + tc % BS;
          scl.k[tt] = *reinterpret_cast<const f32x4*>(a.k_row_scale + off);
          scl.v[tt] = *reinterpret_cast<const f32x4*>(a.v_row_scale + off);
        }
      }
    };

    float m[TW], l[TW];
    f32x4 acc[TW][W];
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      m[t] = -INFINITY;
      l[t] = 0.f;
#pragma unroll
      for (int i = 0; i < W; ++i) acc[t][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (kStarts) {
      // the suffix pass: a sequence's first segment starts from the state the
      // prefix pass left for it (none when it shares no prefix); l is summed
      // over the four lane groups at the end, so one of them holds it
      if (tok0 == 0 && starts[s] > 0) {
        const int64_t row = (int64_t)s * Hq + head[0];
        const f32x2 ml = *reinterpret_cast<const f32x2*>(a.state_ml + 2 * row);
        const float* src = a.state_acc + row * D + 4 * W * gq;
        m[0] = ml[0];
        l[0] = gq == 0 ? ml[1] : 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int dt = 0; dt < W; ++dt) acc[0][dt][jj] = src[W * jj + dt];
      }
    }

    auto compute_chunk = [&](int c, const Raw& raw, const Scales& scl) {
      const int ctok = tok0 + kChunk * c;
      // ---- QK
      i32x4 kop[2][KK];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        if constexpr (kFp4) {
          // dword kk of the lane's piece: the 8 elements MFMA kk takes
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) kop[tt][kk] = fp4x8_to_16<QT>((uint32_t)raw.k[tt][0][kk]);
        } else if constexpr (kFp8) {
#pragma unroll
          for (int u = 0; u < Raw::KR; ++u) {
            const i32x2 lo = fp8x4_to_16<QT>((uint32_t)raw.k[tt][u][0]);
            const i32x2 lo2 = fp8x4_to_16<QT>((uint32_t)raw.k[tt][u][1]);
            const i32x2 hi = fp8x4_to_16<QT>((uint32_t)raw.k[tt][u][2]);
            const i32x2 hi2 = fp8x4_to_16<QT>((uint32_t)raw.k[tt][u][3]);
            kop[tt][2 * u] = i32x4{lo[0], lo[1], lo2[0], lo2[1]};
            kop[tt][2 * u + 1] = i32x4{hi[0], hi[1], hi2[0], hi2[1]};
          }
        } else {
#pragma unroll
          for (int u = 0; u < KK; ++u) kop[tt][u] = raw.k[tt][u];
        }
      }
      f32x4 s0[TW], s1[TW];
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        s0[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        s1[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          s0[t] = mfma32<QT>(kop[0][kk], hc.qop[t][kk], s0[t]);
          s1[t] = mfma32<QT>(kop[1][kk], hc.qop[t][kk], s1[t]);
        }
      }
      i32x4 pop[TW], plo[TW];
      // The softmax of the chunk's scores, written for a chunk some of whose
      // positions a column does not see (masked) and for one whose positions
      // every column sees: with one query per sequence and no window, every
      // chunk of a segment but its last (the selects and checks skipped).
      auto softmax = [&](auto masked) {
        constexpr bool kM = decltype(masked)::value;
#pragma unroll
        for (int t = 0; t < TW; ++t) {
          // ---- online softmax for this lane's column (head) of tile t, positions j
          float sc[8];
          float mx = -INFINITY;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            float raw_s = (j < 4 ? s0[t][j & 3] : s1[t][j & 3]) * a.qk_scale_log2;
            if constexpr (RS) raw_s *= scl.k[j >> 2][j & 3];
            const int tc = 16 * (j >> 2) + 4 * gq + (j & 3);
            const bool seen = !kM || (ctok + tc < tok_end && (!MQ || ctok + tc <= qlim[t]) &&
                                      (!WIN || ctok + tc < win_sink || ctok + tc + win_shift >= win_lo));
            sc[j] = seen ? raw_s : -INFINITY;
            mx = fmaxf(mx, sc[j]);
          }
          if (wave_any(mx > m[t] + kRescaleThreshold)) {
            mx = fmaxf(mx, shfl_xor(mx, 16));
            mx = fmaxf(mx, shfl_xor(mx, 32));
            const float mn = fmaxf(m[t], mx);
            // under MQ or a window a column may have seen no position yet (mn = -inf)
            const float alpha = (kMasked && mn == -INFINITY) ? 1.f : fast_exp2(m[t] - mn);
#pragma unroll
            for (int i = 0; i < W; ++i) acc[t][i] *= alpha;
            l[t] *= alpha;
            m[t] = mn;
          }
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            p[j] = (kMasked && sc[j] == -INFINITY) ? 0.f : fast_exp2(sc[j] - m[t]);
            l[t] += p[j];
          }
          // ---- P as the B operand of PV (weighted by the V rows' scales under
          // RS; a masked position's scale may belong to a slot never written, so
          // its weight is set, not computed)
          float pw[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if constexpr (RS)
              pw[j] = (kM && sc[j] == -INFINITY) ? 0.f : p[j] * scl.v[j >> 2][j & 3];
            else
              pw[j] = p[j];
          }
#pragma unroll
          for (int jp = 0; jp < 4; ++jp) {
            if constexpr (kBf16V) {
              uint32_t hi = pack_bf16(pw[2 * jp], pw[2 * jp + 1]);
              // opaque to the optimiser, which would otherwise convert the
              // first weight a second time instead of shifting the pair
              asm("" : "+v"(hi));
              const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xFFFF0000u);
              pop[t][jp] = (int)hi;
              plo[t][jp] = (int)pack_bf16(pw[2 * jp] - h0, pw[2 * jp + 1] - h1);
            } else {
              pop[t][jp] = (int)pack_f16(pw[2 * jp], pw[2 * jp + 1]);
            }
          }
        }
      };
      if (!MQ && !WIN && ctok + kChunk <= tok_end)
        softmax(std::false_type());
      else
        softmax(std::true_type());
      // ---- V^T as the A operand: 16-bit values per position, then transpose
      uint32_t vt[8][W / 2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (kFp4) {
          if constexpr (W == 8) {
            const i32x4 x = fp4x8_to_16<PT>(raw.v[j][0]);
#pragma unroll
            for (int i = 0; i < 4; ++i) vt[j][i] = (uint32_t)x[i];
          } else {
            const i32x2 x = fp4x4_to_16<PT>(raw.v[j][0]);
            vt[j][0] = (uint32_t)x[0];
            vt[j][1] = (uint32_t)x[1];
          }
        } else if constexpr (kFp8) {
#pragma unroll
          for (int i = 0; i < VD; ++i) {
            const i32x2 x = fp8x4_to_16<PT>(raw.v[j][i]);
            vt[j][2 * i] = (uint32_t)x[0];
            vt[j][2 * i + 1] = (uint32_t)x[1];
          }
        } else {
#pragma unroll
          for (int i = 0; i < W / 2; ++i) vt[j][i] = raw.v[j][i];
        }
      }
#pragma unroll
      for (int dt = 0; dt < W; ++dt) {
        i32x4 vop;
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) {
          const uint32_t a0 = vt[2 * jp][dt >> 1], a1 = vt[2 * jp + 1][dt >> 1];
          vop[jp] = (dt & 1) ? (int)__builtin_amdgcn_perm(a1, a0, 0x07060302u)
                             : (int)__builtin_amdgcn_perm(a1, a0, 0x05040100u);
        }
#pragma unroll
        for (int t = 0; t < TW; ++t) {
          acc[t][dt] = mfma32<PT>(vop, pop[t], acc[t][dt]);
          if constexpr (kBf16V) acc[t][dt] = mfma32<PT>(vop, plo[t], acc[t][dt]);
        }
      }
    };

    // Walk over the segment's chunks with the next chunk in flight while one
    // is computed (16 KiB requested per wave for 16-bit caches, 8 KiB for
    // fp8, whose waves are bound by instruction issue rather than by bytes in
    // flight: a third buffer measured 3% slower there).  Later chunks are
    // always requested (past the end every lane reads the last row), so no
    // load sits under a branch and each wait covers only the chunk it needs.
    // (Under MQ a tile with no query of this sequence among its columns skips
    // the segment.)
    if constexpr (kShared) {
      // this lane's pieces of chunk c: K rows, then V rows, kPieceRow per row
      auto sh_load = [&](int c, i32x4* piece) {
        const int ctok = tok0 + kChunk * c;
        int id[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int x = ring.id(c, i);
          id[i] = (x < 0 || (int64_t)x >= a.num_blocks) ? 0 : x;
        }
#pragma unroll
        for (int q = 0; q < kPieces; ++q) {
          const int pc = (int)threadIdx.x + 64 * NW * q;
          const int kv = pc / (kChunk * kPieceRow);
          const int rem = pc - kv * (kChunk * kPieceRow);
          const int pos = rem / kPieceRow;
          const int col = rem - pos * kPieceRow;
          int bid = id[0];
#pragma unroll
          for (int i = 1; i < NB; ++i)
            if (pos / BS == i) bid = id[i];
          const bool ok = ctok + pos < lim;
          const uint8_t* src = ok ? (kv ? vbase : kbase) + (int64_t)bid * blk_stride + (pos % BS) * RB
                                  : (kv ? hc.last_v : hc.last_k);
          piece[q] = ld16_stream(src + 16 * col);
        }
      };
      auto sh_store = [&](int c, const i32x4* piece) {
        uint8_t* sb = stage + (c & 1) * 2 * kChunk * kPitch;
#pragma unroll
        for (int q = 0; q < kPieces; ++q) {
          const int pc = (int)threadIdx.x + 64 * NW * q;
          const int kv = pc / (kChunk * kPieceRow);
          const int rem = pc - kv * (kChunk * kPieceRow);
          const int pos = rem / kPieceRow;
          const int col = rem - pos * kPieceRow;
          *reinterpret_cast<i32x4*>(sb + (kv * kChunk + pos) * kPitch + 16 * col) = piece[q];
        }
      };
      // the wave's operands of chunk c, in the byte pattern of load_chunk
      auto sh_read = [&](int c, Raw& raw) {
        const uint8_t* sb = stage + (c & 1) * 2 * kChunk * kPitch;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int u = 0; u < Raw::KR; ++u)
            raw.k[tt][u] = *reinterpret_cast<const i32x4*>(sb + (16 * tt + r) * kPitch + (32 * u + 8 * gq) * 2);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int tc = 16 * (j >> 2) + 4 * gq + (j & 3);
          const uint8_t* row = sb + (kChunk + tc) * kPitch + Raw::VB * r;
          if constexpr (Raw::VB == 16) {
            const i32x4 x = *reinterpret_cast<const i32x4*>(row);
            raw.v[j][0] = x[0]; raw.v[j][1] = x[1]; raw.v[j][2] = x[2]; raw.v[j][3] = x[3];
          } else {
            const i32x2 x = *reinterpret_cast<const i32x2*>(row);
            raw.v[j][0] = x[0]; raw.v[j][1] = x[1];
          }
        }
      };
      const bool has = 16 * TW * ht < hc.nqs * a.G;
      i32x4 pieces[kPieces];
      sh_load(0, pieces);
      sh_store(0, pieces);
      __syncthreads();
      for (int c = 0; c < nchunks; ++c) {
        const bool more = c + 1 < nchunks;
        if (more) {
          ring.advance();
          sh_load(c + 1, pieces);
        }
        if (has) {
          Raw raw;
          Scales scl;
          sh_read(c, raw);
          compute_chunk(c, raw, scl);
        }
        if (more) sh_store(c + 1, pieces);
        __syncthreads();
      }
    } else if (!MQ || 16 * TW * ht < hc.nqs * a.G) {
      Raw buf0, buf1;
      Scales sc0, sc1;
      load_chunk(0, buf0, sc0);
      for (int c = 0; c < nchunks; c += 2) {
        ring.advance();
        load_chunk(c + 1, buf1, sc1);
        compute_chunk(c, buf0, sc0);
        if (c + 1 >= nchunks) break;
        ring.advance();
        load_chunk(c + 2, buf0, sc0);
        compute_chunk(c + 1, buf1, sc1);
      }
    }

    // ---- epilogue: per tile the lane holds head[t] (of query cq[t]), d = 4W*gq + W*jj + dt
    const bool whole = whole_sequence(sl, cs, ce);
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      l[t] += shfl_xor(l[t], 16);
      l[t] += shfl_xor(l[t], 32);
      if (live[t]) {
        // the prefix pass keeps a whole prefix unnormalised, as the member's state
        constexpr bool kState = CAS == kPrefixPass;
        float v[4 * W];
        const float f = whole && !kState ? a.v_scale / l[t] : 1.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
#pragma unroll
          for (int dt = 0; dt < W; ++dt) v[W * jj + dt] = acc[t][dt][jj] * f;
        if (whole && kState) {
          const int64_t row = (int64_t)(hc.qrow0 + cq[t]) * Hq + head[t];
          float* o = a.state_acc + row * D + 4 * W * gq;
#pragma unroll
          for (int i = 0; i < 4 * W; i += 4) *reinterpret_cast<f32x4*>(o + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
          if (gq == 0) *reinterpret_cast<f32x2*>(a.state_ml + 2 * row) = f32x2{m[t], l[t]};
        } else if (whole) {
          store_out(a, MQ ? hc.qrow0 + cq[t] : s, head[t], D, 4 * W * gq, v, 4 * W);
        } else {
          const int64_t row = part_row(a, sl.k, s, cq[t], head[t]);
          store_partial(a, row, D, 4 * W * gq, v, 4 * W);
          if (gq == 0) store_ml(a, row, m[t], l[t]);
        }
      }
    }
    if (hc.tail_off >= 0 && lane < 2 * kRowLanes) {
      uint8_t* dst = const_cast<uint8_t*>(lane < kRowLanes ? kbase : vbase) + hc.tail_off;
      *reinterpret_cast<i32x4*>(dst + 16 * (lane % kRowLanes)) = app_row;
    }

    if (nxt.s < 0) break;
    cur = nxt;
    hc = hn;
    if constexpr (kQueryLate) load_query(cur, hc);
    nxt = next_segment(a, sl, cum, lens, cur.s + 1, starts);
    load_header(nxt.s >= 0 ? nxt : cur, hn);
  }
}

}  // namespace pa
