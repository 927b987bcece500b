// Shared parts of the paged decode kernels: launch arguments, the balanced
// split of the batch over wavefronts, the block-id prefetcher and the
// epilogue stores.
//
// Work split.  Every sequence is cut into chunks of kChunk consecutive
// positions (the last chunk may be partial) and the chunks of all sequences
// are laid end to end, sequence after sequence.  That line of C chunks is
// cut into equal slices of S chunks, and one wavefront handles one slice for
// one KV head (and one tile of up to 16 query heads): every wave streams the
// same number of K/V bytes, whatever the mix of context lengths, and it
// streams them as one long run.  A slice may hold the tail of one sequence,
// several whole sequences and the head of another; each such piece is a
// segment.  A segment that is a whole sequence is normalised and written to
// `out` directly.  A sequence cut by slice boundaries leaves one partial
// result per slice -- the running maximum m (log2 domain), the sum
// l = sum 2^(score - m) and acc = sum 2^(score - m) V for each query head --
// and the merge kernel combines them in slice order:
//   M = max_k m_k,  out = v_scale * sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k.
// The partial of sequence s from slice k is stored in row k + s, which is
// unique: the slices that cut s and those that cut s + 1 overlap in at most
// one slice.
//
// Each sequence also costs a wave a fixed amount beyond its chunks (the first
// chunk's latency, which nothing overlaps, a partly filled last chunk, the
// epilogue), so the line charges every non-empty sequence `seg_cost` virtual
// chunks in front of its data: a slice that holds many short sequences holds
// fewer chunks.
//
// Each wave computes the prefix sum of chunk counts itself (the lengths are
// read once into LDS), so no separate planning kernel runs before it.
#pragma once

#include <hip/hip_ext.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// Launch a kernel with the given events (hipExtLaunchKernel's start and
// stop), or as a plain launch when there are none.
template <class K, class... Args>
inline void launch_with_events(K kernel, dim3 grid, dim3 block, hipStream_t stream, const LaunchEvents& ev,
                               Args... args) {
  if (ev.start != nullptr || ev.stop != nullptr)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
}

constexpr int kChunk = 32;        // positions per chunk, the unit of the split
constexpr int kXcds = 8;          // accelerator dies (each with its own L2) that workgroups are dealt to in turn
constexpr int kScanMax = 4096;    // sequences one launch scans in LDS
// with several queries per sequence the first query rows are kept in LDS as
// well; three arrays of this many entries leave room for four waves per CU
constexpr int kScanMaxMQ = 3072;
// Kernels that run two waves per SIMD (eight per CU) scan half as many, so
// that eight workgroups' arrays fit the 160 KiB of LDS.
constexpr int kScanMax2 = 2048;
constexpr int kScanMaxMQ2 = 1536;
// The prefill kernel keeps its query rows and five K/V stages in LDS next to
// the arrays, which leaves room for this many sequences per launch.
constexpr int kScanPrefill = 512;

// Which MFMA kernels run two waves per SIMD.  FP4 with row scales: its waves
// are bound by instruction issue at one wave per SIMD (5% of their cycles
// waiting on memory), and its registers fit the 256 of two waves without
// spilling; a second wave per SIMD took the FP4 decode of the 8B-shaped and
// the heavy-tailed batches 15-16% faster.  fp8 with a scale per tensor at
// block size 8, one query per sequence and not a cascade pass (plain; a
// window included, so that a window covering every position still gives
// decode's bits): a chunk spans four blocks there, and the second wave hides
// their loads (heavy-tailed batch 107 -> 99 us); at block sizes 16 and 32 it
// was 1-2% slower (twice the slices, so more segments per wave).  The host
// sizes launches (scan capacity, slices) with the same rule.
__host__ __device__ constexpr bool mfma_two_waves(int cache_code, bool row_scales, int tiles_per_wave,
                                                  int block_size, bool plain) {
  return tiles_per_wave == 1 && ((cache_code == 4 && row_scales) ||
                                 (cache_code == 3 && !row_scales && plain && block_size == 8));
}
__host__ __device__ constexpr int scan_capacity(bool multi_query, bool two_waves) {
  return two_waves ? (multi_query ? kScanMaxMQ2 : kScanMax2) : (multi_query ? kScanMaxMQ : kScanMax);
}
constexpr int kIdAhead = 6;       // chunks of block ids held ahead of the loads
// Several queries per sequence spanning at least this many tile pairs (16-bit
// caches): a workgroup of this many waves, one per SIMD, shares each K/V
// chunk through LDS instead of every wave loading it.
constexpr int kSharedWaves = 4;
// The same with one tile per wave and two waves per SIMD, the default from
// this many tiles on: a workgroup of this many waves.
constexpr int kSharedWaves1 = 8;

struct DecodeArgs {
  void* out;                   // [B, Hq, D] (already offset to this launch's first sequence)
  const void* q;               // [B, Hq, D]
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables; // [B, M]
  const int32_t* context_lens; // [B]
  int32_t* meta;               // workspace: [0] = S, [1] = slices used, [2 + s] = first chunk of s (B + 1 entries)
  float* part_acc;             // workspace: [rows, Hq, D], rows = nslices + B
  float* part_ml;              // workspace: [rows, Hq, 2] = (m, l)
  int64_t num_blocks;
  int32_t B, Hkv, G, M;        // M = max_blocks_per_seq
  int32_t max_ctx;             // lengths are clamped to [0, max_ctx]
  int32_t nslices;             // slices per (KV head, head tile) in the grid
  int32_t min_slice;           // fewest chunks per slice
  int32_t seg_cost;            // virtual chunks charged per non-empty sequence
  int32_t head_tiles;          // query-head tiles of 16 per KV head (MFMA kernel), 1 otherwise
  int32_t out_dtype;           // 0 f32, 1 f16, 2 bf16
  float qk_scale_log2;         // scale * k_scale * log2(e)
  float v_scale;
  // Appending in the same launch (16-bit caches): the row of position L - 1
  // of every sequence, [B, Hkv, D] in the cache dtype; null = no append.
  // Loads of that position read these rows, never the cache, and the wave
  // that owns a sequence's last chunk (query-head tile 0) stores them into
  // the cache, so nothing in the launch reads a slot written by it.
  const uint8_t* new_k;
  const uint8_t* new_v;
  // Several queries per sequence (multi-query kernels only): the queries of
  // sequence s are rows q_start[s] .. q_start[s + 1] - 1 of q and out, at
  // most nq of them; query j of n sees positions 0 .. L - n + j.  Decode
  // kernels have nq == 1 and row s.
  const int32_t* q_start;
  int32_t nq;
  int32_t q_rows;  // rows of q and out (a query range outside them is dropped)
  // FP8 caches with a scale per (slot, kv head) row: [num_blocks, Hkv, bs]
  // fp32 each (row-scale kernels only; the per-tensor scales are then 1)
  const float* k_row_scale;
  const float* v_row_scale;
  // Attention sinks plus a sliding window (window > 0; window kernels
  // only): a sequence of L positions attends to t < sink and t >= L - window.
  // Its walk visits the chunks that hold such positions: the sink chunks
  // [0, ceil(sink / kChunk)), then the chunks from the one holding L - window
  // on.  Chunk-aligned positions of that walk ("visited" positions) equal
  // real ones in the sink chunks and are window_shift() below them after.
  int32_t sink;
  int32_t window;
  // Shared prefixes (pa_decode_shared_prefix): group p is sequences
  // group_start[p] .. group_start[p + 1] - 1, which share their first
  // prefix_lens[p] positions.  The prefix pass is a several-queries launch
  // over the groups (q_start = group_start, context_lens = prefix_lens, every
  // member sees the whole prefix, the table row of the group's first member);
  // it leaves each member's unnormalised state (m, l, acc) in state_ml /
  // state_acc ([B, Hq, 2] and [B, Hq, D], by sequence).  The suffix pass is a
  // decode launch whose sequences attend from their group's prefix_lens on
  // (a window with no sink and a first position of its own) and start from
  // that state.
  const int32_t* group_start;
  const int32_t* prefix_lens;
  int32_t n_groups;
  float* state_ml;
  float* state_acc;
};

// Positions the walk of a sequence skips between its first chunks (those
// holding positions below `sink`) and the chunks from the one holding `lo`
// on (a multiple of kChunk; 0 when they meet).
__host__ __device__ __forceinline__ int visit_shift(int sink, int lo) {
  const int sink_chunks = (sink + kChunk - 1) / kChunk;
  const int win_chunk = lo > 0 ? lo / kChunk : 0;
  return win_chunk > sink_chunks ? (win_chunk - sink_chunks) * kChunk : 0;
}

// What a sequence of L positions attends to, besides t < L: t < sink or
// t >= lo.  With a window, sink and L - window; in the suffix pass of
// shared prefixes, no sink and its own first position `start`; otherwise
// every position (lo = 0).
__device__ __forceinline__ int attend_sink(const DecodeArgs& a) { return a.window > 0 ? a.sink : 0; }
__device__ __forceinline__ int attend_lo(const DecodeArgs& a, int L, int start) {
  return a.window > 0 ? L - a.window : start;
}

// Positions the walk of a sequence of L positions visits.
__device__ __forceinline__ int visit_len(const DecodeArgs& a, int L, int start) {
  return L - visit_shift(attend_sink(a), attend_lo(a, L, start));
}

// Queries of sequence s under MQ (qs = q_start, in memory or in LDS): first
// row and count, clamped to at most nq, at most the sequence's length
// (causal: query j of n sees up to L - n + j) and to rows that exist.
__device__ __forceinline__ void query_range(const DecodeArgs& a, const int* qs, int s, int L, int& row0, int& n,
                                            bool causal = true) {
  row0 = qs[s];
  n = max(0, min(qs[s + 1] - row0, causal ? min(a.nq, L) : a.nq));
  if (row0 < 0 || row0 > a.q_rows - n) n = 0, row0 = 0;
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int wave_inclusive_sum(int x) {
  const int lane = __lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// This wave's slice [c0, c1) of the chunk line, and the first sequence it
// visits.  cum[s] (LDS) = where sequence s starts on the line (its charge,
// then its chunks), cum[B] = C.
struct Slice {
  int k;        // slice index
  int S;        // chunks per slice
  int neff;     // slices that hold work (>= 1)
  int c0, c1;   // chunk range
  bool last;    // the last slice also owns empty sequences at the very end
  int s_first;  // first sequence it visits
};

// Fills cum[], lens[] (clamped context lengths), qrow[] and sl; returns false
// when the slice holds nothing.  qrow (null if the kernel has none) gets
// q_start with several queries per sequence, or, in the suffix pass of
// shared prefixes (no q_start), each sequence's first attended position
// (its group's prefix length).  Wave 0 also publishes S, the slice count and
// cum[] for the merge kernel.
__device__ __forceinline__ bool slice_setup(const DecodeArgs& a, int* cum, int* lens, int* qrow, int k, Slice& sl) {
  const int lane = __lane_id();
  int carry = 0;
  const bool starts = qrow != nullptr && a.q_start == nullptr;
  if (qrow != nullptr && lane == 0) qrow[a.B] = starts ? 0 : a.q_start[a.B];
  if (starts) {
    for (int s = lane; s < a.B; s += 64) qrow[s] = 0;
    __syncthreads();
    for (int p = lane; p < a.n_groups; p += 64) {
      const int lo = max(a.group_start[p], 0), hi = min(a.group_start[p + 1], a.B);
      const int pl = max(a.prefix_lens[p], 0);
      for (int s = lo; s < hi; ++s) qrow[s] = pl;
    }
    __syncthreads();
  }
  for (int base = 0; base < a.B; base += 64) {
    const int s = base + lane;
    int n = 0;
    if (s < a.B) {
      int L = a.context_lens[s];
      L = L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
      lens[s] = L;
      if (qrow != nullptr && !starts) qrow[s] = a.q_start[s];
      n = L > 0 ? (visit_len(a, L, starts ? min(qrow[s], L) : 0) + kChunk - 1) / kChunk + a.seg_cost : 0;
    }
    const int inc = wave_inclusive_sum(n);
    if (s < a.B) cum[s + 1] = carry + inc;
    carry += __builtin_amdgcn_readlane(inc, 63);
  }
  if (lane == 0) cum[0] = 0;
  __syncthreads();
  const int C = carry;
  const int S = max(a.min_slice, (C + a.nslices - 1) / a.nslices);
  const int neff = max(1, (C + S - 1) / S);
  if (blockIdx.x == 0) {
    if (lane == 0) {
      a.meta[0] = S;
      a.meta[1] = neff;
    }
    for (int s = lane; s <= a.B; s += 64) a.meta[2 + s] = cum[s];
  }
  if (k >= neff) return false;
  sl.k = k;
  sl.S = S;
  sl.neff = neff;
  sl.c0 = k * S;
  sl.c1 = min(C, sl.c0 + S);
  sl.last = k == neff - 1;
  // first s that does not lie wholly before c0; an empty sequence at c0
  // belongs to this slice (binary search over a monotone predicate)
  int lo = 0, hi = a.B;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int e = cum[mid + 1];
    const bool before = e < sl.c0 || (e == sl.c0 && e > cum[mid]);
    if (before) lo = mid + 1; else hi = mid;
  }
  sl.s_first = uniform(lo);
  return true;
}

// Does sequence s (chunks [cs, ce)) lie beyond this slice?  An empty
// sequence at c1 belongs to the next slice, except at the very end.
__device__ __forceinline__ bool past_slice(const Slice& sl, int cs, int ce) {
  return cs > sl.c1 || (cs == sl.c1 && (ce > cs || !sl.last));
}

// The piece of one sequence a slice covers (wave-uniform values); s == -1
// means none.  Positions are those the walk visits (visit_len): they are the
// real ones, except past the sink chunks of a windowed sequence, where the
// real position is the visited one plus `shift`.
struct Segment {
  int s;
  int cs, ce;        // the range of the sequence's chunks on the line (after its charge)
  int tok0, tok_end; // visited positions of the piece
  int nchunks;
  int shift;         // visit_shift of the sequence (0 when its walk skips nothing)
};

// First sequence at or after s_from that is not empty and has chunks in the
// slice.  starts: each sequence's first attended position (the suffix pass of
// shared prefixes), or null.
__device__ __forceinline__ Segment next_segment(const DecodeArgs& a, const Slice& sl, const int* cum,
                                                const int* lens, int s_from, const int* starts = nullptr) {
  Segment g;
  g.s = -1;
  g.cs = g.ce = g.tok0 = g.tok_end = g.nchunks = g.shift = 0;
  for (int s = s_from; s < a.B; ++s) {
    const int L = lens[s];
    const int ce = cum[s + 1];
    if (L == 0) {
      if (past_slice(sl, cum[s], ce)) break;
      continue;
    }
    const int Lv = visit_len(a, L, starts != nullptr ? min(starts[s], L) : 0);
    const int cs = ce - (Lv + kChunk - 1) / kChunk;  // the charge lies before cs
    if (cs >= sl.c1) break;
    g.s = uniform(s);
    g.cs = uniform(cs);
    g.ce = uniform(ce);
    g.tok0 = (max(sl.c0, cs) - cs) * kChunk;
    g.tok_end = min((min(sl.c1, ce) - cs) * kChunk, Lv);
    g.nchunks = (g.tok_end - g.tok0 + kChunk - 1) / kChunk;
    g.shift = uniform(L - Lv);
    break;
  }
  return g;
}

// Pieces sequence s is cut into, and whether this slice's piece is the whole.
__device__ __forceinline__ bool whole_sequence(const Slice& sl, int cs, int ce) {
  return cs / sl.S == (ce - 1) / sl.S;
}

// Block ids of a segment, held in one register as a ring of 64 slots: block
// j of the segment (counted from its first block) sits in lane j % 64.  The
// ring holds the blocks of the next kIdAhead + 1 chunks; each step requests
// one more chunk's ids (an unconditional load whose lanes that do not take
// part re-read a valid entry), and a request is merged two steps after it
// was issued, so a merge never waits on a table read newer than the chunk
// loads it is followed by.
//
// Windowed sequences (WIN): the segment's blocks are those of its visited
// positions, and block j of the segment is table entry j, or j + gap from
// block `split` of the segment on (the window chunks after the sink chunks).
template <int BS, bool WIN = false>
struct IdRing {
  static constexpr int NB = kChunk / BS;  // blocks per chunk
  static_assert((kIdAhead + 3) * NB <= 64, "ring too small for the lookahead");
  const int32_t* row;  // block table row of the sequence, from the segment's first block
  int nblk;            // blocks in the segment
  int split, gap;      // WIN: segment blocks from `split` on are `gap` entries further on
  int ids;             // the ring
  int pending0;        // ids of chunk `next`, not merged yet
  int pending1;        // ids of chunk `next + 1`
  int next;

  __device__ __forceinline__ int entry(int j) const {
    if constexpr (WIN) return row[j + (j >= split ? gap : 0)];
    return row[j];
  }
  __device__ __forceinline__ int fetch(int chunk) const {
    const int lane = __lane_id();
    const int slot0 = (chunk * NB) & 63;
    const int j = chunk * NB + ((lane - slot0) & 63);
    return entry(j < nblk ? j : nblk - 1);
  }
  __device__ __forceinline__ void start(const int32_t* table_row, int blocks, int split_block = 0,
                                        int gap_blocks = 0) {
    row = table_row;
    nblk = blocks;
    split = split_block;
    gap = gap_blocks;
    const int lane = __lane_id();
    ids = entry(lane < nblk ? lane : nblk - 1);  // chunks 0 .. 64/NB - 1
    next = kIdAhead + 1;
    pending0 = fetch(next);
    pending1 = fetch(next + 1);
  }
  // merge the oldest pending chunk's ids, then request one more
  __device__ __forceinline__ void advance() {
    const int lane = __lane_id();
    const int slot0 = (next * NB) & 63;
    if (((lane - slot0) & 63) < NB) ids = pending0;
    pending0 = pending1;
    pending1 = fetch(next + 2);
    ++next;
  }
  // id of block i (< NB) of chunk c; valid for chunks within the lookahead
  __device__ __forceinline__ int id(int c, int i) const {
    return __builtin_amdgcn_readlane(ids, (c * NB + i) & 63);
  }
};

// Store n consecutive outputs of output row `orow` (the sequence for decode,
// the query token otherwise), query head `head`, starting at d0.
__device__ __forceinline__ void store_out(const DecodeArgs& a, int orow, int head, int D, int d0,
                                          const float* v, int n) {
  const int64_t base = ((int64_t)orow * a.Hkv * a.G + head) * D + d0;
  if (a.out_dtype == 0) {
    float* o = reinterpret_cast<float*>(a.out) + base;
    for (int i = 0; i < n; i += 4) *reinterpret_cast<f32x4*>(o + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
  } else {
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + base;
    for (int i = 0; i < n; i += 4) {
      uint32_t w0, w1;
      if (a.out_dtype == 2) {
        w0 = f32_to_bf16_rne(v[i]) | ((uint32_t)f32_to_bf16_rne(v[i + 1]) << 16);
        w1 = f32_to_bf16_rne(v[i + 2]) | ((uint32_t)f32_to_bf16_rne(v[i + 3]) << 16);
      } else {
        w0 = f32_to_f16_rne(v[i]) | ((uint32_t)f32_to_f16_rne(v[i + 1]) << 16);
        w1 = f32_to_f16_rne(v[i + 2]) | ((uint32_t)f32_to_f16_rne(v[i + 3]) << 16);
      }
      *reinterpret_cast<i32x2*>(o + i) = i32x2{(int)w0, (int)w1};
    }
  }
}

// workspace row of the partial of sequence s from slice k, for its query j
// and query head `head`
__device__ __forceinline__ int64_t part_row(const DecodeArgs& a, int k, int s, int j, int head) {
  return ((int64_t)(k + s) * a.nq + j) * a.Hkv * a.G + head;
}

__device__ __forceinline__ void store_partial(const DecodeArgs& a, int64_t row, int D, int d0,
                                              const float* v, int n) {
  float* o = a.part_acc + row * D + d0;
  for (int i = 0; i < n; i += 4) *reinterpret_cast<f32x4*>(o + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
}

__device__ __forceinline__ void store_ml(const DecodeArgs& a, int64_t row, float m, float l) {
  *reinterpret_cast<f32x2*>(a.part_ml + 2 * row) = f32x2{m, l};
}

}  // namespace pa
