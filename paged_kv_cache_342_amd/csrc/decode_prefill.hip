// Several queries per sequence over a 16-bit cache when a sequence's
// (query, head) columns are many (chunked prefill: 64 queries x 4 heads =
// 256 columns per KV head): 32 x 32 matrix tiles, with the K/V chunks and
// the query rows shared by a workgroup through LDS and fetched by the LDS
// DMA (global_load_lds, 16 bytes a lane, 1 KiB an instruction).
//
// A workgroup of kPrefillWaves waves (two per SIMD) takes one slice of the
// chunk line (decode_common.h), one KV head and 256 columns, 32 per wave
// (column c of wave w is column 256 * group + 32 * w + c; its query is
// column / G, its head column % G).
//   - At a sequence's start each wave sends its 32 query rows to LDS.
//   - K and V rows of each 32-position chunk go from HBM into one of
//     kStages LDS stages, two per even step, two and three steps before K
//     is used.  Every even step waits on the vector memory counter for all
//     of the wave's requests, then a barrier makes the two chunks visible to
//     every wave; odd steps neither wait nor synchronise.  Block ids come
//     through scalar loads, which that counter does not see.  Rows keep their natural
//     layout with the 16-byte pieces of each row permuted (an XOR of the
//     piece index with a function of the row), so that the operand reads
//     below hit every bank once.
//   - QK: S^T[32 positions x 32 columns] += K[32 x 16 d] . Q^T[16 d x 32]
//     over the D / 16 slices of d (v_mfma_f32_32x32x16), both operands read
//     with ds_read_b128.
//   - Softmax per column in fp32, log2 domain: each lane holds 16 positions
//     of one column, the other 16 sit in lane ^ 32.
//   - PV: O^T[D x 32 columns] += V^T[32 d x 16 positions] . P^T, where the
//     16 position slots of each product are the 8 positions each lane
//     already holds per half (so P needs no lane exchange); the V^T operand
//     comes from the row-major V rows through the transposing LDS read
//     (ds_read_b64_tr_b16: within 16 lanes, lane i receives element i % 4
//     of the 8 bytes lanes 4 e + i / 4 point at, e = 0..3).  P is split into
//     two bf16 terms for bf16 (about 16 bits of each weight), one fp16 term
//     for fp16.
//   - The products of chunk i run beside the softmax arithmetic of chunk
//     i - 1, in an instruction order written out in the code.
// The query j of n a column belongs to sees positions up to L - n + j.
// Segments, partial results and the merge are those of the other decode
// kernels (partial rows [slice + sequence, query, head]).
#include "decode_mfma_kernel.h"

namespace pa {

constexpr int kPrefillWaves = 8;    // waves per workgroup (two per SIMD), one 32-column tile each
constexpr int kPrefillCols = 32 * kPrefillWaves;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const int32_t const_i32;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

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

// max and sum of x over lanes l and l ^ 32, exchanged without a trip
// through LDS (the swap leaves x of both lanes in the two results, and the
// order does not matter to either)
__device__ __forceinline__ float half_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 bytes a lane from src into LDS at lds + 16 * lane (lds uniform).  The
// instruction is issued from asm so the compiler, which would otherwise wait
// for every such load before any LDS read, leaves the waits to the kernel;
// M0 (the LDS base of the instruction) is restored after it.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// wait until at most n vector memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// the same for n = per * x, x = min(later, MAX) known only at run time
template <int PER, int MAX>
__device__ __forceinline__ void wait_vm_groups(int later) {
  if constexpr (MAX == 0) {
    wait_vm<0>();
  } else {
    if (later >= MAX)
      wait_vm<PER * MAX>();
    else
      wait_vm_groups<PER, MAX - 1>(later);
  }
}

// LDS layout of a chunk's rows (K or V): row r of kChunk, 16-byte piece q of
// PR at slot r * PR + (q ^ swz(r)).  K rows are read 16 positions at a time
// at one piece (the swizzle spreads them over all banks); V rows four
// positions x four pieces at a time by the transposing read.
template <int PR>
__device__ __forceinline__ int swz_k(int r) {
  return PR == 16 ? r % 16 : (r / 2) % 8;
}
template <int PR>
__device__ __forceinline__ int swz_v(int r) {
  return PR == 16 ? 4 * (r % 4) : 4 * ((r / 2) % 2);
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
  constexpr int PR = RB / 16;                 // 16-byte pieces per row
  constexpr int kRowsPerDma = 64 / PR;        // rows one DMA instruction (64 lanes x 16 B) carries
  constexpr int kDmaPerTensor = kChunk / kRowsPerDma;
  constexpr int kDmaPerWave = 2 * kDmaPerTensor / kPrefillWaves;
  static_assert(kDmaPerWave * kPrefillWaves == 2 * kDmaPerTensor && kRowsPerDma <= BS, "DMA split");
  constexpr int kTensorBytes = kChunk * RB;   // a chunk's K (or V) rows; also a wave's 32 query rows
  constexpr int kStageBytes = 2 * kTensorBytes;  // K rows, then V rows
  constexpr int kStages = 5;

  constexpr int kScan = kScanPrefill;
  __shared__ int cum[kScan + 1];
  __shared__ int lens[kScan];
  __shared__ int qrow[kScan + 1];
  __shared__ __attribute__((aligned(1024))) uint8_t stage[kStages * kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t qtile[kPrefillWaves * kTensorBytes];

  const int lane = threadIdx.x & 63;
  const int wv = uniform(threadIdx.x >> 6);
  const int j = lane & 31;   // column within the wave's tile; row of A operands
  const int g2 = lane >> 5;  // which 8 of each product's 16 k slots the lane holds
  const int Hq = a.Hkv * a.G;
  const uint32_t stride32 = (uint32_t)(a.Hkv * kChunkBytes);  // bytes per block (the launch checks it fits)
  // a table entry is read if 0 <= id < num_blocks (else block 0 stands in)
  const uint32_t id_bound = (uint32_t)min<int64_t>(a.num_blocks, (int64_t)1 << 31);

  // workgroup -> (slice, column group, KV head), the KV head fastest
  const int h = blockIdx.x % a.Hkv;
  const int rest = blockIdx.x / a.Hkv;
  const int grp = rest % a.head_tiles;
  const int k = rest / a.head_tiles;

  if (a.B > kScan) return;
  Slice sl;
  if (!slice_setup(a, cum, lens, qrow, k, sl)) return;

  // the lane's column: column kPrefillCols * grp + 32 * wv + j of the KV
  // head's (query, head) columns
  const int col = kPrefillCols * grp + 32 * wv + j;
  const int cq = col / a.G;
  const int head = h * a.G + (cq < a.nq ? col - cq * a.G : 0);

  // this wave's DMA instructions u: tensor tn (0 K, 1 V), rows
  // kRowsPerDma * n .. + kRowsPerDma - 1 of the chunk (one block, bi[u] of
  // the chunk's NB); lane offsets within the block, and within the stage
  int bi[kDmaPerWave], lds_off[kDmaPerWave], row0_of[kDmaPerWave];
  uint32_t lane_off[kDmaPerWave];
  const uint8_t* tbase[kDmaPerWave];
#pragma unroll
  for (int u = 0; u < kDmaPerWave; ++u) {
    const int gi = u * kPrefillWaves + wv;
    const int tn = gi / kDmaPerTensor, n = gi % kDmaPerTensor;
    const int row = kRowsPerDma * n + lane / PR;
    const int q = (lane % PR) ^ (tn == 0 ? swz_k<PR>(row) : swz_v<PR>(row));
    bi[u] = (kRowsPerDma * n) / BS;
    row0_of[u] = kRowsPerDma * n;
    lane_off[u] = (uint32_t)((row % BS) * RB + 16 * q);
    lds_off[u] = tn * kTensorBytes + 1024 * n;
    tbase[u] = (tn == 0 ? a.k_cache : a.v_cache) + (int64_t)h * kChunkBytes;
  }
  // operand reads (byte offsets): K row j of a stage and Q row j of the
  // wave's query rows (same layout), pieces (2 kk + g2) ^ swz_k(j); V rows
  // p0 + vr, pieces 4 E + vc at slot 4 (E ^ (swz_v / 4)) + vc
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)stage;  // LDS address of stage 0
  const uint32_t qlds = uniform((int)((uint32_t)(uintptr_t)(lds_u8*)qtile + wv * kTensorBytes));
  uint32_t koff[KS], voff[DB];
  {
    const int kx = g2 ^ swz_k<PR>(j);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) koff[kk] = (uint32_t)(j * RB + 16 * ((2 * kk) ^ kx));
    const int vr = (lane % 16) / 4;
    const int vc = 2 * ((lane / 16) % 2) + (lane % 4) / 2;
    const int vs = swz_v<PR>(vr) / 4;  // the p0 of every read is a multiple of 4
#pragma unroll
    for (int E = 0; E < DB; ++E)
      voff[E] = (uint32_t)(kTensorBytes + (4 * g2 + vr) * RB + 16 * vc + 8 * (lane % 2) + 64 * (E ^ vs));
  }

  Segment cur = next_segment(a, sl, cum, lens, sl.s_first);
  while (cur.s >= 0) {
    const int s = cur.s;
    int row0, nqs;
    query_range(a, qrow, s, lens[s], row0, nqs);
    row0 = uniform(row0);
    nqs = uniform(nqs);
    if (nqs == 0 || cur.nchunks == 0) {  // nothing to attend for this sequence here
      cur = next_segment(a, sl, cum, lens, s + 1);
      continue;
    }
    const bool live = cq < nqs;
    const int qlim = lens[s] - nqs + cq;  // last position the column's query sees

    // block ids of the segment (scalar loads) and the row read by positions
    // past its end
    const int tok0 = cur.tok0, tok_end = cur.tok_end, nchunks = cur.nchunks;
    const int blk0 = tok0 / BS;
    const int last_blk = (tok_end - 1) / BS - blk0;  // the segment's last block, counted from blk0
    const_i32* trow = (const_i32*)(a.block_tables + (int64_t)s * a.M + blk0);
    // a table entry as read (checked when used, so the scalar load of the
    // next step's entries is not waited for where it is issued)
    auto block_entry = [&](int jb) { return trow[min(jb, last_blk)]; };
    auto checked = [&](int x) { return (uint32_t)x < id_bound ? x : 0; };
    const int last_id = checked(block_entry(last_blk));
    const uint32_t last_row_off = (uint32_t)((tok_end - 1) % BS) * RB;

    // DMA of chunk c (< nchunks) into its stage: every wave issues
    // kDmaPerWave instructions; past the segment's last position a lane
    // re-reads its last row
    auto dma = [&](int c, const int* ids) {
      const int ctok = tok0 + kChunk * c;
      const uint32_t st = lds0 + (c % kStages) * kStageBytes;
#pragma unroll
      for (int u = 0; u < kDmaPerWave; ++u) {
        const int r0 = ctok + row0_of[u];  // the instruction's first position
        const uint8_t* src;
        const int id = checked(ids[u]);
        if (r0 + kRowsPerDma <= tok_end) {
          src = tbase[u] + (uint64_t)(uint32_t)id * stride32 + lane_off[u];
        } else {
          const bool ok = r0 + lane / PR < tok_end;
          const uint32_t off = ok ? lane_off[u] : last_row_off + (lane_off[u] % RB);
          src = tbase[u] + (uint64_t)(uint32_t)(ok ? id : last_id) * stride32 + off;
        }
        dma16(src, (uint32_t)uniform((int)(st + lds_off[u])));
      }
    };
    auto chunk_ids = [&](int c, int* ids) {
#pragma unroll
      for (int u = 0; u < kDmaPerWave; ++u) ids[u] = block_entry(c * NB + bi[u]);
    };

    float m = -INFINITY, l = 0.f;
    f32x16 acc[DB];
#pragma unroll
    for (int e = 0; e < DB; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[e][r] = 0.f;

    // S^T[pos][col] of chunk c; lane (j, g2) register r holds position
    // 8 (r / 4) + 4 g2 + r % 4
    auto qk = [&](int c, f32x16& S) {
      const uint32_t sb = uniform(lds0 + (c % kStages) * kStageBytes);
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const i32x4 kop = *(lds_i32x4*)(uintptr_t)(sb + koff[kk]);
        const i32x4 qop = *(lds_i32x4*)(uintptr_t)(qlds + koff[kk]);
        S = mfma32x32<CT>(kop, qop, S);
      }
    };
    // online softmax of chunk c's scores (in place: sc holds S^T of the
    // chunk and leaves with the masked scores, still unscaled: the weights
    // apply the scale, which the launch guarantees is > 0, so the largest
    // scaled score is the scaled largest score)
    auto scores = [&](int c, f32x16& sc) {
      // the lane's slot r is seen if 8 (r / 4) + r % 4 < lim
      const int lim = min(tok_end, qlim + 1) - (tok0 + kChunk * c) - 4 * g2;
      if (wave_any(lim < 28)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = 8 * (r >> 2) + (r & 3) < lim ? sc[r] : -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      mx *= a.qk_scale_log2;
      // both lanes of a column hold the same m; it only moves when a score
      // passes it by more than the threshold
      if (wave_any(mx > m + kRescaleThreshold)) {
        const float mn = fmaxf(m, half_pair_max(mx));
        const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
#pragma unroll
        for (int e = 0; e < DB; ++e) acc[e] *= alpha;
        l *= alpha;
        m = mn;
      }
    };
    // weights of slots 2 e, 2 e + 1 of product t (the lane's score
    // registers 8 t + 2 e, + 1) as a 16-bit pair (hi) and the pair of what
    // rounding left (lo); nmu is minus the running maximum made finite (a
    // column that has seen nothing yet keeps m = -inf: its scores are all
    // -inf and their weights 0)
    auto weight_pair = [&](const f32x16& sc, float nmu, int t, int e, i32x4& phi, i32x4& plo) {
      const float qs = a.qk_scale_log2;
      const float q0 = fast_exp2(fmaf(sc[8 * t + 2 * e], qs, nmu));
      const float q1 = fast_exp2(fmaf(sc[8 * t + 2 * e + 1], qs, nmu));
      l += q0 + q1;
      if constexpr (kBf16) {
        uint32_t hi = pack_bf16(q0, q1);
        // opaque to the optimiser, which would otherwise convert q0 a second
        // time for the low half instead of shifting the pair
        asm("" : "+v"(hi));
        phi[e] = (int)hi;
        plo[e] = (int)pack_bf16(q0 - __uint_as_float(hi << 16), q1 - __uint_as_float(hi & 0xFFFF0000u));
      } else {
        phi[e] = (int)pack_f16(q0, q1);
        plo[e] = 0;
      }
    };
    // the V^T operand of d block E, product t of the chunk at stage base sb:
    // slots 0..3 are positions 16 t + 4 g2 .. + 3, slots 4..7 positions
    // 16 t + 8 + 4 g2 .. + 3; rows d = 32 E + j
    auto v_operand = [&](uint32_t sb, int t, int E) {
      const uint32_t ve = sb + voff[E] + (16 * t) * RB;
      const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)ve);
      const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(ve + 8 * RB));
      return i32x4{__builtin_bit_cast(int, __builtin_shufflevector(v0, v0, 0, 1)),
                   __builtin_bit_cast(int, __builtin_shufflevector(v0, v0, 2, 3)),
                   __builtin_bit_cast(int, __builtin_shufflevector(v1, v1, 0, 1)),
                   __builtin_bit_cast(int, __builtin_shufflevector(v1, v1, 2, 3))};
    };
    auto k_operand = [&](uint32_t sb, int kk) { return *(lds_i32x4*)(uintptr_t)(sb + koff[kk]); };
    auto q_operand = [&](int kk) { return *(lds_i32x4*)(uintptr_t)(qlds + koff[kk]); };

    // Softmax and PV of chunk c whose S^T is in sc; with with_qk, S of chunk
    // cn as well.  The instruction order is written out (each group fenced
    // with a scheduling barrier): operand reads run two products ahead of
    // their products, and the weights of the chunk fill the time the matrix
    // unit spends on the products -- S of chunk cn beside the product-0
    // weights, then product 0 of PV beside the product-1 weights, then
    // product 1.
    auto softmax_pv = [&](int c, f32x16& sc, auto with_qk, int cn, f32x16& s_new) {
      constexpr bool kQk = decltype(with_qk)::value;
      scores(c, sc);
      const float nmu = -fmaxf(m, -__FLT_MAX__);
      const uint32_t sbv = uniform(lds0 + (c % kStages) * kStageBytes);
      i32x4 phi0, plo0, phi1, plo1;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kQk) {
        const uint32_t sbk = uniform(lds0 + (cn % kStages) * kStageBytes);
        i32x4 ko[KS], qo[KS];
        ko[0] = k_operand(sbk, 0); qo[0] = q_operand(0);
        ko[1] = k_operand(sbk, 1); qo[1] = q_operand(1);
#pragma unroll
        for (int r = 0; r < 16; ++r) s_new[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          __builtin_amdgcn_sched_barrier(0);
          if (kk + 2 < KS) {
            ko[kk + 2] = k_operand(sbk, kk + 2);
            qo[kk + 2] = q_operand(kk + 2);
          }
          s_new = mfma32x32<CT>(ko[kk], qo[kk], s_new);
          __builtin_amdgcn_sched_barrier(0);
          if ((kk * 4) % KS == 0) weight_pair(sc, nmu, 0, kk * 4 / KS, phi0, plo0);  // the four pairs over the KS products
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) weight_pair(sc, nmu, 0, e, phi0, plo0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // product 0 of PV beside the product-1 weights
      {
        i32x4 vo[DB];
        vo[0] = v_operand(sbv, 0, 0);
        vo[1] = v_operand(sbv, 0, 1);
#pragma unroll
        for (int E = 0; E < DB; ++E) {
          __builtin_amdgcn_sched_barrier(0);
          if (E + 2 < DB) vo[E + 2] = v_operand(sbv, 0, E + 2);
          acc[E] = mfma32x32<CT>(vo[E], phi0, acc[E]);
          if constexpr (kBf16) acc[E] = mfma32x32<CT>(vo[E], plo0, acc[E]);
          __builtin_amdgcn_sched_barrier(0);
          weight_pair(sc, nmu, 1, E, phi1, plo1);
        }
#pragma unroll
        for (int e = DB; e < 4; ++e) weight_pair(sc, nmu, 1, e, phi1, plo1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // product 1 of PV
      {
        i32x4 vo[DB];
        vo[0] = v_operand(sbv, 1, 0);
        vo[1] = v_operand(sbv, 1, 1);
#pragma unroll
        for (int E = 0; E < DB; ++E) {
          __builtin_amdgcn_sched_barrier(0);
          if (E + 2 < DB) vo[E + 2] = v_operand(sbv, 1, E + 2);
          acc[E] = mfma32x32<CT>(vo[E], phi1, acc[E]);
          if constexpr (kBf16) acc[E] = mfma32x32<CT>(vo[E], plo1, acc[E]);
        }
      }
    };

    // The wave's query rows go to LDS by DMA (a row per column, the layout
    // of the K rows; a column past the queries reads the first query row).
    // Then step i computes S of chunk i beside the softmax and PV of chunk
    // i - 1 (it reads the stages of chunks i - 1 and i), and every chunk's
    // DMA is waited for by an even step no later than its own, so the next
    // segment starts with nothing outstanding.
    __builtin_amdgcn_s_barrier();  // every wave is done with the stages of the last segment
#pragma unroll
    for (int n = 0; n < kChunk / kRowsPerDma; ++n) {
      const int row = kRowsPerDma * n + lane / PR;
      const int qcol = kPrefillCols * grp + 32 * wv + row;
      const int qq = qcol / a.G;
      const bool qlive = qq < nqs;
      const int64_t qr = row0 + (qlive ? qq : 0);
      const int qh = qlive ? h * a.G + (qcol - qq * a.G) : h * a.G;
      const int piece = (lane % PR) ^ swz_k<PR>(row);
      dma16(reinterpret_cast<const uint8_t*>(a.q) + (qr * Hq + qh) * RB + 16 * piece, qlds + 1024 * n);
    }
    // block ids of the first four chunks (their scalar loads issued
    // together), then the DMA of the first two
    int ids0[2][kDmaPerWave], idn[2][kDmaPerWave];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      chunk_ids(c, ids0[c]);
      chunk_ids(c + 2, idn[c]);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
      if (c < nchunks) dma(c, ids0[c]);
    f32x16 sa, sb;
    // Even steps wait for every DMA the wave issued (chunks i and i + 1,
    // requested at step i - 2), and the barrier makes all waves' rows
    // visible and ends every read of steps i - 2 and i - 1; they then send
    // chunks i + 2 and i + 3 into the stages chunks i - 3 and i - 2 left.
    // Odd steps need neither: their chunk landed before the last barrier.
    // They load the block ids the next even step sends (idn is read at the
    // start of an even step and loaded again at the odd step after it, so
    // no loaded value is copied).
    auto step = [&](int i, auto even, auto first, f32x16& s_prev, f32x16& s_new) {
      if constexpr (decltype(even)::value) {
        wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        if (i + 2 < nchunks) dma(i + 2, idn[0]);
        if (i + 3 < nchunks) dma(i + 3, idn[1]);
      } else {
        chunk_ids(i + 3, idn[0]);  // scalar loads, used by step i + 1
        chunk_ids(i + 4, idn[1]);
      }
      if constexpr (decltype(first)::value)
        qk(0, s_new);
      else
        softmax_pv(i - 1, s_prev, std::true_type(), i, s_new);
    };
    step(0, std::true_type(), std::true_type(), sb, sa);
    int i = 1;
    for (; i + 1 < nchunks; i += 2) {
      step(i, std::false_type(), std::false_type(), sa, sb);
      step(i + 1, std::true_type(), std::false_type(), sb, sa);
    }
    if (i < nchunks) {  // i = nchunks - 1: S of chunk i - 1 in sa
      step(i, std::false_type(), std::false_type(), sa, sb);
      softmax_pv(i, sb, std::false_type(), 0, sa);
    } else {            // i = nchunks: S of chunk i - 1 in sa
      softmax_pv(i - 1, sa, std::false_type(), 0, sb);
    }

    // ---- epilogue: lane (j, g2) holds d = 32 e + 8 R + 4 g2 + 0..3 of its column
    const float lt = half_pair_sum(l);
    if (live) {
      const bool whole = whole_sequence(sl, cur.cs, cur.ce);
      const float f = whole ? 1.f / lt : 1.f;
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
      if (!whole && g2 == 0) store_ml(a, prow, m, lt);
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
