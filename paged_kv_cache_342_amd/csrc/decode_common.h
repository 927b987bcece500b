// Shared definitions of the paged decode kernels: launch arguments, work
// items and the epilogue stores.
//
// Work decomposition.  A sequence of L tokens is cut into partitions of
// `part_tokens` consecutive positions (split-K over the context).  One
// wavefront handles one (sequence, partition, KV head[, head tile]) item and
// produces, for each query head of that KV head, the running maximum m (log2
// domain), the sum l of 2^(score - m) and the unnormalised accumulator
// acc = sum 2^(score - m) * V.  A sequence that fits in one partition is
// normalised and written to `out` directly; otherwise the partials go to the
// workspace and the reduce kernel merges them:
//   M = max_p m_p,  out = v_scale * sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
#pragma once

#include "pa_device.h"

namespace pa {

struct DecodeArgs {
  void* out;
  const void* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* work;  // [0] = item count; items as (seq, partition) int pairs from work + 2
  float* part_acc;      // [B, Hq, nparts, D]
  float* part_ml;       // [B, Hq, nparts, 2] = (m, l)
  int64_t num_blocks;
  int32_t B, Hkv, G, M;  // M = max_blocks_per_seq
  int32_t max_ctx;       // effective bound: min(max_context_len, M * bs)
  int32_t nparts;        // partitions per sequence the workspace holds
  int32_t part_tokens;
  int32_t head_tiles;    // query-head tiles of 16 per KV head (MFMA kernel), 1 otherwise
  int32_t dense;         // 1: item i is (sequence i, partition 0) and there are B items
  int32_t out_dtype;     // 0 f32, 1 f16, 2 bf16
  float qk_scale_log2;   // scale * k_scale * log2(e)
  float v_scale;
};

struct Item {
  int s, p, h, ht;
  int L;        // clamped context length
  int nparts;   // partitions of this sequence (>= 1)
  int tok0;     // first position of the partition
  int tok_end;  // one past its last position
};

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int item_count(const DecodeArgs& a) {
  return a.dense ? a.B : uniform(a.work[0]);
}

// context length of sequence s, clamped to [0, max_ctx]
__device__ __forceinline__ int context_len(const DecodeArgs& a, int s) {
  const int L = uniform(a.context_lens[s]);
  return L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
}

__device__ __forceinline__ Item item_at(const DecodeArgs& a, int flat) {
  const int per = a.Hkv * a.head_tiles;
  const int it = flat / per;
  const int rem = flat - it * per;
  Item t;
  t.h = rem / a.head_tiles;
  t.ht = rem - t.h * a.head_tiles;
  if (a.dense) {
    t.s = it;
    t.p = 0;
  } else {
    t.s = uniform(a.work[2 + 2 * it]);
    t.p = uniform(a.work[3 + 2 * it]);
  }
  const int L = context_len(a, t.s);
  t.L = L;
  t.nparts = L > 0 ? (L + a.part_tokens - 1) / a.part_tokens : 1;
  t.tok0 = t.p * a.part_tokens;
  int e = t.tok0 + a.part_tokens;
  t.tok_end = e < L ? e : L;
  return t;
}

// The partition's block ids, one per lane (lane j holds logical block
// tok0 / bs + j); ids outside the pool read as block 0 so no access leaves
// the pool.  A partition spans at most 64 blocks.
__device__ __forceinline__ int load_block_ids(const DecodeArgs& a, const Item& t, int bs) {
  const int lane = __lane_id();
  const int blk0 = t.tok0 / bs;
  const int nblk = (t.tok_end + bs - 1) / bs - blk0;
  int id = 0;
  if (lane < nblk) {
    id = a.block_tables[(int64_t)t.s * a.M + blk0 + lane];
    if (id < 0 || (int64_t)id >= a.num_blocks) id = 0;
  }
  return id;
}

// Byte offset, from the start of a KV head's first chunk, of the partition's
// last position (tok_end - 1), which always holds written data.  Lanes whose
// position lies past the end load this row instead of predicating the load:
// every load stays unconditional (so the compiler can keep several chunks in
// flight and wait on them one at a time), and the masked lanes' scores are
// set to -inf, so the row they read adds exactly zero.
__device__ __forceinline__ int64_t last_row_offset(const Item& t, int ids, int bs, int64_t blk_stride,
                                                   int row_bytes) {
  const int last = t.tok_end - 1;
  const int id = __builtin_amdgcn_readlane(ids, last / bs - t.tok0 / bs);
  return (int64_t)id * blk_stride + (int64_t)(last % bs) * row_bytes;
}

// Store n consecutive outputs of (s, head) starting at d0.
__device__ __forceinline__ void store_out(const DecodeArgs& a, int s, int head, int D, int d0,
                                          const float* v, int n) {
  const int64_t base = ((int64_t)s * a.Hkv * a.G + head) * D + d0;
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

__device__ __forceinline__ int64_t part_index(const DecodeArgs& a, int s, int head, int p) {
  return ((int64_t)s * a.Hkv * a.G + head) * a.nparts + p;
}

__device__ __forceinline__ void store_partial(const DecodeArgs& a, int s, int head, int p, int D,
                                              int d0, const float* v, int n) {
  float* o = a.part_acc + part_index(a, s, head, p) * D + d0;
  for (int i = 0; i < n; i += 4) *reinterpret_cast<f32x4*>(o + i) = f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
}

__device__ __forceinline__ void store_ml(const DecodeArgs& a, int s, int head, int p, float m, float l) {
  *reinterpret_cast<f32x2*>(a.part_ml + 2 * part_index(a, s, head, p)) = f32x2{m, l};
}

}  // namespace pa
