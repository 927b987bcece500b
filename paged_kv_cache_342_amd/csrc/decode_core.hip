// Host side of pa_decode (slice count, workspace layout, kernel choice,
// launches) and the kernel that merges the partial results of sequences cut
// by slice boundaries.
#include <climits>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "decode_common.h"
#include "pa_internal.h"

namespace pa {

bool launch_decode_mfma(const DecodeArgs& a, int ct, int qt, int head_dim, int bs, bool multi_query,
                        int tiles_per_wave, int waves_per_group, dim3 grid, hipStream_t stream,
                        const LaunchEvents& ev);
bool mfma_kernel_built(int ct, int qt, int head_dim, int bs, bool multi_query, bool row_scales);
bool launch_decode_valu(const DecodeArgs& a, int ct, int qt, int head_dim, int bs, int group,
                        dim3 grid, hipStream_t stream, const LaunchEvents& ev);
bool valu_supports(int ct, int qt, int head_dim, int bs, int group);
bool launch_prefill(const DecodeArgs& a, int ct, int qt, int head_dim, int bs, dim3 grid, hipStream_t stream,
                    const LaunchEvents& ev);
// waves per workgroup of the prefill kernel (decode_prefill.hip): 256 columns
// in 32-column tiles, two waves per SIMD
constexpr int kPrefillWavesHost = 8;

// Workgroups per (KV head, sequence) -- one for decode, more when its
// queries hold more outputs than a workgroup has threads: merge the slices'
// partials of every query head of the group, in slice order, with an online
// rescale:
//   M = max_k m_k;  out = v_scale * sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k.
// Thread j handles four consecutive outputs of one query head, so all heads
// of the group (and, with several queries per sequence, all its queries) are
// merged at once, and the loads of up to kMergeUnroll pieces are issued
// before any of them is used.  Sequences that are whole in one slice were
// written by the decode kernel and are skipped here.  A piece that saw no
// position holds m = -inf and is skipped: under MQ one whose positions all
// lie past what a query sees, with a window one that lies in the gap between
// the sink and the window.  A sequence's chunks on the line start seg_cost
// after its place in the scan (meta), whatever its walk visits.
//
// STATE (the prefix pass of shared prefixes): every member of a group sees
// the whole prefix, and the merged (M, den) and num are written unnormalised
// to the member's state rows, where the suffix pass starts from them.
constexpr int kMergeUnroll = 8;

template <int D, bool MQ, bool STATE = false>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  static_assert(!STATE || MQ, "the prefix pass is a several-queries launch");
  constexpr int LPH = D / 4;  // threads per head
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int S = a.meta[0];
  const int neff = a.meta[1];
  const int ce = a.meta[3 + s];
  int L = a.context_lens[s];
  L = L < 0 ? 0 : (L > a.max_ctx ? a.max_ctx : L);
  if (L == 0) return;
  const int cs = a.meta[2 + s] + a.seg_cost;  // the sequence's chunks, after its charge
  const int kf = cs / S;
  const int kl = min((ce - 1) / S, neff - 1);
  if (kl <= kf) return;
  const int np = kl - kf + 1;
  int qrow0 = s, nqs = 1;
  if constexpr (MQ) query_range(a, a.q_start, s, L, qrow0, nqs, !STATE);
  for (int idx = blockIdx.z * blockDim.x + threadIdx.x; idx < nqs * a.G * LPH; idx += gridDim.z * blockDim.x) {
    const int jq = MQ ? idx / (a.G * LPH) : 0;
    const int rem = idx - jq * a.G * LPH;
    const int i = rem / LPH;
    const int d = 4 * (rem - i * LPH);
    const int head = h * a.G + i;
    float M = -INFINITY, den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    // pieces in batches of U, their loads issued before any is used
    auto merge = [&](auto unroll) {
      constexpr int U = decltype(unroll)::value;
      for (int p0 = 0; p0 < np; p0 += U) {
        f32x2 ml[U];
        f32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int p = min(p0 + u, np - 1);
          const int64_t row = part_row(a, kf + p, s, jq, head);
          ml[u] = *reinterpret_cast<const f32x2*>(a.part_ml + 2 * row);
          x[u] = *reinterpret_cast<const f32x4*>(a.part_acc + row * D + d);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (p0 + u < np && ml[u][0] > -INFINITY) {
            const float Mn = fmaxf(M, ml[u][0]);
            const float ca = fast_exp2(M - Mn);
            const float cb = fast_exp2(ml[u][0] - Mn);
            den = den * ca + ml[u][1] * cb;
            num = num * ca + x[u] * cb;
            M = Mn;
          }
        }
      }
    };
    // (np is the same for the whole workgroup; a batch never loads a piece twice
    // for the common counts of 2 to 4)
    if (np <= 2)
      merge(std::integral_constant<int, 2>());
    else if (np <= 4)
      merge(std::integral_constant<int, 4>());
    else
      merge(std::integral_constant<int, kMergeUnroll>());
    if constexpr (STATE) {
      const int64_t row = (int64_t)(qrow0 + jq) * a.Hkv * a.G + head;
      *reinterpret_cast<f32x4*>(a.state_acc + row * D + d) = num;
      if (d == 0) *reinterpret_cast<f32x2*>(a.state_ml + 2 * row) = f32x2{M, den};
    } else {
      const float f = a.v_scale / den;
      const float v[4] = {num[0] * f, num[1] * f, num[2] * f, num[3] * f};
      store_out(a, qrow0 + jq, head, D, d, v, 4);
    }
  }
}

// ---------------------------------------------------------------- host side

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = kPlanMaxCUs;
  if (dev < 64) cache[dev] = n;
  return n;
}

// compute units a launch plans with: the device's, at most kPlanMaxCUs
static int plan_cus() { return std::min(device_cu_count(), kPlanMaxCUs); }

// virtual chunks a sequence is charged on the line for its fixed costs: the
// kernel's own charge unless PA_DECODE_SEGMENT_COST gives one
static int segment_cost(int charge) {
  const char* v = std::getenv("PA_DECODE_SEGMENT_COST");
  const int n = v ? std::atoi(v) : -1;
  return n >= 0 && n <= 64 ? n : charge;
}

// The charge per sequence: 2 chunks, and 3 for fp8 caches at one wave per
// SIMD with one query per sequence, whose loop runs ~1.5 us a chunk against a
// segment's fixed costs.  Measured on the heavy-tailed fp8 batch (A/B on one
// machine), 3 against 2: block size 16 kernel 95.0 -> 92.7 us, block size 32
// 92.7 -> 89.8 us, with a scale per row 109.3 -> 107.8 us; 4 and 1 were
// worse, and the 16-bit lines and fp8 at two waves per SIMD were best at 2.
static int sequence_charge(int cache_dtype, bool two_waves, bool multi_query) {
  return cache_dtype == PA_FP8_E4M3 && !two_waves && !multi_query ? 3 : 2;
}

// waves the grid gives each CU: one per SIMD, or two for the kernels that
// run two per SIMD (PA_DECODE_WAVES_PER_CU overrides it, within
// [1, kMaxWavesPerCU])
static int waves_per_cu(bool two_waves) {
  const char* v = std::getenv("PA_DECODE_WAVES_PER_CU");
  const int n = v ? std::atoi(v) : 0;
  return n >= 1 && n <= kMaxWavesPerCU ? n : (two_waves ? 8 : 4);
}

DecodePlan plan_decode(int B, int Hkv, int G, int D, int bs, int max_ctx, int head_tiles, int64_t waves, int nq,
                       bool multi_query, bool two_waves, int scan_cap, int charge) {
  (void)bs;
  DecodePlan p{};
  const int64_t per = (int64_t)Hkv * head_tiles;
  p.nslices = (int)std::max<int64_t>(1, (waves + per - 1) / per);
  p.min_slice = 4;
  p.seg_cost = segment_cost(charge);
  const int64_t chunks = ((int64_t)std::max(max_ctx, 1) + kChunk - 1) / kChunk + p.seg_cost;
  // the kernel's LDS scan arrays bound the sequences of one launch
  int64_t sub = std::min<int64_t>(scan_cap > 0 ? scan_cap : scan_capacity(multi_query, two_waves), INT_MAX / chunks);
  p.sub_batch = (int)std::max<int64_t>(1, std::min<int64_t>(sub, std::max(B, 1)));
  const size_t Hq = (size_t)Hkv * G * std::max(nq, 1);  // partial rows per (slice, sequence)
  const size_t rows = (size_t)p.nslices + p.sub_batch;
  p.meta_off = 0;
  p.ml_off = align256(sizeof(int32_t) * (3 + (size_t)p.sub_batch));
  p.acc_off = p.ml_off + align256(sizeof(float) * 2 * rows * Hq);
  p.bytes = p.acc_off + align256(sizeof(float) * (size_t)D * rows * Hq);
  return p;
}

// The bound plans the most slices any launch can have (kMaxWavesPerCU waves
// on each of kPlanMaxCUs CUs, one head tile per KV head) at both
// occupancies, so it depends on the arguments alone, not on the device.
size_t decode_workspace_bound(int B, int Hkv, int G, int D, int bs, int max_ctx, int nq, bool multi_query) {
  const int64_t waves = (int64_t)kMaxWavesPerCU * kPlanMaxCUs;
  return std::max(plan_decode(B, Hkv, G, D, bs, max_ctx, 1, waves, nq, multi_query, false).bytes,
                  plan_decode(B, Hkv, G, D, bs, max_ctx, 1, waves, nq, multi_query, true).bytes);
}

// Events the next decode call records around its attention kernels
// (pa_time_next_attention_kernel); one pair per thread.
static thread_local hipEvent_t g_time_start = nullptr;
static thread_local hipEvent_t g_time_stop = nullptr;

void set_timing_events(hipEvent_t start, hipEvent_t stop) {
  g_time_start = start;
  g_time_stop = stop;
}

// Long query chunks on a 16-bit cache (PA_DECODE_MQ_SHARED, for comparisons):
// 3 = the prefill kernel, workgroups of kPrefillWaves waves with 32 x 32
// tiles (the default from kSharedWaves1 16-column tiles on); 2 = workgroups
// of kSharedWaves1 waves with one 16-column tile each at two waves per SIMD
// (16 x 64-query chunked prefill 122 us against 144 us for mode 1 and 145 us
// for mode 0); 1 = kSharedWaves waves with two tiles each at one wave per
// SIMD (also where the queries span fewer than kSharedWaves1 tiles); 0 = one
// wave per workgroup
static int mq_shared_mode() {
  const char* v = std::getenv("PA_DECODE_MQ_SHARED");
  if (v && v[0] == '0') return 0;
  if (v && v[0] == '1') return 1;
  if (v && v[0] == '2') return 2;
  return 3;
}

int decode_variant_override() {
  const char* v = std::getenv("PA_DECODE_VARIANT");
  if (!v) return 0;
  if (!std::strcmp(v, "valu")) return 1;
  if (!std::strcmp(v, "mfma")) return 2;
  return 0;
}

// The MFMA kernel is the default for every group size: even at groups 1 and 2,
// where most of its 16-column tile is padding, it issues far fewer
// instructions per chunk than the VALU/DPP kernel and measured 9-26% faster
// on both cache dtypes; the VALU/DPP kernel stays selectable.
bool decode_uses_valu(int variant, int G) {
  (void)G;
  return variant == 1;
}

static int elem_size(int dtype) { return dtype == PA_F32 ? 4 : (dtype == PA_FP8_E4M3 ? 1 : 2); }

pa_status decode_launch(const DecodeRequest& r, hipStream_t stream) {
  const bool mq = r.q_start != nullptr;  // several queries per sequence: MFMA kernel only
  const bool rs = r.k_row_scale != nullptr;  // a scale per row: MFMA kernel only
  const int nq = mq ? r.nq : 1;
  const bool win = r.window > 0;  // sinks plus a window: MFMA kernel only
  const bool valu = !mq && !rs && !win && decode_uses_valu(decode_variant_override(), r.G);
  if (valu && !valu_supports(r.cache_dtype, r.q_dtype, r.D, r.bs, r.G)) {
    set_error("pa_decode: the VALU kernel is not built for group %d, head_dim %d, block size %d",
              r.G, r.D, r.bs);
    return PA_ERR_UNSUPPORTED;
  }
  // 16-column tiles of (query, head) columns per KV head; a wave computes one,
  // or two when a sequence's queries span several (the K/V loads and the V
  // transposes are then shared)
  const int col_tiles = valu ? 1 : (int)(((int64_t)nq * r.G + 15) / 16);
  // queries spanning kSharedWaves or more tile pairs of a 16-bit cache: the
  // waves of a workgroup share each K/V chunk through LDS
  const int shared_mode = mq && !rs && (r.cache_dtype == PA_F16 || r.cache_dtype == PA_BF16) ? mq_shared_mode() : 0;
  // the prefill kernel: 256 (query, head) columns per workgroup of kPrefillWaves waves
  // (it addresses a block with a 32-bit stride, and scales its scores inside
  // the exponential, which needs a scale > 0; other scales take the
  // 16-column kernels)
  const bool prefill = shared_mode == 3 && col_tiles >= kSharedWaves1 &&
                       (int64_t)r.Hkv * r.bs * r.D * 2 <= (int64_t)UINT32_MAX && r.scale > 0.f;
  const int prefill_groups = (int)(((int64_t)nq * r.G + 255) / 256);
  const bool shared1 = shared_mode == 2 && col_tiles >= kSharedWaves1;  // one tile per wave
  const int tw = mq && col_tiles >= 2 && !shared1 && !prefill ? 2 : 1;
  // waves per (slice, KV head)
  const int tiles = prefill ? prefill_groups * kPrefillWavesHost : (col_tiles + tw - 1) / tw;
  const bool two_waves = !valu && (prefill || shared1 || mfma_two_waves(r.cache_dtype, rs, tw, r.bs, !mq));
  const int scan_cap = prefill ? kScanPrefill : scan_capacity(mq, two_waves);
  const bool shared = shared1 || (shared_mode >= 1 && tw == 2 && tiles >= kSharedWaves);
  const int group_waves = prefill ? kPrefillWavesHost : (shared1 ? kSharedWaves1 : (shared ? kSharedWaves : 1));
  const int group_tiles = (tiles + group_waves - 1) / group_waves;  // workgroups per (slice, KV head)
  const DecodePlan plan = plan_decode(r.B, r.Hkv, r.G, r.D, r.bs, r.plan_ctx, tiles,
                                      (int64_t)waves_per_cu(two_waves) * plan_cus(), nq, mq, two_waves, scan_cap,
                                      sequence_charge(r.cache_dtype, two_waves, mq));
  if (r.workspace_bytes < plan.bytes) {
    set_error("pa_decode: workspace of %zu bytes needed, %zu given", plan.bytes, r.workspace_bytes);
    return PA_ERR_WORKSPACE;
  }
  if (plan.sub_batch > scan_cap) {  // cannot happen: plan_decode caps it
    set_error("pa_decode: internal error: %d sequences per launch exceed the kernel's scan arrays", plan.sub_batch);
    return PA_ERR_HIP;
  }
  const int64_t grid_waves = (int64_t)plan.nslices * r.Hkv * tiles;
  if (grid_waves >= ((int64_t)1 << 31)) {
    set_error("pa_decode: %lld waves exceed the grid limit", (long long)grid_waves);
    return PA_ERR_UNSUPPORTED;
  }
  // Every choice that can refuse the call is made before anything is
  // enqueued (the fp8 append below writes the cache).
  if (!valu && !mfma_kernel_built(r.cache_dtype, r.q_dtype, r.D, r.bs, mq, rs)) {
    set_error("pa_decode: no kernel built for cache dtype %d, q dtype %d, head_dim %d, block size %d", r.cache_dtype,
              r.q_dtype, r.D, r.bs);
    return PA_ERR_UNSUPPORTED;
  }
  const int Hq = r.Hkv * r.G;
  // Appending: 16-bit rows are stored by the decode kernel itself; fp8 rows
  // are encoded into the cache by a scatter first.
  const bool fused_append = r.new_k != nullptr && r.cache_dtype != PA_FP8_E4M3;
  if (r.new_k != nullptr && !fused_append) {
    const pa_status st = append_last_launch(r.new_k, r.new_v, const_cast<void*>(r.k_cache),
                                            const_cast<void*>(r.v_cache), r.block_tables, r.context_lens, r.B,
                                            r.M, r.max_ctx, r.Hkv, r.D, r.bs, r.num_blocks, r.src_dtype,
                                            r.cache_dtype, r.k_scale, r.v_scale, stream);
    if (st != PA_OK) return st;
  }
  const size_t new_row = (size_t)r.Hkv * r.D * 2;
  uint8_t* ws = reinterpret_cast<uint8_t*>(r.workspace);
  DecodeArgs a{};
  a.k_cache = reinterpret_cast<const uint8_t*>(r.k_cache);
  a.v_cache = reinterpret_cast<const uint8_t*>(r.v_cache);
  a.meta = reinterpret_cast<int32_t*>(ws + plan.meta_off);
  a.part_ml = reinterpret_cast<float*>(ws + plan.ml_off);
  a.part_acc = reinterpret_cast<float*>(ws + plan.acc_off);
  a.num_blocks = r.num_blocks;
  a.Hkv = r.Hkv;
  a.G = r.G;
  a.M = r.M;
  a.max_ctx = r.max_ctx;
  a.nslices = plan.nslices;
  a.min_slice = plan.min_slice;
  a.seg_cost = plan.seg_cost;
  a.head_tiles = group_tiles;
  a.out_dtype = r.out_dtype == PA_F32 ? 0 : (r.out_dtype == PA_F16 ? 1 : 2);
  const bool fp8 = r.cache_dtype == PA_FP8_E4M3;
  a.qk_scale_log2 = r.scale * (fp8 && !rs ? r.k_scale : 1.f) * 1.4426950408889634f;
  a.v_scale = fp8 && !rs ? r.v_scale : 1.f;
  a.k_row_scale = r.k_row_scale;
  a.v_row_scale = r.v_row_scale;
  a.sink = win ? r.sink : 0;
  a.window = win ? r.window : 0;
  a.nq = nq;
  a.q_rows = mq ? r.q_rows : r.B;
  const int ct = r.cache_dtype, qt = r.q_dtype;
  const size_t out_row = (size_t)Hq * r.D * elem_size(r.out_dtype);
  const size_t q_row = (size_t)Hq * r.D * 2;
  // timing events of this call, if the caller asked for them: start on the
  // first attention kernel, stop on the last
  const hipEvent_t t_start = g_time_start, t_stop = g_time_stop;
  g_time_start = g_time_stop = nullptr;
  // batches beyond one launch's scan capacity run as consecutive launches;
  // they share the workspace, which stream order makes safe
  for (int s0 = 0; s0 < r.B; s0 += plan.sub_batch) {
    const LaunchEvents ev{s0 == 0 ? t_start : nullptr, s0 + plan.sub_batch >= r.B ? t_stop : nullptr};
    a.B = std::min(plan.sub_batch, r.B - s0);
    // decode rows follow the sequences; query rows are named by q_start
    a.out = reinterpret_cast<uint8_t*>(r.out) + (mq ? 0 : (size_t)s0 * out_row);
    a.q = reinterpret_cast<const uint8_t*>(r.q) + (mq ? 0 : (size_t)s0 * q_row);
    a.q_start = mq ? r.q_start + s0 : nullptr;
    if (!mq) a.q_rows = a.B;
    a.block_tables = r.block_tables + (int64_t)s0 * r.M;
    a.context_lens = r.context_lens + s0;
    a.new_k = fused_append ? reinterpret_cast<const uint8_t*>(r.new_k) + (size_t)s0 * new_row : nullptr;
    a.new_v = fused_append ? reinterpret_cast<const uint8_t*>(r.new_v) + (size_t)s0 * new_row : nullptr;
    const dim3 grid((unsigned)((int64_t)plan.nslices * r.Hkv * group_tiles));
    const bool ok = valu      ? launch_decode_valu(a, ct, qt, r.D, r.bs, r.G, grid, stream, ev)
                    : prefill ? launch_prefill(a, ct, qt, r.D, r.bs, grid, stream, ev)
                              : launch_decode_mfma(a, ct, qt, r.D, r.bs, mq, tw, group_waves, grid, stream, ev);
    if (!ok) {
      set_error("pa_decode: no kernel built for cache dtype %d, q dtype %d, head_dim %d, block size %d, group %d (%s)",
                ct, qt, r.D, r.bs, r.G, valu ? "valu" : "mfma");
      return PA_ERR_UNSUPPORTED;
    }
    if (plan.nslices > 1) {
      const int64_t threads = (int64_t)nq * r.G * (r.D / 4);
      const dim3 mgrid(r.Hkv, a.B, (unsigned)std::min<int64_t>(65535, (threads + 255) / 256));
      const dim3 mblock(threads >= 256 ? 256 : (unsigned)(((threads + 63) / 64) * 64));
      if (r.D == 64 && !mq)
        hipLaunchKernelGGL((decode_merge_kernel<64, false>), mgrid, mblock, 0, stream, a);
      else if (!mq)
        hipLaunchKernelGGL((decode_merge_kernel<128, false>), mgrid, mblock, 0, stream, a);
      else if (r.D == 64)
        hipLaunchKernelGGL((decode_merge_kernel<64, true>), mgrid, mblock, 0, stream, a);
      else
        hipLaunchKernelGGL((decode_merge_kernel<128, true>), mgrid, mblock, 0, stream, a);
    }
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
      set_error("pa_decode: launch failed: %s", hipGetErrorString(err));
      return PA_ERR_HIP;
    }
  }
  return PA_OK;
}

// ------------------------------------------------- shared prefixes (cascade)

bool launch_cascade_pass(bool prefix, const DecodeArgs& a, int ct, int qt, int head_dim, int bs, dim3 grid,
                         hipStream_t stream, const LaunchEvents& ev);

// 16-column tiles of a group's (member, head) columns; a prefix-pass wave
// computes two
static int prefix_tiles(int max_group, int G) {
  const int64_t col_tiles = ((int64_t)max_group * G + 15) / 16;
  return (int)((col_tiles + 1) / 2);
}

// Workspace of one cascade call: [prefix plan][suffix plan][state m, l][state acc]
struct CascadeLayout {
  DecodePlan pre, suf;
  size_t suf_off, state_ml_off, state_acc_off, bytes;
};

static CascadeLayout cascade_layout(int B, int P, int max_group, int Hkv, int G, int D, int bs, int max_ctx,
                                    int64_t waves, int pre_tiles) {
  CascadeLayout c{};
  c.pre = plan_decode(P, Hkv, G, D, bs, max_ctx, pre_tiles, waves, max_group, true, false);
  // the suffix pass keeps first positions in LDS: the several-queries scan capacity
  c.suf = plan_decode(B, Hkv, G, D, bs, max_ctx, 1, waves, 1, true, false);
  const size_t Hq = (size_t)Hkv * G;
  c.suf_off = align256(c.pre.bytes);
  c.state_ml_off = c.suf_off + align256(c.suf.bytes);
  c.state_acc_off = c.state_ml_off + align256(sizeof(float) * 2 * (size_t)B * Hq);
  c.bytes = c.state_acc_off + align256(sizeof(float) * (size_t)D * B * Hq);
  return c;
}

size_t cascade_workspace_bound(int B, int n_groups, int max_group, int Hkv, int G, int D, int bs, int max_ctx) {
  return cascade_layout(B, n_groups, max_group, Hkv, G, D, bs, max_ctx, (int64_t)kMaxWavesPerCU * kPlanMaxCUs, 1)
      .bytes;
}

int cascade_max_sequences() { return scan_capacity(true, false); }

template <bool STATE>
static void launch_merge(const DecodeArgs& a, int D, int nq, hipStream_t stream) {
  const int64_t threads = (int64_t)nq * a.G * (D / 4);
  const dim3 mgrid(a.Hkv, a.B, (unsigned)std::min<int64_t>(65535, (threads + 255) / 256));
  const dim3 mblock(threads >= 256 ? 256 : (unsigned)(((threads + 63) / 64) * 64));
  if (D == 64)
    hipLaunchKernelGGL((decode_merge_kernel<64, STATE, STATE>), mgrid, mblock, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_merge_kernel<128, STATE, STATE>), mgrid, mblock, 0, stream, a);
}

pa_status cascade_launch(const DecodeRequest& r, hipStream_t stream) {
  const int P = r.n_groups, nq = r.nq;
  const int tiles = prefix_tiles(nq, r.G);
  const CascadeLayout c = cascade_layout(r.B, P, nq, r.Hkv, r.G, r.D, r.bs, r.plan_ctx,
                                         (int64_t)waves_per_cu(false) * plan_cus(), tiles);
  if (r.workspace_bytes < c.bytes) {
    set_error("pa_decode_shared_prefix: workspace of %zu bytes needed, %zu given", c.bytes, r.workspace_bytes);
    return PA_ERR_WORKSPACE;
  }
  if (P > c.pre.sub_batch || r.B > c.suf.sub_batch) {
    set_error("pa_decode_shared_prefix: %d sequences in %d groups exceed one launch (%d, %d)", r.B, P,
              c.suf.sub_batch, c.pre.sub_batch);
    return PA_ERR_UNSUPPORTED;
  }
  if ((int64_t)std::max(c.pre.nslices * tiles, c.suf.nslices) * r.Hkv >= ((int64_t)1 << 31)) {
    set_error("pa_decode_shared_prefix: the grid is too large");
    return PA_ERR_UNSUPPORTED;
  }
  uint8_t* ws = reinterpret_cast<uint8_t*>(r.workspace);
  const bool fp8 = r.cache_dtype == PA_FP8_E4M3;
  DecodeArgs a{};
  a.k_cache = reinterpret_cast<const uint8_t*>(r.k_cache);
  a.v_cache = reinterpret_cast<const uint8_t*>(r.v_cache);
  a.num_blocks = r.num_blocks;
  a.Hkv = r.Hkv;
  a.G = r.G;
  a.M = r.M;
  a.max_ctx = r.max_ctx;
  a.out_dtype = r.out_dtype == PA_F32 ? 0 : (r.out_dtype == PA_F16 ? 1 : 2);
  a.qk_scale_log2 = r.scale * (fp8 ? r.k_scale : 1.f) * 1.4426950408889634f;
  a.v_scale = fp8 ? r.v_scale : 1.f;
  a.out = r.out;
  a.q = r.q;
  a.block_tables = r.block_tables;
  a.group_start = r.group_start;
  a.prefix_lens = r.prefix_lens;
  a.n_groups = P;
  a.state_ml = reinterpret_cast<float*>(ws + c.state_ml_off);
  a.state_acc = reinterpret_cast<float*>(ws + c.state_acc_off);
  const hipEvent_t t_start = g_time_start, t_stop = g_time_stop;
  g_time_start = g_time_stop = nullptr;

  // prefix pass: the groups, their members as the queries, each member seeing
  // the whole prefix; whole prefixes leave states, cut ones partials merged
  // into states
  DecodeArgs pre = a;
  pre.meta = reinterpret_cast<int32_t*>(ws + c.pre.meta_off);
  pre.part_ml = reinterpret_cast<float*>(ws + c.pre.ml_off);
  pre.part_acc = reinterpret_cast<float*>(ws + c.pre.acc_off);
  pre.B = P;
  pre.context_lens = r.prefix_lens;
  pre.q_start = r.group_start;
  pre.nq = nq;
  pre.q_rows = r.B;
  pre.nslices = c.pre.nslices;
  pre.min_slice = c.pre.min_slice;
  pre.seg_cost = c.pre.seg_cost;
  pre.head_tiles = tiles;
  if (!launch_cascade_pass(true, pre, r.cache_dtype, r.q_dtype, r.D, r.bs,
                           dim3((unsigned)((int64_t)c.pre.nslices * r.Hkv * tiles)), stream,
                           LaunchEvents{t_start, nullptr})) {
    set_error("pa_decode_shared_prefix: no kernel built for cache dtype %d, q dtype %d, head_dim %d, block size %d",
              r.cache_dtype, r.q_dtype, r.D, r.bs);
    return PA_ERR_UNSUPPORTED;
  }
  if (c.pre.nslices > 1) launch_merge<true>(pre, r.D, nq, stream);

  // suffix pass: every sequence from its group's prefix length on, starting
  // from its state
  DecodeArgs suf = a;
  const uint8_t* sw = ws + c.suf_off;
  suf.meta = reinterpret_cast<int32_t*>(const_cast<uint8_t*>(sw) + c.suf.meta_off);
  suf.part_ml = reinterpret_cast<float*>(const_cast<uint8_t*>(sw) + c.suf.ml_off);
  suf.part_acc = reinterpret_cast<float*>(const_cast<uint8_t*>(sw) + c.suf.acc_off);
  suf.B = r.B;
  suf.context_lens = r.context_lens;
  suf.q_start = nullptr;
  suf.nq = 1;
  suf.q_rows = r.B;
  suf.nslices = c.suf.nslices;
  suf.min_slice = c.suf.min_slice;
  suf.seg_cost = c.suf.seg_cost;
  suf.head_tiles = 1;
  launch_cascade_pass(false, suf, r.cache_dtype, r.q_dtype, r.D, r.bs, dim3((unsigned)((int64_t)c.suf.nslices * r.Hkv)),
                      stream, LaunchEvents{nullptr, t_stop});
  if (c.suf.nslices > 1) launch_merge<false>(suf, r.D, 1, stream);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error("pa_decode_shared_prefix: launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}

}  // namespace pa
