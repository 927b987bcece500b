// Split-K planning, the work-list and reduce kernels, and the host side of
// pa_decode: partition sizing, workspace layout and kernel choice.
#include <cstdlib>
#include <cstring>

#include "decode_common.h"
#include "pa_internal.h"

namespace pa {

bool launch_decode_mfma(const DecodeArgs& a, int ct, int qt, int head_dim, int bs, dim3 grid,
                        hipStream_t stream);
bool launch_decode_valu(const DecodeArgs& a, int ct, int qt, int head_dim, int bs, int group,
                        dim3 grid, hipStream_t stream);
bool valu_supports(int ct, int qt, int head_dim, int bs, int group);

// Work list: one (sequence, partition) pair per partition that holds at
// least one position; an empty sequence gets one item (it writes zeros).
// One workgroup; sequences are taken 1024 at a time with an LDS scan.
__global__ __launch_bounds__(1024) void decode_plan_kernel(const int32_t* context_lens, int B,
                                                           int max_ctx, int part_tokens,
                                                           int32_t* work) {
  __shared__ int scan[1024];
  const int tid = threadIdx.x;
  int total = 0;
  for (int base = 0; base < B; base += 1024) {
    const int s = base + tid;
    int n = 0;
    if (s < B) {
      int L = context_lens[s];
      L = L < 0 ? 0 : (L > max_ctx ? max_ctx : L);
      n = L > 0 ? (L + part_tokens - 1) / part_tokens : 1;
    }
    scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int first = total + scan[tid] - n;
    for (int k = 0; k < n; ++k) {
      work[2 + 2 * (first + k)] = s;
      work[3 + 2 * (first + k)] = k;
    }
    total += scan[1023];
    __syncthreads();
  }
  if (tid == 0) work[0] = total;
}

// Merge the partitions of one (sequence, KV head) for every query head of
// the group:  M = max m_p;  out = v_scale * sum 2^(m_p-M) acc_p / sum 2^(m_p-M) l_p.
// Partitions are visited in increasing order, so the result does not depend
// on where the blocks sit in the pool.
template <int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int L = context_len(a, s);
  const int n = L > 0 ? (L + a.part_tokens - 1) / a.part_tokens : 1;
  if (n <= 1) return;  // written directly by the partition kernel
  constexpr int D4 = D / 4;
  for (int idx = threadIdx.x; idx < a.G * D4; idx += blockDim.x) {
    const int i = idx / D4;
    const int d = 4 * (idx - i * D4);
    const int head = h * a.G + i;
    const int64_t base = part_index(a, s, head, 0);
    float M = -INFINITY;
    for (int p = 0; p < n; ++p) M = fmaxf(M, a.part_ml[2 * (base + p)]);
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int p = 0; p < n; ++p) {
      const f32x2 ml = *reinterpret_cast<const f32x2*>(a.part_ml + 2 * (base + p));
      const float w = fast_exp2(ml[0] - M);
      den = fmaf(w, ml[1], den);
      const f32x4 x = *reinterpret_cast<const f32x4*>(a.part_acc + (base + p) * D + d);
      num += w * x;
    }
    const float f = a.v_scale / den;
    const float v[4] = {num[0] * f, num[1] * f, num[2] * f, num[3] * f};
    store_out(a, s, head, D, d, v, 4);
  }
}

// ---------------------------------------------------------------- host side

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodePlan plan_decode(int B, int Hkv, int G, int D, int bs, int max_ctx) {
  DecodePlan p{};
  // Partition length: 256 positions, shorter while the batch would give
  // fewer than ~4096 items (16 per compute unit), longer while a sequence
  // would need more than 64 partitions (bounded by 64 blocks per partition).
  int P = 256;
  auto parts = [&](int len) { return max_ctx > 0 ? (max_ctx + len - 1) / len : 1; };
  while (P > 64 && (int64_t)B * Hkv * parts(P) < 4096) P /= 2;
  while (parts(P) > 64 && P * 2 <= 64 * bs) P *= 2;
  p.part_tokens = P;
  p.nparts = parts(P);
  if (p.nparts <= 1) {
    p.nparts = 1;
    return p;  // every sequence fits in one partition: no workspace
  }
  const size_t Hq = (size_t)Hkv * G;
  const size_t rows = (size_t)B * Hq * p.nparts;
  p.work_off = 0;
  p.ml_off = align256(sizeof(int32_t) * (2 + 2 * (size_t)B * p.nparts));
  p.acc_off = p.ml_off + align256(sizeof(float) * 2 * rows);
  p.bytes = p.acc_off + align256(sizeof(float) * (size_t)D * rows);
  return p;
}

int decode_variant_override() {
  const char* v = std::getenv("PA_DECODE_VARIANT");
  if (!v) return 0;
  if (!std::strcmp(v, "valu")) return 1;
  if (!std::strcmp(v, "mfma")) return 2;
  return 0;
}

bool decode_uses_valu(int variant, int G) { return variant == 1 || (variant == 0 && G <= 2); }

bool decode_valu_supported(int ct, int qt, int D, int bs, int G) { return valu_supports(ct, qt, D, bs, G); }

pa_status decode_launch(const DecodeRequest& r, hipStream_t stream) {
  const DecodePlan plan = plan_decode(r.B, r.Hkv, r.G, r.D, r.bs, r.plan_ctx);
  const bool valu = decode_uses_valu(decode_variant_override(), r.G);
  if (valu && !valu_supports(r.cache_dtype, r.q_dtype, r.D, r.bs, r.G)) {
    set_error("pa_decode: the VALU kernel is not built for group %d, head_dim %d, block size %d",
              r.G, r.D, r.bs);
    return PA_ERR_UNSUPPORTED;
  }

  {
    const int64_t items = (int64_t)r.B * plan.nparts * r.Hkv * (valu ? 1 : (r.G + 15) / 16);
    if (items >= ((int64_t)1 << 31)) {
      set_error("pa_decode: %lld work items exceed the 32-bit item index", (long long)items);
      return PA_ERR_UNSUPPORTED;
    }
  }
  DecodeArgs a{};
  a.out = r.out;
  a.q = r.q;
  a.k_cache = reinterpret_cast<const uint8_t*>(r.k_cache);
  a.v_cache = reinterpret_cast<const uint8_t*>(r.v_cache);
  a.block_tables = r.block_tables;
  a.context_lens = r.context_lens;
  a.num_blocks = r.num_blocks;
  a.B = r.B;
  a.Hkv = r.Hkv;
  a.G = r.G;
  a.M = r.M;
  a.max_ctx = r.max_ctx;
  a.nparts = plan.nparts;
  a.part_tokens = plan.part_tokens;
  a.head_tiles = valu ? 1 : (r.G + 15) / 16;
  a.dense = plan.nparts == 1;
  a.out_dtype = r.out_dtype == PA_F32 ? 0 : (r.out_dtype == PA_F16 ? 1 : 2);
  const bool fp8 = r.cache_dtype == PA_FP8_E4M3;
  a.qk_scale_log2 = r.scale * (fp8 ? r.k_scale : 1.f) * 1.4426950408889634f;
  a.v_scale = fp8 ? r.v_scale : 1.f;
  if (!a.dense) {
    uint8_t* ws = reinterpret_cast<uint8_t*>(r.workspace);
    a.work = reinterpret_cast<const int32_t*>(ws + plan.work_off);
    a.part_ml = reinterpret_cast<float*>(ws + plan.ml_off);
    a.part_acc = reinterpret_cast<float*>(ws + plan.acc_off);
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, stream, r.context_lens, r.B,
                       r.max_ctx, plan.part_tokens, reinterpret_cast<int32_t*>(ws + plan.work_off));
  }
  const int64_t upper = (int64_t)r.B * plan.nparts * r.Hkv * a.head_tiles;
  const int64_t cap = 16384;
  const dim3 grid((unsigned)(upper < cap ? upper : cap));
  const int ct = r.cache_dtype, qt = r.q_dtype;
  const bool ok = valu ? launch_decode_valu(a, ct, qt, r.D, r.bs, r.G, grid, stream)
                       : launch_decode_mfma(a, ct, qt, r.D, r.bs, grid, stream);
  if (!ok) {
    set_error("pa_decode: no kernel built for cache dtype %d, q dtype %d, head_dim %d, block size %d, group %d (%s)",
              ct, qt, r.D, r.bs, r.G, valu ? "valu" : "mfma");
    return PA_ERR_UNSUPPORTED;
  }
  if (!a.dense) {
    const dim3 rgrid(r.Hkv, r.B);
    if (r.D == 64)
      hipLaunchKernelGGL(decode_reduce_kernel<64>, rgrid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_reduce_kernel<128>, rgrid, dim3(256), 0, stream, a);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    set_error("pa_decode: launch failed: %s", hipGetErrorString(err));
    return PA_ERR_HIP;
  }
  return PA_OK;
}

}  // namespace pa
