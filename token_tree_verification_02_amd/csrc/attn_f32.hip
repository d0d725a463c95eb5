// Tree attention in fp32 on the vector ALUs, and the split-K merge.
//
// The fp32 path serves fp32 workloads (small models, tests at full precision):
// one wave per (sequence, node, query head).  Keys are spread over the 64 lanes
// for the scores, values over lanes by head dimension for the weighted sum (each step reads a
// 64-token run of one head-dim column), with
// the usual running max / running sum of an online softmax over 64-key chunks.
// The set attended is the same as the bf16 path: every cached prefix token plus
// the tree nodes whose bit is set in the node's ancestor mask (SpecInfer
// explainer, token-tree structure section, attention equation and mask).
//
// The merge combines per-chunk partials (m, l, O) of long prefixes exactly:
// softmax over a disjoint union factorises into the chunks' log-sum-exp terms.
#include <float.h>

#include "tv_internal.h"

namespace tv {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a, int cap) {
  constexpr int DP = D / 64;  // head-dim entries per lane in the weighted sum
  __shared__ float qs[D];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const int n = a.n, Hq = a.Hq, Hkv = a.Hkv, G = a.G;
  const int h = blockIdx.x % Hq;
  const int u = (blockIdx.x / Hq) % n;
  const int b = blockIdx.x / (Hq * n);
  const int g = h / G;
  const float* __restrict__ kc = (const float*)a.kc;
  const float* __restrict__ vc = (const float*)a.vc;
  const float* __restrict__ ktr = (const float*)a.kt;
  const float* __restrict__ vtr = (const float*)a.vt;

  const float* qp = (const float*)a.q + ((size_t)(b * n + u) * Hq + h) * D;
  for (int d = lane; d < D; d += 64) qs[d] = qp[d];
  const int Lraw = a.plen[b];
  const int L = Lraw < 0 ? 0 : (Lraw > cap ? cap : Lraw);
  if (a.status != nullptr && u == 0 && h == 0) {
    int bad = (Lraw < 0 || Lraw > cap);
    if (a.paged)
      for (int i = lane; i < (L + TV_PAGE - 1) / TV_PAGE; i += 64) {
        const int id = a.bt[(size_t)b * a.max_blocks + i];
        bad |= (id < 0 || id >= a.num_blocks);
      }
    bad = __any(bad);
    if (lane == 0) a.status[b] = bad ? TV_EINVAL : TV_OK;
  }
  __syncthreads();
  const uint64_t* mrow = a.mask + ((size_t)b * n + u) * a.W;

  float m = -INFINITY, l = 0.f;
  float o[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) o[i] = 0.f;

  // key row pointer of prefix token j (nullptr: block id out of range -> zero key)
  auto krow = [&](int j) -> const float* {
    if (a.paged) {
      const int blk = a.bt[(size_t)b * a.max_blocks + (j >> 4)];
      if (blk < 0 || blk >= a.num_blocks) return nullptr;
      return kc + (((size_t)blk * Hkv + g) * TV_PAGE + (j & 15)) * D;
    }
    return kc + (((size_t)b * Hkv + g) * a.Lmax + j) * D;
  };
  auto vval = [&](int d, int j) -> float {
    if (a.paged) {
      const int blk = a.bt[(size_t)b * a.max_blocks + (j >> 4)];
      if (blk < 0 || blk >= a.num_blocks) return 0.f;
      return vc[(((size_t)blk * Hkv + g) * TV_PAGE + (j & 15)) * D + d];
    }
    return vc[(((size_t)b * Hkv + g) * a.Lmax + j) * D + d];
  };
  // fold one chunk of scores (lane = key) into the running state
  auto fold = [&](float s, bool valid, int cnt, auto&& value_of) {
    const float mx = wave_max(valid ? s : -INFINITY);
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) return;
    const float alpha = (m == -INFINITY) ? 0.f : exp2f(m - m_new);
    const float p = valid ? exp2f(s - m_new) : 0.f;
    l = l * alpha + wave_sum(p);
    ps[lane] = p;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < DP; ++i) {
      const int d = lane + 64 * i;
      float acc = o[i] * alpha;
      for (int jj = 0; jj < cnt; ++jj)
        if (ps[jj] != 0.f) acc += ps[jj] * value_of(d, jj);
      o[i] = acc;
    }
    __syncthreads();
    m = m_new;
  };

  for (int k0 = 0; k0 < L; k0 += 64) {
    const int j = k0 + lane;
    const bool valid = j < L;
    float s = 0.f;
    if (valid) {
      const float* kr = krow(j);
      if (kr)
        for (int d = 0; d < D; ++d) s += qs[d] * kr[d];
      s *= a.scale_log2;
    }
    fold(s, valid, min(64, L - k0), [&](int d, int jj) { return vval(d, k0 + jj); });
  }
  for (int v0 = 0; v0 < n; v0 += 64) {
    const int v = v0 + lane;
    const bool valid = v < n && ((mrow[v >> 6] >> (v & 63)) & 1);
    float s = 0.f;
    if (valid) {
      const float* kr = ktr + (((size_t)b * n + v) * Hkv + g) * D;
      for (int d = 0; d < D; ++d) s += qs[d] * kr[d];
      s *= a.scale_log2;
    }
    fold(s, valid, min(64, n - v0),
         [&](int d, int jj) { return vtr[(((size_t)b * n + v0 + jj) * Hkv + g) * D + d]; });
  }

  float* op = (float*)a.out + ((size_t)(b * n + u) * Hq + h) * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int i = 0; i < DP; ++i) op[lane + 64 * i] = o[i] * inv;
  if (a.lse != nullptr && lane == 0) a.lse[(size_t)(b * n + u) * Hq + h] = (m + log2f(l)) * kLn2;
}

// One thread per (row, 4 head-dim entries) of a (sequence, KV head).
template <int OUT>  // tv_dtype of the output
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, int nchunks, int chunk_len, int cap,
                                                    int row_blocks) {
  const int D = a.D, rows = a.n * a.G;
  const int tpr = D / 4;                    // threads per row
  const int rpb = 256 / tpr;                // rows per block
  const int rblk = blockIdx.x % row_blocks;
  const int bg = blockIdx.x / row_blocks;
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int row = rblk * rpb + threadIdx.x / tpr;
  const int d0 = (threadIdx.x % tpr) * 4;
  if (row >= rows) return;
  const int Lraw = a.plen[b];
  const int L = Lraw < 0 ? 0 : (Lraw > cap ? cap : Lraw);
  const int ncb = L > 0 ? (L + chunk_len - 1) / chunk_len : 1;
  if (ncb == 1) return;  // the single chunk wrote the output itself
  const size_t base = (size_t)(b * a.Hkv + g) * nchunks;
  float M = -INFINITY;
  for (int c = 0; c < ncb; ++c) M = fmaxf(M, a.ws_ml[2 * ((base + c) * rows + row)]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float lt = 0.f;
  for (int c = 0; c < ncb; ++c) {
    const size_t pi = (base + c) * rows + row;
    const float mc = a.ws_ml[2 * pi], lc = a.ws_ml[2 * pi + 1];
    const float w = (mc == -INFINITY) ? 0.f : exp2f(mc - M);
    const float4 oc = *(const float4*)(a.ws_o + pi * D + d0);
    acc.x += w * oc.x;
    acc.y += w * oc.y;
    acc.z += w * oc.z;
    acc.w += w * oc.w;
    lt += w * lc;
  }
  const float inv = 1.f / lt;
  const int u = row / a.G, gi = row % a.G, h = g * a.G + gi;
  const size_t oi = ((size_t)(b * a.n + u) * a.Hq + h) * D + d0;
  if (OUT == TV_BF16) {
    uint2 w;
    w.x = (uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
    w.y = (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
    *(uint2*)((uint16_t*)a.out + oi) = w;
  } else if (OUT == TV_F16) {
    const auto h = [](float x) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x); };
    uint2 w;
    w.x = h(acc.x * inv) | (h(acc.y * inv) << 16);
    w.y = h(acc.z * inv) | (h(acc.w * inv) << 16);
    *(uint2*)((uint16_t*)a.out + oi) = w;
  } else {
    *(float4*)((float*)a.out + oi) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (a.lse != nullptr && d0 == 0) a.lse[(size_t)(b * a.n + u) * a.Hq + h] = (M + log2f(lt)) * kLn2;
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  const int grid = a.B * a.n * a.Hq;
  if (grid == 0) return hipSuccess;
  if (a.D == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(grid), dim3(64), 0, s, a, p.cap);
  else
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(grid), dim3(64), 0, s, a, p.cap);
  return hipGetLastError();
}

hipError_t launch_merge(const AttnArgs& a, const AttnPlan& p, int out_dtype, hipStream_t s) {
  if (p.nchunks <= 1 || a.B == 0) return hipSuccess;
  const int rpb = 256 / (a.D / 4);
  const int row_blocks = (p.rows + rpb - 1) / rpb;
  const int grid = a.B * a.Hkv * row_blocks;
  if (out_dtype == TV_BF16)
    hipLaunchKernelGGL(merge_kernel<TV_BF16>, dim3(grid), dim3(256), 0, s, a, p.nchunks, p.chunk_len, p.cap,
                       row_blocks);
  else if (out_dtype == TV_F16)
    hipLaunchKernelGGL(merge_kernel<TV_F16>, dim3(grid), dim3(256), 0, s, a, p.nchunks, p.chunk_len, p.cap,
                       row_blocks);
  else
    hipLaunchKernelGGL(merge_kernel<TV_F32>, dim3(grid), dim3(256), 0, s, a, p.nchunks, p.chunk_len, p.cap,
                       row_blocks);
  return hipGetLastError();
}

}  // namespace tv
