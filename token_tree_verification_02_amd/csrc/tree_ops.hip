// Topology encoder and greedy verification kernels.
//
// tree_build precomputes the topology-aware causal mask (SpecInfer explainer,
// kernel-fusion section: a mask matrix built from ancestor relations): node u's
// row is the set S_u of nodes on its root path, u included (token-tree
// structure section), stored as W = ceil(n/64) 64-bit words.
//
// Greedy verification (tree-verification section) is an HBM-streaming vocab
// argmax per node followed by a walk from the root.  The walk accepts a child
// whose draft token equals the argmax at its parent and stops at the first node
// with none; the argmax there is the one token the target model adds (the
// sequence rule of the speculative-decoding explainer's mechanism section and
// the operations guide's diagram, applied branch by branch).
#include <limits.h>

#include "tv_internal.h"

namespace tv {
namespace {

// One workgroup per sequence, one thread per node.
__global__ __launch_bounds__(256) void tree_build_kernel(int n, const int32_t* __restrict__ parent,
                                                         const int32_t* __restrict__ depth,
                                                         const int32_t* __restrict__ plen,
                                                         uint64_t* __restrict__ mask, int32_t* __restrict__ pos,
                                                         int32_t* __restrict__ status) {
  __shared__ int sp[TV_NMAX];
  const int b = blockIdx.x, u = threadIdx.x;
  const int W = (n + 63) >> 6;
  if (u < n) sp[u] = parent[(size_t)b * n + u];
  __syncthreads();
  int bad = 0;
  if (u < n) {
    const int p = sp[u];
    const int du = depth[(size_t)b * n + u];
    if (u == 0)
      bad = (p != -1) || (du != 0);
    else
      bad = (p < 0) || (p >= u) || (du != depth[(size_t)b * n + p] + 1);
    uint64_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
    int v = u;
    // walk the parent chain; every hop must move to a smaller id, so at most u+1 steps
    for (int step = 0; step <= u; ++step) {
      const uint64_t bit = 1ull << (v & 63);
      const int wd = v >> 6;
      w0 |= (wd == 0) ? bit : 0;
      w1 |= (wd == 1) ? bit : 0;
      w2 |= (wd == 2) ? bit : 0;
      w3 |= (wd == 3) ? bit : 0;
      if (v == 0) break;
      const int pv = sp[v];
      if (pv < 0 || pv >= v) {
        bad = 1;
        break;
      }
      v = pv;
    }
    uint64_t* mr = mask + ((size_t)b * n + u) * W;
    mr[0] = w0;
    if (W > 1) mr[1] = w1;
    if (W > 2) mr[2] = w2;
    if (W > 3) mr[3] = w3;
    pos[(size_t)b * n + u] = plen[b] + du;
  }
  bad = __syncthreads_or(bad);
  if (u == 0) status[b] = bad ? TV_ETOPOLOGY : TV_OK;
}

struct Best {
  float v;
  int i;
};
// (value desc, index asc): does (v2, i2) beat (v1, i1)?
__device__ __forceinline__ bool beats(float v2, int i2, float v1, int i1) {
  return v2 > v1 || (v2 == v1 && i2 < i1) || (i1 == INT_MAX && i2 != INT_MAX);
}

// One workgroup of 256 threads per logits row.  Each thread scans its elements
// in increasing index order keeping the first maximum, then a wave shuffle and
// an LDS step reduce (value, index) pairs under the same order.
template <bool BF16>
__global__ __launch_bounds__(256) void argmax_kernel(const void* __restrict__ logits, int V,
                                                     int32_t* __restrict__ am) {
  constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte vector
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x;
  float bv = -INFINITY;
  int bi = INT_MAX;
  auto take = [&](float x, int i) {
    if (x > bv || bi == INT_MAX) {
      bv = x;
      bi = i;
    }
  };
  const size_t es = BF16 ? 2 : 4;
  const char* rp = (const char*)logits + row * (size_t)V * es;
  int done = 0;
  if ((((uintptr_t)rp) & 15) == 0) {
    const int nv = V / EPV;
    const uint4* vp = (const uint4*)rp;
    int i = tid;
    for (; i + 3 * 256 < nv; i += 4 * 256) {
      uint4 w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = vp[i + k * 256];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
        const int e0 = (i + k * 256) * EPV;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (BF16) {
            take(bf16lo(ws[e]), e0 + 2 * e);
            take(bf16hi(ws[e]), e0 + 2 * e + 1);
          } else {
            take(__uint_as_float(ws[e]), e0 + e);
          }
        }
      }
    }
    // the 4-way batches above all precede this thread's remaining vectors, and
    // each thread's indices still increase monotonically
    for (; i < nv; i += 256) {
      const uint4 w = vp[i];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      const int e0 = i * EPV;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (BF16) {
          take(bf16lo(ws[e]), e0 + 2 * e);
          take(bf16hi(ws[e]), e0 + 2 * e + 1);
        } else {
          take(__uint_as_float(ws[e]), e0 + e);
        }
      }
    }
    done = nv * EPV;
  }
  for (int i = done + tid; i < V; i += 256) {
    const float x = BF16 ? bf16_to_f32(((const uint16_t*)rp)[i]) : ((const float*)rp)[i];
    take(x, i);
  }
  // reduce
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (beats(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  if ((tid & 63) == 0) {
    sv[tid >> 6] = bv;
    si[tid >> 6] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < 4; ++k)
      if (beats(sv[k], si[k], bv, bi)) {
        bv = sv[k];
        bi = si[k];
      }
    am[row] = bi;
  }
}

// One wave per sequence.  Every step moves to a child with a larger id, so the
// walk ends within n steps whatever the input.
__global__ __launch_bounds__(64) void walk_kernel(int n, const int32_t* __restrict__ am,
                                                  const int32_t* __restrict__ tokens,
                                                  const int32_t* __restrict__ parent, int32_t* __restrict__ path,
                                                  int32_t* __restrict__ plen, int32_t* __restrict__ bonus) {
  __shared__ int sp[TV_NMAX], st[TV_NMAX], sa[TV_NMAX];
  const int b = blockIdx.x, lane = threadIdx.x;
  for (int i = lane; i < n; i += 64) {
    sp[i] = parent[(size_t)b * n + i];
    st[i] = tokens[(size_t)b * n + i];
    sa[i] = am[(size_t)b * n + i];
  }
  __syncthreads();
  int cur = 0, len = 1;
  int32_t* pr = path + (size_t)b * n;
  if (lane == 0) pr[0] = 0;
  for (int step = 1; step < n; ++step) {
    const int target = sa[cur];
    int best = INT_MAX;
    for (int v = lane; v < n; v += 64)
      if (v > cur && sp[v] == cur && st[v] == target) best = min(best, v);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) best = min(best, __shfl_xor(best, o));
    if (best == INT_MAX) break;
    cur = best;
    if (lane == 0) pr[len] = cur;
    ++len;
  }
  for (int i = len + lane; i < n; i += 64) pr[i] = -1;
  if (lane == 0) {
    plen[b] = len;
    bonus[b] = sa[cur];
  }
}

}  // namespace

hipError_t launch_tree_build(int B, int n, const int32_t* parent, const int32_t* depth, const int32_t* plen,
                             uint64_t* mask, int32_t* pos, int32_t* status, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int threads = ((n + 63) / 64) * 64;
  hipLaunchKernelGGL(tree_build_kernel, dim3(B), dim3(threads), 0, s, n, parent, depth, plen, mask, pos, status);
  return hipGetLastError();
}

hipError_t launch_verify(int B, int n, int V, int bf16, const void* logits, const int32_t* tokens,
                         const int32_t* parent, int32_t* am, int32_t* path, int32_t* plen, int32_t* bonus,
                         hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(argmax_kernel<true>, dim3(B * n), dim3(256), 0, s, logits, V, am);
  else
    hipLaunchKernelGGL(argmax_kernel<false>, dim3(B * n), dim3(256), 0, s, logits, V, am);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(walk_kernel, dim3(B), dim3(64), 0, s, n, am, tokens, parent, path, plen, bonus);
  return hipGetLastError();
}

}  // namespace tv
