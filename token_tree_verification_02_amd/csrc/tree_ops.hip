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

// One workgroup per sequence, one thread per node.  parent, depth and the
// prefix length arrive in one round of global loads; everything after that
// (validation, the parent-chain walk) reads LDS.
__global__ __launch_bounds__(256) void tree_build_kernel(int n, const int32_t* __restrict__ parent,
                                                         const int32_t* __restrict__ depth,
                                                         const int32_t* __restrict__ plen,
                                                         uint64_t* __restrict__ mask, int32_t* __restrict__ pos,
                                                         int32_t* __restrict__ status) {
  __shared__ int sp[TV_NMAX], sd[TV_NMAX];
  const int b = blockIdx.x, u = threadIdx.x;
  const int W = (n + 63) >> 6;
  const int L = plen[b];
  if (u < n) {
    sp[u] = parent[(size_t)b * n + u];
    sd[u] = depth[(size_t)b * n + u];
  }
  __syncthreads();
  int bad = 0;
  if (u < n) {
    const int p = sp[u];
    const int du = sd[u];
    if (u == 0)
      bad = (p != -1) || (du != 0);
    else
      bad = (p < 0) || (p >= u) || (du != sd[p] + 1);
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
    pos[(size_t)b * n + u] = L + du;
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

// (bv, bi) := the better of itself and its DPP partner's pair (all lanes active:
// a lane reads its partner's register whether or not the partner is active)
template <int CTRL>
__device__ __forceinline__ void best_with(float& bv, int& bi) {
  const float ov = dpp<CTRL>(bv);
  const int oi = dpp<CTRL>(bi);
  if (beats(ov, oi, bv, bi)) {
    bv = ov;
    bi = oi;
  }
}

// One workgroup of 256 threads per logits row.  Each thread loads 16 16-byte
// vectors per round before it compares anything, keeps the index of the first
// vector whose maximum beats its running best, and at the end re-reads that one
// vector (a cache hit) to find the lowest index of the maximum inside it; DPP moves
// and an LDS step then reduce (value, index) pairs.
// the low / high 16-bit element of a 32-bit word, as float (exact)
template <int DT>
__device__ __forceinline__ float lo16(uint32_t w) {
  return DT == TV_BF16 ? bf16lo(w) : f16_to_f32((uint16_t)w);
}
template <int DT>
__device__ __forceinline__ float hi16(uint32_t w) {
  return DT == TV_BF16 ? bf16hi(w) : f16_to_f32((uint16_t)(w >> 16));
}

// DT: tv_dtype of the logits (16-bit types decode exactly to float)
template <int DT>
__global__ __launch_bounds__(256) void argmax_kernel(const void* __restrict__ logits, int V,
                                                     int32_t* __restrict__ am) {
  constexpr bool W16 = DT != TV_F32;
  constexpr int EPV = W16 ? 8 : 4;  // elements per 16-byte vector
  constexpr int R = 16;              // vectors in flight per thread (a 32000-entry bf16 row in one round)
  const size_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t es = W16 ? 2 : 4;
  const char* rp = (const char*)logits + row * (size_t)V * es;
  float bv = -INFINITY;
  int bi = INT_MAX;
  int done = 0;
  if ((((uintptr_t)rp) & 15) == 0) {
    const int nv = V / EPV;
    const uint4* vp = (const uint4*)rp;
    float vbest = -INFINITY;
    int vidx = -1;
    for (int base = 0; base < nv; base += R * 256) {
      uint4 w[R];
#pragma unroll
      for (int k = 0; k < R; ++k)  // unconditional loads (clamped index): all R stay in flight
        w[k] = vp[min(base + k * 256 + tid, nv - 1)];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int i = base + k * 256 + tid;
        float m;
        if (W16) {
          m = fmaxf(fmaxf(fmaxf(lo16<DT>(w[k].x), hi16<DT>(w[k].x)), fmaxf(lo16<DT>(w[k].y), hi16<DT>(w[k].y))),
                    fmaxf(fmaxf(lo16<DT>(w[k].z), hi16<DT>(w[k].z)), fmaxf(lo16<DT>(w[k].w), hi16<DT>(w[k].w))));
        } else {
          m = fmaxf(fmaxf(__uint_as_float(w[k].x), __uint_as_float(w[k].y)),
                    fmaxf(__uint_as_float(w[k].z), __uint_as_float(w[k].w)));
        }
        // vectors are visited in increasing index order: strict > keeps the first
        const bool take = i < nv && (m > vbest || vidx < 0);
        vbest = take ? m : vbest;
        vidx = take ? i : vidx;
      }
    }
    if (vidx >= 0) {  // lowest index of the maximum inside the winning vector (re-read: cached)
      const uint4 v = vp[vidx];
      const uint32_t w0 = v.x, w1 = v.y, w2 = v.z, w3 = v.w;
      int e = EPV;
      if (W16) {
        e = hi16<DT>(w3) == vbest ? 7 : e;
        e = lo16<DT>(w3) == vbest ? 6 : e;
        e = hi16<DT>(w2) == vbest ? 5 : e;
        e = lo16<DT>(w2) == vbest ? 4 : e;
        e = hi16<DT>(w1) == vbest ? 3 : e;
        e = lo16<DT>(w1) == vbest ? 2 : e;
        e = hi16<DT>(w0) == vbest ? 1 : e;
        e = lo16<DT>(w0) == vbest ? 0 : e;
      } else {
        e = __uint_as_float(w3) == vbest ? 3 : e;
        e = __uint_as_float(w2) == vbest ? 2 : e;
        e = __uint_as_float(w1) == vbest ? 1 : e;
        e = __uint_as_float(w0) == vbest ? 0 : e;
      }
      // no element compares equal only when vbest is NaN (out of contract): the
      // index still stays inside the winning vector, so inside [0, V)
      bi = vidx * EPV + min(e, EPV - 1);
      bv = vbest;
    }
    done = nv * EPV;
  }
  for (int i = done + tid; i < V; i += 256) {  // unaligned rows and the tail
    const float x = W16 ? lo16<DT>(((const uint16_t*)rp)[i]) : ((const float*)rp)[i];
    if (x > bv || bi == INT_MAX) {
      bv = x;
      bi = i;
    }
  }
  // the wave's best: within rows of 16 lanes by DPP moves, then the other rows'
  // bests read from lanes 16, 32, 48 (the order is a total one, so any
  // combination order gives the same pair)
  best_with<kDppXor1>(bv, bi);
  best_with<kDppXor2>(bv, bi);
  best_with<kDppHalfMirror>(bv, bi);
  best_with<kDppMirror>(bv, bi);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float ov = lane_read(bv, 16 * r);
    const int oi = lane_read(bi, 16 * r);
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

// One workgroup per sequence, one thread per node.  Every node first decides in
// parallel whether its draft token equals the argmax at its parent; the lowest
// such child of each node is kept with an LDS atomic min.  The walk is then a
// pointer chase through that table, each hop to a larger node id, so it ends
// within n steps whatever the input.
__global__ __launch_bounds__(256) void walk_kernel(int n, const int32_t* __restrict__ am,
                                                   const int32_t* __restrict__ tokens,
                                                   const int32_t* __restrict__ parent, int32_t* __restrict__ path,
                                                   int32_t* __restrict__ plen, int32_t* __restrict__ bonus) {
  __shared__ int sa[TV_NMAX], fc[TV_NMAX], sp[TV_NMAX];
  __shared__ int slen;
  const int b = blockIdx.x, v = threadIdx.x;
  int p = -1, tok = 0;
  if (v < n) {
    sa[v] = am[(size_t)b * n + v];
    p = parent[(size_t)b * n + v];
    tok = tokens[(size_t)b * n + v];
    fc[v] = INT_MAX;
  }
  __syncthreads();
  if (v < n && v > 0 && p >= 0 && p < v && tok == sa[p]) atomicMin(&fc[p], v);
  __syncthreads();
  int32_t* pr = path + (size_t)b * n;
  if (v == 0) {
    int cur = 0, len = 1;
    sp[0] = 0;
    while (len < n) {
      const int c = fc[cur];
      if (c == INT_MAX) break;
      cur = c;
      sp[len++] = cur;
    }
    slen = len;
    plen[b] = len;
    bonus[b] = sa[cur];
  }
  __syncthreads();
  if (v < n) pr[v] = v < slen ? sp[v] : -1;
}

}  // namespace

hipError_t launch_tree_build(int B, int n, const int32_t* parent, const int32_t* depth, const int32_t* plen,
                             uint64_t* mask, int32_t* pos, int32_t* status, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int threads = ((n + 63) / 64) * 64;
  hipLaunchKernelGGL(tree_build_kernel, dim3(B), dim3(threads), 0, s, n, parent, depth, plen, mask, pos, status);
  return hipGetLastError();
}

hipError_t launch_verify(int B, int n, int V, int dtype, const void* logits, const int32_t* tokens,
                         const int32_t* parent, int32_t* am, int32_t* path, int32_t* plen, int32_t* bonus,
                         hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (dtype == TV_BF16)
    hipLaunchKernelGGL(argmax_kernel<TV_BF16>, dim3(B * n), dim3(256), 0, s, logits, V, am);
  else if (dtype == TV_F16)
    hipLaunchKernelGGL(argmax_kernel<TV_F16>, dim3(B * n), dim3(256), 0, s, logits, V, am);
  else
    hipLaunchKernelGGL(argmax_kernel<TV_F32>, dim3(B * n), dim3(256), 0, s, logits, V, am);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(walk_kernel, dim3(B), dim3(((n + 63) / 64) * 64), 0, s, n, am, tokens, parent, path, plen,
                     bonus);
  return hipGetLastError();
}

}  // namespace tv
