// Token-tree construction: the expansion step (top-k children per frontier node)
// and the merge of several drafts into one tree.
//
// SpecInfer explainer, multi-draft section: in the expansion-based strategy one
// SSM proposes its top-k tokens at each step and the tree grows in depth
// (configuration <k1, ..., km>); in the merge-based strategy the outputs of
// several SSMs are merged into one token tree (its figure: two SSMs' drafts
// sharing their first token's node).
//
// topk_kernel reads one SSM logits row per workgroup in two passes of 16-byte
// vectors.  The first takes each thread's maximum, then the maxima of the
// workgroup's groups of 16 threads (32 of them): they are entries of the row, so
// the k-th largest of them (k <= 16) bounds the row's k-th largest value from
// below.  The second pass
// (mostly cache hits) skips every vector whose maximum is below that bound and
// keeps, per thread, its best 16 (value desc, index asc) among the entries at
// or above it, which are few, so the insertion code rarely runs.  k rounds of a
// workgroup argmax over the threads' heads then pick the row's top k, and the
// children are written straight into the caller's tree arrays after the
// existing nodes.
//
// merge_kernel builds the trie of one sequence's drafts without sequential
// insertion: position d of draft m names the node of prefix drafts[m][0..d];
// that node belongs to the first draft sharing the prefix, draft m creates the
// nodes from its longest overlap with any earlier draft onward, and a prefix
// sum over the drafts' counts places them in creation order.
#include <limits.h>

#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kKeep = TV_TOPK_MAX;  // per-thread list length (>= k)
// threads per SSM row: 512 keep twice 256's loads in flight (128000-entry rows
// 9% faster, 32000-entry rows 2%); 1024 lose more to the k rounds' barriers
// across 16 waves than they gain
constexpr int kTopkThreads = 512;

// Workgroup barrier that orders LDS accesses only (no wait for global stores).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// (value desc, index asc): does (v2, i2) rank before (v1, i1)?
__device__ __forceinline__ bool before(float v2, int i2, float v1, int i1) {
  return v2 > v1 || (v2 == v1 && i2 < i1) || (i1 == INT_MAX && i2 != INT_MAX);
}

// insert (v, i) into a sorted list; i is larger than every index already kept,
// so it goes after every entry with value >= v
__device__ __forceinline__ void keep_insert(float (&lv)[kKeep], int (&li)[kKeep], float v, int i) {
  if (!(v > lv[kKeep - 1]) && li[kKeep - 1] != INT_MAX) return;
#pragma unroll
  for (int s = kKeep - 1; s > 0; --s) {
    const bool shift = v > lv[s - 1] || li[s - 1] == INT_MAX;  // the new entry goes at or above s-1
    const bool here = !shift && (v > lv[s] || li[s] == INT_MAX);
    lv[s] = shift ? lv[s - 1] : (here ? v : lv[s]);
    li[s] = shift ? li[s - 1] : (here ? i : li[s]);
  }
  if (v > lv[0] || li[0] == INT_MAX) {
    lv[0] = v;
    li[0] = i;
  }
}

// One workgroup of 256 threads per (sequence, frontier slot).  Every workgroup
// checks its sequence's frontier (ids in [0, n_cur), room for the children)
// before writing; slot 0 reports status and the new node count.
template <bool BF16>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(int F, int V, int k, int n_max, const void* __restrict__ logits,
                                                   const int32_t* __restrict__ frontier,
                                                   const int32_t* __restrict__ n_cur, int32_t* __restrict__ parent,
                                                   int32_t* __restrict__ depth, int32_t* __restrict__ tokens,
                                                   float* __restrict__ scores, int32_t* __restrict__ n_out,
                                                   int32_t* __restrict__ status) {
  constexpr int NW = kTopkThreads / 64, NG = kTopkThreads / 16;
  __shared__ float sv[2][NW];  // per round (double-buffered): each wave's best head
  __shared__ int si[2][NW];
  __shared__ unsigned long long sb[NW];
  __shared__ float s_gmax[NG];
  __shared__ float s_thr;
  __shared__ float s_v[kKeep];  // the k winners, written out after the rounds
  __shared__ int s_i[kKeep];
  const int b = blockIdx.x / F, f = blockIdx.x - b * F;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nc = n_cur[b];
  // ---- the sequence's frontier (F <= 256: one slot per thread): valid slots, this slot's rank
  const int fr = tid < F ? frontier[(size_t)b * F + tid] : -1;
  const bool valid = fr >= 0;
  int bad = valid && fr >= nc;
  const unsigned long long bl = __ballot(valid);
  if (lane == 0) sb[wv] = bl;
  bad = __syncthreads_or(bad);
  int nvalid = 0, valid_before = 0;
  for (int w = 0; w < NW; ++w) {
    nvalid += __popcll(sb[w]);
    if (w < (f >> 6)) valid_before += __popcll(sb[w]);
  }
  valid_before += __popcll(sb[f >> 6] & ((1ull << (f & 63)) - 1));
  bad = bad || nc < 1 || nc > n_max || (long long)nc + (long long)nvalid * k > n_max;
  if (f == 0 && tid == 0) {
    status[b] = bad ? TV_EINVAL : TV_OK;
    n_out[b] = bad ? nc : nc + nvalid * k;
  }
  const int p = frontier[(size_t)b * F + f];
  if (bad || p < 0) return;

  const size_t es = BF16 ? 2 : 4;
  const char* row = (const char*)logits + ((size_t)b * F + f) * V * es;
  constexpr int EPV = BF16 ? 8 : 4;
  // vectors in flight per thread in each pass; 8 and 8 measured best (4 and 4:
  // a 128000-entry row 9% slower; 16 in pass 2 spills next to the 32 registers
  // of the per-thread lists)
  constexpr int R1 = 8;
  constexpr int R2 = 8;
  const bool aligned = ((uintptr_t)row & 15) == 0;
  const int nv = aligned ? V / EPV : 0;
  const uint4* vp = (const uint4*)row;
  // Visit every element of this thread's share in increasing index order:
  // 16-byte vectors first, then the unaligned tail one by one.
  auto sweep = [&](auto&& fn) {
    for (int base = 0; base < nv; base += R1 * kTopkThreads) {
      uint4 w[R1];
#pragma unroll
      for (int r = 0; r < R1; ++r) w[r] = vp[min(base + r * kTopkThreads + tid, nv - 1)];
#pragma unroll
      for (int r = 0; r < R1; ++r) {
        const int vi = base + r * kTopkThreads + tid;
        if (vi >= nv) continue;
        const uint32_t q[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
#pragma unroll
        for (int e = 0; e < EPV; ++e)
          fn(BF16 ? ((e & 1) ? bf16hi(q[e >> 1]) : bf16lo(q[e >> 1])) : __uint_as_float(q[e]), vi * EPV + e);
      }
    }
    for (int i = nv * EPV + tid; i < V; i += kTopkThreads)
      fn(BF16 ? bf16_to_f32(((const uint16_t*)row)[i]) : ((const float*)row)[i], i);
  };

  // ---- pass 1: each thread's maximum, then the maxima of NG groups of 16
  // threads; the k-th largest of those NG entries bounds the row's k-th largest
  // value from below
  float tmax = -INFINITY;
  sweep([&](float x, int) { tmax = fmaxf(tmax, x); });
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o));
  if ((tid & 15) == 0) s_gmax[tid >> 4] = tmax;
  lds_sync();
  if (tid < NG) {
    const float mine = s_gmax[tid];
    int above = 0;  // group maxima ranked before mine: larger, or equal from a lower group
#pragma unroll
    for (int t = 0; t < NG; ++t) {
      const float o = s_gmax[t];
      above += o > mine || (o == mine && t < tid);
    }
    if (above == k - 1) s_thr = mine;
  }
  lds_sync();
  const float thr = s_thr;

  // ---- pass 2 (mostly cache hits): each thread's best 16 among entries >= thr
  float lv[kKeep];
  int li[kKeep];
#pragma unroll
  for (int s = 0; s < kKeep; ++s) lv[s] = -INFINITY, li[s] = INT_MAX;
  for (int base = 0; base < nv; base += R2 * kTopkThreads) {
    uint4 w[R2];
#pragma unroll
    for (int r = 0; r < R2; ++r) w[r] = vp[min(base + r * kTopkThreads + tid, nv - 1)];
#pragma unroll
    for (int r = 0; r < R2; ++r) {
      const int vi = base + r * kTopkThreads + tid;
      const uint32_t q[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
      float m;  // the vector's maximum: most vectors stop here
      if (BF16)
        m = fmaxf(fmaxf(fmaxf(bf16lo(q[0]), bf16hi(q[0])), fmaxf(bf16lo(q[1]), bf16hi(q[1]))),
                  fmaxf(fmaxf(bf16lo(q[2]), bf16hi(q[2])), fmaxf(bf16lo(q[3]), bf16hi(q[3]))));
      else
        m = fmaxf(fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1])), fmaxf(__uint_as_float(q[2]), __uint_as_float(q[3])));
      // a full list takes only values above its last entry (an equal value comes
      // with a larger index, so it ranks after it): such vectors are skipped whole
      const bool full = li[kKeep - 1] != INT_MAX;
      if (vi < nv && (full ? m > lv[kKeep - 1] : m >= thr)) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          const float x = BF16 ? ((e & 1) ? bf16hi(q[e >> 1]) : bf16lo(q[e >> 1])) : __uint_as_float(q[e]);
          if (x >= thr) keep_insert(lv, li, x, vi * EPV + e);
        }
      }
    }
  }
  for (int i = nv * EPV + tid; i < V; i += kTopkThreads) {  // unaligned rows and the tail
    const float x = BF16 ? bf16_to_f32(((const uint16_t*)row)[i]) : ((const float*)row)[i];
    if (x >= thr) keep_insert(lv, li, x, i);
  }

  // ---- k rounds: the best head among all threads; its owner drops it
  const int dp = depth[(size_t)b * n_max + p];
  const int u0 = nc + valid_before * k;
  for (int j = 0; j < k; ++j) {
    float bv = lv[0];
    int bi = li[0];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (before(ov, oi, bv, bi)) bv = ov, bi = oi;
    }
    if (lane == 0) sv[j & 1][wv] = bv, si[j & 1][wv] = bi;
    lds_sync();  // (the buffers alternate, so the next round's writes need no second barrier)
    float v = sv[j & 1][0];  // every thread takes the workgroup's winner itself
    int i = si[j & 1][0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
      if (before(sv[j & 1][w], si[j & 1][w], v, i)) v = sv[j & 1][w], i = si[j & 1][w];
    if (tid == 0) s_v[j] = v, s_i[j] = i;
    if (li[0] == i) {  // indices are unique, so exactly one thread owns the winner
#pragma unroll
      for (int s = 0; s < kKeep - 1; ++s) lv[s] = lv[s + 1], li[s] = li[s + 1];
      lv[kKeep - 1] = -INFINITY, li[kKeep - 1] = INT_MAX;
    }
  }
  lds_sync();
  if (tid < k) {
    const int u = u0 + tid;
    parent[(size_t)b * n_max + u] = p;
    depth[(size_t)b * n_max + u] = dp + 1;
    tokens[(size_t)b * n_max + u] = s_i[tid];
    if (scores) scores[(size_t)b * n_max + u] = s_v[tid];
  }
}

// One workgroup of 256 threads per sequence.
__global__ __launch_bounds__(256) void merge_kernel(int M, int Ld, int n_max, const int32_t* __restrict__ drafts,
                                                    const int32_t* __restrict__ draft_len,
                                                    const int32_t* __restrict__ root_token,
                                                    int32_t* __restrict__ parent, int32_t* __restrict__ depth,
                                                    int32_t* __restrict__ tokens, int32_t* __restrict__ n_out,
                                                    int32_t* __restrict__ node_of, int32_t* __restrict__ status) {
  __shared__ int len[TV_MERGE_MMAX];
  __shared__ int lcp[TV_MERGE_MMAX][TV_MERGE_MMAX];  // lcp[a][m] for a < m
  __shared__ int start[TV_MERGE_MMAX], base[TV_MERGE_MMAX];
  __shared__ int s_n;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int32_t* dr = drafts + (size_t)b * M * Ld;
  int bad = 0;
  if (tid < M) {
    len[tid] = draft_len[(size_t)b * M + tid];
    bad = len[tid] < 0 || len[tid] > Ld;
  }
  bad = __syncthreads_or(bad);
  if (!bad) {
    // common-prefix length of every pair of drafts (a < m)
    for (int pq = tid; pq < M * M; pq += 256) {
      const int a = pq / M, m = pq - a * M;
      if (a >= m) continue;
      const int lim = min(len[a], len[m]);
      int l = 0;
      while (l < lim && dr[(size_t)a * Ld + l] == dr[(size_t)m * Ld + l]) ++l;
      lcp[a][m] = l;
    }
    __syncthreads();
    if (tid < M) {  // draft m creates the nodes of its positions from its longest overlap on
      int s = 0;
      for (int a = 0; a < tid; ++a) s = max(s, lcp[a][tid]);
      start[tid] = s;
    }
    __syncthreads();
    if (tid == 0) {  // creation order: drafts in order, positions in order
      int acc = 1;
      for (int m = 0; m < M; ++m) {
        base[m] = acc;
        acc += len[m] - start[m];
      }
      s_n = acc;
    }
    __syncthreads();
    bad = s_n > n_max;
  }
  int32_t* par = parent + (size_t)b * n_max;
  int32_t* dep = depth + (size_t)b * n_max;
  int32_t* tok = tokens + (size_t)b * n_max;
  int32_t* nof = node_of ? node_of + (size_t)b * M * Ld : nullptr;
  const int n = bad ? 0 : s_n;
  for (int u = tid; u < n_max; u += 256) {
    if (u >= n) par[u] = -1, dep[u] = -1, tok[u] = -1;
  }
  if (tid == 0) {
    n_out[b] = n;
    status[b] = bad ? TV_EINVAL : TV_OK;
    if (!bad) {
      par[0] = -1, dep[0] = 0;
      tok[0] = root_token ? root_token[b] : 0;
    }
  }
  // node id of position d of draft m: created by the first draft sharing the prefix
  auto node = [&](int m, int d) {
    int a = 0;
    while (a < m && lcp[a][m] <= d) ++a;
    return base[a] + (d - start[a]);
  };
  for (int pos = tid; pos < M * Ld; pos += 256) {
    const int m = pos / Ld, d = pos - m * Ld;
    if (bad || d >= len[m]) {
      if (nof) nof[pos] = -1;
      continue;
    }
    const int u = node(m, d);
    if (nof) nof[pos] = u;
    if (d >= start[m]) {  // this draft created the node
      par[u] = d == 0 ? 0 : node(m, d - 1);
      dep[u] = d + 1;
      tok[u] = dr[(size_t)m * Ld + d];
    }
  }
}

}  // namespace

hipError_t launch_expand(int B, int F, int V, int k, int n_max, int bf16, const void* logits, const int32_t* frontier,
                         const int32_t* n_cur, int32_t* parent, int32_t* depth, int32_t* tokens, float* scores,
                         int32_t* n_out, int32_t* status, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (bf16)
    hipLaunchKernelGGL(topk_kernel<true>, dim3(B * F), dim3(kTopkThreads), 0, s, F, V, k, n_max, logits, frontier, n_cur,
                       parent, depth, tokens, scores, n_out, status);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3(B * F), dim3(kTopkThreads), 0, s, F, V, k, n_max, logits, frontier, n_cur,
                       parent, depth, tokens, scores, n_out, status);
  return hipGetLastError();
}

hipError_t launch_merge_drafts(int B, int M, int Ld, int n_max, const int32_t* drafts, const int32_t* draft_len,
                               const int32_t* root_token, int32_t* parent, int32_t* depth, int32_t* tokens,
                               int32_t* n_out, int32_t* node_of, int32_t* status, hipStream_t s) {
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3(B), dim3(256), 0, s, M, Ld, n_max, drafts, draft_len, root_token, parent,
                     depth, tokens, n_out, node_of, status);
  return hipGetLastError();
}

}  // namespace tv
