// Commit of the accepted root path's keys and values into the KV cache.
//
// After verification the accepted nodes are ordinary tokens of the sequence:
// node path[t] becomes cache position L_b + t, so the cache again holds one
// linear sequence and the next step attends it like any prefix (SpecInfer
// explainer, kernel-fusion section: depth-first order keeps the tree's KV
// consistent with the existing cache; "practical applications" section: the
// block-wise layout of PagedAttention, here 16-token blocks).
//
// It is a gather-scatter of at most n token rows of Hkv*D elements per K and V
// per sequence: a few MB per step, so a launch of one workgroup per (sequence,
// path position) with 16-byte vector copies, coalesced along each head row.
#include "tv_internal.h"

namespace tv {
namespace {

// grid: B*n workgroups, workgroup b*n + t copies path position t of sequence b.
// Every workgroup that writes first checks its sequence's whole contract (path
// length, node ids, capacity, block ids), so a rejected sequence is left
// untouched by all of them; workgroup t == 0 reports status and new length.
__global__ __launch_bounds__(256) void commit_kernel(int n, int Hkv, int row_shift, int paged, int Lmax,
                                                     int max_blocks, int num_blocks, uint4* __restrict__ kc,
                                                     uint4* __restrict__ vc, const int32_t* __restrict__ bt,
                                                     const int32_t* __restrict__ plen,
                                                     const uint4* __restrict__ kt, const uint4* __restrict__ vt,
                                                     const int32_t* __restrict__ path,
                                                     const int32_t* __restrict__ path_len,
                                                     int32_t* __restrict__ new_len, int32_t* __restrict__ status) {
  const int b = blockIdx.x / n, t = blockIdx.x - b * n;
  const int tid = threadIdx.x;
  const int L = plen[b];
  const int P = path_len[b];
  if (t != 0 && t >= P) return;  // nothing to write here (covers a P out of range too)
  const long long cap = paged ? (long long)max_blocks * TV_PAGE : Lmax;
  int bad = !(L >= 0 && P >= 0 && P <= n && (long long)L + P <= cap);
  const int32_t* pr = path + (size_t)b * n;
  if (!bad) {
    if (tid < P) bad = (unsigned)pr[tid] >= (unsigned)n;
    if (paged && P > 0) {
      const int first = L / TV_PAGE, nblk = (L + P - 1) / TV_PAGE - first + 1;  // <= 17
      if (tid < nblk) bad |= (unsigned)bt[(size_t)b * max_blocks + first + tid] >= (unsigned)num_blocks;
    }
  }
  bad = __syncthreads_or(bad);
  if (t == 0 && tid == 0) {
    if (status) status[b] = bad ? TV_EINVAL : TV_OK;
    new_len[b] = bad ? L : L + P;
  }
  if (bad || t >= P) return;

  const int u = pr[t];
  const int j = L + t;
  const int rowv = 1 << row_shift;  // 16-byte vectors per head row (D * element size / 16)
  // token j's row of head h sits at dst + h * hstride (in 16-byte vectors)
  size_t dst, hstride;
  if (paged) {
    const size_t blk = (size_t)bt[(size_t)b * max_blocks + j / TV_PAGE];
    dst = (blk * Hkv * TV_PAGE + (j % TV_PAGE)) * rowv;
    hstride = (size_t)TV_PAGE * rowv;
  } else {
    dst = ((size_t)b * Hkv * Lmax + j) * rowv;
    hstride = (size_t)Lmax * rowv;
  }
  const size_t src = ((size_t)b * n + u) * Hkv * rowv;  // tree rows [Hkv][D] of node u are contiguous
  const int total = Hkv << row_shift;
  for (int v = tid; v < total; v += 256) {
    const int h = v >> row_shift, c = v & (rowv - 1);
    const uint4 kx = kt[src + v];
    const uint4 vx = vt[src + v];
    const size_t o = dst + h * hstride + c;
    kc[o] = kx;
    vc[o] = vx;
  }
}

}  // namespace

hipError_t launch_commit(const tv_attn_desc* d, void* kc, void* vc, const int32_t* bt, const int32_t* plen,
                         const void* kt, const void* vt, const int32_t* path, const int32_t* path_len,
                         int32_t* new_len, int32_t* status, hipStream_t s) {
  if (d->B == 0) return hipSuccess;
  const int es = d->dtype == TV_F32 ? 4 : 2;
  const int rowv = d->D * es / 16;  // 8, 16 or 32
  const int row_shift = __builtin_ctz(rowv);
  hipLaunchKernelGGL(commit_kernel, dim3(d->B * d->n), dim3(256), 0, s, d->n, d->Hkv, row_shift, d->paged,
                     d->Lmax, d->max_blocks, d->num_blocks, (uint4*)kc, (uint4*)vc, bt, plen, (const uint4*)kt,
                     (const uint4*)vt, path, path_len, new_len, status);
  return hipGetLastError();
}

}  // namespace tv
