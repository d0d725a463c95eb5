// Stochastic tree verification: multi-step speculative sampling over the tree.
//
// SpecInfer explainer, tree-verification section: a child's draft token x is
// accepted with probability min(1, P_LLM(x) / P_SSM(x)); after a rejection the
// LLM distribution is replaced by the normalised residual max(0, P_LLM - P_SSM),
// and the scheme then samples exactly from the LLM's distribution.  At the
// current node the children are tried in node-id order, each against the
// residual left by its rejected elder siblings; an accepted child becomes the
// current node; when all are rejected (or there are none) one token is drawn
// from the current distribution by inverse CDF.  The uniforms are inputs.
//
// The walk is sequential per sequence and touches only the rows of the nodes it
// visits.  It runs as one 512-thread workgroup per sequence that streams just
// those vocab rows (the rows of a node already visited stay in L2/MALL), or,
// sliced, as up to 16 workgroups of 256 threads per sequence, each streaming its
// own range of chunks of those rows and exchanging per-slice statistics at each
// step of the walk:
//   node entry     one pass: online (max, sum) of the node's LLM logits and of
//                  its first child's SSM logits
//   child test     scalar loads of the two logits at the draft token
//   rejection      one pass writing the residual r = max(0, p - q) to an fp32
//                  workspace row (and its sum), fused with the next child's
//                  SSM statistics; the next child's p(x) is caught in LDS by the
//                  thread that owns x
//   final draw     one pass of per-segment sums (512 elements per segment),
//                  a prefix over segments in fp64 by one wave, and a scan
//                  inside the chosen segment
// Element e of a row belongs to thread (e % chunk) / 8 of the workgroup owning
// its chunk in every pass, so a thread only ever reads back residual values it
// wrote itself.
#include <limits.h>

#include <atomic>

#include "tv_internal.h"

namespace tv {
namespace {

constexpr int kThreads = 512;             // one workgroup per sequence
constexpr int kThreadsSliced = 256;        // several per sequence: three fit on a CU
constexpr int kEPT = 8;                      // elements per thread per chunk
constexpr int kChunk = kThreads * kEPT;      // 4096 (the workspace's row padding)
constexpr int kSeg = 64 * kEPT;              // 512 elements: one wave's share of a chunk
constexpr int kMaxSeg = TV_MSS_VMAX / kSeg;  // 2048
constexpr int kMaxNS = 16;                   // vocabulary slices per sequence (sliced walk)
constexpr int kXRec = 8;                     // doubles per exchange record
constexpr int kSpinMax = 1 << 18;            // default: polls before a slice gives up on its peers
// A pass over a row visits chunks in groups of kU whose loads are all issued
// before any of them is used, so a workgroup keeps kU chunks of each row in
// flight instead of waiting out one memory latency per chunk.  The sliced walk
// takes groups of 6 (bf16): a slice of workload-sized rows is then one group,
// within the register budget of three workgroups per compute unit.
template <bool BF16>
constexpr int kGroup = BF16 ? 8 : 4;
template <bool BF16>
constexpr int kGroupSliced = BF16 ? 6 : 3;

template <bool BF16>
__device__ __forceinline__ void load8(const void* row, int e0, int V, bool vec, float (&v)[kEPT]) {
  if (BF16) {
    const uint16_t* r = (const uint16_t*)row;
    if (vec && e0 + kEPT <= V) {
      const uint4 w = *(const uint4*)(r + e0);
      v[0] = bf16lo(w.x), v[1] = bf16hi(w.x), v[2] = bf16lo(w.y), v[3] = bf16hi(w.y);
      v[4] = bf16lo(w.z), v[5] = bf16hi(w.z), v[6] = bf16lo(w.w), v[7] = bf16hi(w.w);
    } else {
#pragma unroll
      for (int j = 0; j < kEPT; ++j) v[j] = e0 + j < V ? bf16_to_f32(r[e0 + j]) : -INFINITY;
    }
  } else {
    const float* r = (const float*)row;
    if (vec && e0 + kEPT <= V) {
      const float4 a = *(const float4*)(r + e0);
      const float4 b = *(const float4*)(r + e0 + 4);
      v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < kEPT; ++j) v[j] = e0 + j < V ? r[e0 + j] : -INFINITY;
    }
  }
}

// Eight elements known to lie inside the row, loaded as raw 16-byte words and
// unpacked only when used, so a group of chunks in flight costs 4 VGPRs per
// chunk for bf16 rows (8 for fp32).
template <bool BF16>
struct Raw {
  uint4 w[BF16 ? 1 : 2];
  __device__ __forceinline__ void load(const void* row, int e0) {
    const uint4* p = (const uint4*)((const char*)row + (size_t)e0 * (BF16 ? 2 : 4));
    w[0] = p[0];
    if (!BF16) w[1] = p[1];
  }
  __device__ __forceinline__ void unpack(float (&v)[kEPT]) const {
    if (BF16) {
      v[0] = bf16lo(w[0].x), v[1] = bf16hi(w[0].x), v[2] = bf16lo(w[0].y), v[3] = bf16hi(w[0].y);
      v[4] = bf16lo(w[0].z), v[5] = bf16hi(w[0].z), v[6] = bf16lo(w[0].w), v[7] = bf16hi(w[0].w);
    } else {
      v[0] = __uint_as_float(w[0].x), v[1] = __uint_as_float(w[0].y), v[2] = __uint_as_float(w[0].z);
      v[3] = __uint_as_float(w[0].w), v[4] = __uint_as_float(w[1].x), v[5] = __uint_as_float(w[1].y);
      v[6] = __uint_as_float(w[1].z), v[7] = __uint_as_float(w[1].w);
    }
  }
};

template <bool BF16>
__device__ __forceinline__ float load1(const void* row, int x) {
  return BF16 ? bf16_to_f32(((const uint16_t*)row)[x]) : ((const float*)row)[x];
}
// The same as raw bits, decoded by use1 where the value is needed: a load issued
// early then waits there, not right after its issue.
template <bool BF16>
__device__ __forceinline__ uint32_t load1raw(const void* row, int x) {
  return BF16 ? (uint32_t)((const uint16_t*)row)[x] : ((const uint32_t*)row)[x];
}
template <bool BF16>
__device__ __forceinline__ float use1(uint32_t raw) {
  asm volatile("" : "+v"(raw));  // the decode stays here
  return BF16 ? bf16_to_f32((uint16_t)raw) : __uint_as_float(raw);
}

// exp(v - r / log2(e)) as exp2(v * log2(e) - r): one FMA and the hardware exp2;
// the FMA rounds the argument once, so a value carries about 1e-7 relative error.
__device__ __forceinline__ float ex(float v, float nr) { return __builtin_amdgcn_exp2f(fmaf(v, kLog2e, nr)); }

__device__ __forceinline__ float max8(const float (&v)[kEPT]) {
  float m = v[0];
#pragma unroll
  for (int j = 1; j < kEPT; ++j) m = fmaxf(m, v[j]);
  return m;
}

// Softmax statistics of a row, gathered in one pass: the terms exp2(v*log2(e) - R)
// summed in fp64, with R a whole number at least max(v)*log2(e), so no term
// exceeds 1.  R only ever moves by whole numbers and the sum follows it by
// ldexp, which is exact: the online pass adds no rounding beyond the terms' own,
// and p(v) = exp2(v*log2(e) - R) / S.
struct Stat {
  float R = -INFINITY;
  double S = 0.0;
};

__device__ __forceinline__ double shift(double s, float from, float to) {  // s * 2^(from - to), to >= from
  return ldexp(s, (int)fmaxf(from - to, -2000.f));
}

__device__ __forceinline__ void stat_add8(Stat& st, const float (&v)[kEPT]) {
  const float cm = max8(v);
  if (cm == -INFINITY) return;
  const float r = ceilf(cm * kLog2e);
  if (r > st.R) {
    st.S = st.R == -INFINITY ? 0.0 : shift(st.S, st.R, r);
    st.R = r;
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kEPT; ++j) s += ex(v[j], -st.R);
  st.S += (double)s;
}

// The same statistics over a group of chunks already in registers: the group's
// largest value first, so the reference moves at most once per group, then per
// chunk one fp32 sum of its eight terms, added in fp64.  Chunks u >= nv lie past
// the end of the range (a partial last group) and are skipped.
template <bool BF16, int G>
__device__ __forceinline__ void stat_add_group(Stat& st, const Raw<BF16> (&q)[G], int nv) {
  float cm = -INFINITY;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    if (u >= nv) break;
    float v[kEPT];
    q[u].unpack(v);
    cm = fmaxf(cm, max8(v));
  }
  if (cm == -INFINITY) return;
  const float r = ceilf(cm * kLog2e);
  if (r > st.R) {
    st.S = st.R == -INFINITY ? 0.0 : shift(st.S, st.R, r);
    st.R = r;
  }
#pragma unroll
  for (int u = 0; u < G; ++u) {
    if (u >= nv) break;
    float v[kEPT];
    q[u].unpack(v);
    float sm = ex(v[0], -st.R);
#pragma unroll
    for (int j = 1; j < kEPT; ++j) sm += ex(v[j], -st.R);
    st.S += (double)sm;
  }
}

__device__ __forceinline__ void stat_merge(Stat& a, float R, double S) {
  if (R == -INFINITY) return;
  if (a.R == -INFINITY) {
    a.R = R, a.S = S;
    return;
  }
  const float M = fmaxf(a.R, R);
  a.S = shift(a.S, a.R, M) + shift(S, R, M);
  a.R = M;
}

template <int NW>
struct Shared {
  int par[TV_NMAX];
  int tok[TV_NMAX];
  float uacc[TV_NMAX];
  int child[TV_NMAX];
  int path[TV_NMAX];
  unsigned long long ball[4];
  float rR[2][2][NW];
  double rS[2][3][NW];
  float cap_prev[2], cap_r[2];  // by pass parity: a pass never overwrites what the last one caught
  double segd[kMaxSeg];
  double xr[kMaxNS][kXRec];     // the slices' exchange records, in slice order
  double xtot;
  int wok[NW];  // each wave's exchange status
  int result;
};

// Cross-lane reductions: DPP steps within each row of 16 lanes; since every step
// combines a lane's own value with its partner's by a commutative operation, all
// 16 lanes of a row hold the same bits.  The four rows' results are then read from
// lanes 0, 16, 32, 48 and combined in that fixed order, uniformly.  Called with
// every lane of the wave active (the walk's reductions are workgroup-uniform).
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  return fmaxf(x, dpp<kDppMirror>(x));
}
__device__ __forceinline__ double row_sum(double x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x + dpp<kDppMirror>(x);
}
__device__ __forceinline__ float wave_max(float x) {
  x = row_max(x);
  return fmaxf(fmaxf(lane_read(x, 0), lane_read(x, 16)), fmaxf(lane_read(x, 32), lane_read(x, 48)));
}
__device__ __forceinline__ double wave_sum(double x) {
  x = row_sum(x);
  return (lane_read(x, 0) + lane_read(x, 16)) + (lane_read(x, 32) + lane_read(x, 48));
}
// a wave's statistics: the largest reference, every lane's sum moved onto it
// (exactly), then one plain fp64 sum
__device__ __forceinline__ Stat wave_stat(Stat a) {
  const float R = wave_max(a.R);
  const double s = a.R == -INFINITY ? 0.0 : shift(a.S, a.R, R);
  return Stat{R, wave_sum(s)};
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads also waits for
// every outstanding global store (the residual row a pass has just written);
// nothing after these barriers reads another wave's global stores before the
// draw pass, whose full barrier waits for them, since a thread only reads back
// residual values it wrote itself.  So the stores drain while the reduction
// and the exchange go on.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The merge of NW entries (R_k, S_k) held in LDS: every entry read at once, the
// largest reference, each sum moved onto it (exactly: a power-of-two scale), and
// one fp64 sum in entry order.  Equal, bit for bit, to merging them one by one,
// since a power-of-two scale of a rounded sum is exact.
template <int NW>
__device__ __forceinline__ Stat merge_entries(const float (&R)[NW], const double (&Sv)[NW]) {
  float r[NW];
  double sv[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) r[k] = R[k], sv[k] = Sv[k];
  float M = r[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) M = fmaxf(M, r[k]);
  double t = 0.0;
#pragma unroll
  for (int k = 0; k < NW; ++k) t += r[k] == -INFINITY ? 0.0 : shift(sv[k], r[k], M);
  return Stat{M, t};
}

// Workgroup-wide merge of one or (TWO) two row statistics and one plain fp64 sum
// per thread.  Every thread ends with the same values, merged in the same order
// from LDS.  One barrier; alternating LDS slots so back-to-back calls never
// overwrite values another wave is still reading.
template <int NW, bool TWO>
__device__ __forceinline__ void block_reduce(Shared<NW>& S, int& slot, Stat& a, Stat& b, double& t) {
  const Stat wa = wave_stat(a);
  Stat wb;
  if constexpr (TWO) wb = wave_stat(b);
  const double wt = wave_sum(t);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    S.rR[slot][0][w] = wa.R, S.rS[slot][0][w] = wa.S;
    if constexpr (TWO) S.rR[slot][1][w] = wb.R, S.rS[slot][1][w] = wb.S;
    S.rS[slot][2][w] = wt;
  }
  lds_sync();
  a = merge_entries<NW>(S.rR[slot][0], S.rS[slot][0]);
  if constexpr (TWO) b = merge_entries<NW>(S.rR[slot][1], S.rS[slot][1]);
  t = 0.0;
#pragma unroll
  for (int k = 0; k < NW; ++k) t += S.rS[slot][2][k];
  slot ^= 1;
}

// Exchange between the NS slices (workgroups) of one sequence's walk: each
// publishes its record for reduction r and reads every slice's record; all
// slices then merge the NS records in slice order, so they take the same
// decisions.
//   - A record is kXRec doubles as 2 * kXRec 64-bit words: the low 32 bits carry
//     half of a value, the high 32 bits the tag r + 1.  Words are written and
//     read with relaxed device-scope atomics (coherent across the XCDs' caches,
//     no cache flush, each word single-copy atomic), so a reader that sees tag
//     r + 1 in both words of a value has that value of reduction r.  No counter
//     and no wait for the writes: a reader polls the words themselves.
//   - Two record slots alternate (tags r + 1 and r + 3 differ): a slice writes
//     slot r & 1 again only at r + 2, after it has read every slice's record of
//     r + 1, which each slice wrote after reading reduction r.  The tags start at
//     0 (cleared before the walk by mss_clear_kernel, or by the statistics pass
//     in the all-row mode), so a record of an earlier call is never taken.
//   - The wait is bounded: after `spin` polls of a word (kSpinMax unless the
//     host set another limit) the slice gives up and
//     the caller ends the walk with an error, so every workgroup exits.
// The first 2 kXRec threads write the slice's record (thread j word j); then every
// thread takes up to 2 kXRec * NS / NTH of the words (one, with 256 threads and
// up to 16 slices), so all of them are polled at once: its own slice's words come
// straight from registers.  Returns false (uniformly) on a timeout.
constexpr int kXW = 2 * kXRec;  // 64-bit words per record
template <int NW>
__device__ __forceinline__ bool exchange(Shared<NW>& S, const double (&mine)[kXRec], uint64_t* rec, int NS, int s,
                                         int r, int spin) {
  const int t = threadIdx.x;
  uint64_t* slot = rec + (size_t)(r & 1) * NS * kXW;
  const uint32_t tag = (uint32_t)(r + 1);
  auto own_word = [&](int j) -> uint32_t {  // half (j & 1) of value j / 2 (no dynamic index into mine)
    uint32_t h = 0;
#pragma unroll
    for (int i = 0; i < kXRec; ++i) {
      const uint64_t bits = __builtin_bit_cast(uint64_t, mine[i]);
      h = (j >> 1) == i ? ((j & 1) ? (uint32_t)(bits >> 32) : (uint32_t)bits) : h;
    }
    return h;
  };
  if (t < kXW)
    __hip_atomic_store(slot + s * kXW + t, ((uint64_t)tag << 32) | own_word(t), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  int ok = 1;
  for (int idx = t; idx < NS * kXW; idx += NW * 64) {
    uint32_t v;
    if (idx / kXW == s) {
      v = own_word(idx % kXW);
    } else {
      uint64_t w = 0;
      int it = 0;
      for (; it < spin; ++it) {
        w = __hip_atomic_load(slot + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(w >> 32) == tag) break;
        __builtin_amdgcn_s_sleep(1);
      }
      ok &= it < spin;
      v = (uint32_t)w;
    }
    ((uint32_t*)&S.xr[0][0])[idx] = v;  // word t*2*kXRec + j: half (j & 1) of value j/2 of slice t
  }
  ok = __all(ok);
  if ((t & 63) == 0) S.wok[t >> 6] = ok;
  lds_sync();
  int all = 1;
#pragma unroll
  for (int w = 0; w < NW; ++w) all &= S.wok[w];
  return all != 0;
}

// Combining the slices' records: lane t of every wave takes slice t's entry (at
// most 16 slices, so all in the first row of 16 lanes); the largest reference,
// every entry moved onto it exactly, and one sum, all with row-wide DPP
// reductions; every lane then takes lane 0's result, so all threads of all
// slices hold the same value (the same data, combined in the same fixed order).
__device__ __forceinline__ Stat row_stat(Stat a) {
  const float R = row_max(a.R);
  const double s = a.R == -INFINITY ? 0.0 : shift(a.S, a.R, R);
  return Stat{lane_read(R, 0), lane_read(row_sum(s), 0)};
}
template <int NW>
__device__ __forceinline__ Stat xmerge_stat(const Shared<NW>& S, int NS, int iR, int iS) {
  const int lane = threadIdx.x & 63;
  Stat a;
  if (lane < NS) a = Stat{(float)S.xr[lane][iR], S.xr[lane][iS]};
  return row_stat(a);
}
// Two statistics (records' entries iR0/iS0 and iR1/iS1) side by side, so their
// reductions overlap.
template <int NW>
__device__ __forceinline__ void xmerge_stat2(const Shared<NW>& S, int NS, int iR0, int iS0, int iR1, int iS1,
                                             Stat& a, Stat& c) {
  const int lane = threadIdx.x & 63;
  a = Stat{}, c = Stat{};
  if (lane < NS) a = Stat{(float)S.xr[lane][iR0], S.xr[lane][iS0]}, c = Stat{(float)S.xr[lane][iR1], S.xr[lane][iS1]};
  a = row_stat(a);
  c = row_stat(c);
}
template <int NW>
__device__ __forceinline__ double xsum(const Shared<NW>& S, int NS, int i) {
  const int lane = threadIdx.x & 63;
  return lane_read(row_sum(lane < NS ? S.xr[lane][i] : 0.0), 0);
}

template <bool B>  // a compile-time flag as a type (selects a specialised pass)
struct BoolC {
  static constexpr bool value = B;
};

// One chunk of a residual pass: p (from raw logits via max/normaliser, or from
// the previous unnormalised residual via its sum), minus q from its logits;
// writes r = max(0, p - q) to the output row, catches p and r at the next
// child's token, returns the chunk's sum of r.
struct Resid {
  float nm;   // -R of the LLM row's statistics
  float sp_hi, sp_lo;  // scale of p (1/S or 1/T) as a two-float sum
  float nmq;  // -R of the SSM row's
  float sq_hi, sq_lo;  // 1/S of the SSM row likewise
  float* rout;
  int xn;
  float* cap_prev;
  float* cap_r;
  template <bool FL>  // p from raw logits (else from the residual row)
  __device__ __forceinline__ float chunk(int e0, float (&pv)[kEPT], const float (&qv)[kEPT]) const {
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
      const float e = FL ? ex(pv[j], nm) : pv[j];
      pv[j] = fmaf(e, sp_hi, e * sp_lo);
    }
    float r[kEPT];
    float sm = 0.f;
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
      const float e = ex(qv[j], nmq);
      r[j] = fmaxf(0.f, pv[j] - fmaf(e, sq_hi, e * sq_lo));
      sm += r[j];
    }
    *(float4*)(rout + e0) = make_float4(r[0], r[1], r[2], r[3]);
    *(float4*)(rout + e0 + 4) = make_float4(r[4], r[5], r[6], r[7]);
    if ((unsigned)(xn - e0) < (unsigned)kEPT) {
      const int j = xn - e0;
      float pj = pv[0], rj = r[0];
#pragma unroll
      for (int jj = 1; jj < kEPT; ++jj) {
        pj = jj == j ? pv[jj] : pj;
        rj = jj == j ? r[jj] : rj;
      }
      *cap_prev = pj;
      *cap_r = rj;
    }
    return sm;
  }
};

// a double as hi + lo floats (the product e * hi + e * lo then rounds once per
// element instead of carrying one shared rounding of the scale)
__device__ __forceinline__ void split2(double d, float& hi, float& lo) {
  hi = (float)d;
  lo = (float)(d - (double)hi);
}

// fp64 sum of one wave's 512 values of a chunk into its segment slot
template <int NW>
__device__ __forceinline__ void seg_store(Shared<NW>& S, int ch, const float (&v)[kEPT]) {
  double sd = 0.0;
#pragma unroll
  for (int j = 0; j < kEPT; ++j) sd += (double)v[j];
  sd = wave_sum(sd);
  if ((threadIdx.x & 63) == 0) S.segd[ch * NW + (threadIdx.x >> 6)] = sd;
}

// Precomputed statistics of one row (the second mode: every LLM and SSM row's
// statistics first, in a fully parallel kernel, so the walk needs no entry pass).
struct StatRec {
  float R;
  float pad;
  double S;
};

// One 256-thread workgroup per row: row r of the grid is (sequence, node, which)
// with which 0 = the LLM row, 1 = the SSM row (node 0 has none).  Same exact
// online statistics as the walk's own passes.  Before a sliced walk (xrec set)
// it also does what mss_clear_kernel does, one word per thread (the grid has
// B * n * 512 threads, the exchange area B * 512 words).
constexpr int kXWords = 2 * kMaxNS * 2 * kXRec;  // exchange words per sequence
template <bool BF16>
__global__ __launch_bounds__(256) void row_stats_kernel(int n, int V, int vec, const void* __restrict__ logits,
                                                        const void* __restrict__ ssm, StatRec* __restrict__ out,
                                                        int B, uint64_t* __restrict__ xrec,
                                                        int32_t* __restrict__ status) {
  __shared__ float sR[4];
  __shared__ double sS[4];
  const int r = blockIdx.x, which = r & 1, node = (r >> 1) % n, b = (r >> 1) / n;
  const int tid = threadIdx.x;
  if (xrec != nullptr) {
    const size_t i = (size_t)r * 256 + tid;
    if (i < (size_t)B * kXWords) xrec[i] = 0ull;
    if (i < (size_t)B) status[i] = TV_OK;
  }
  if (which == 1 && node == 0) return;
  const size_t es = BF16 ? 2 : 4;
  const char* row = (const char*)(which ? ssm : logits) + ((size_t)b * n + node) * V * es;
  constexpr int kC = 256 * kEPT;  // elements per chunk of this kernel
  const int nch = (V + kC - 1) / kC, nfull = vec ? V / kC : 0;
  Stat st;
  int c = 0;
  // full chunks in groups of kG, every load of a group in flight before any is
  // used; a last, partial group loads in-range chunks in the missing places and
  // skips them, so a row is a few rounds of loads, not one per chunk
  constexpr int kG = BF16 ? 8 : 4;
  for (; c < nfull; c += kG) {
    Raw<BF16> q[kG];
#pragma unroll
    for (int u = 0; u < kG; ++u) q[u].load(row, min(c + u, nfull - 1) * kC + tid * kEPT);
    stat_add_group<BF16, kG>(st, q, nfull - c);
  }
  for (c = nfull; c < nch; ++c) {
    float v[kEPT];
    load8<BF16>(row, c * kC + tid * kEPT, V, vec, v);
    stat_add8(st, v);
  }
  const Stat w = wave_stat(st);
  if ((tid & 63) == 0) sR[tid >> 6] = w.R, sS[tid >> 6] = w.S;
  __syncthreads();
  if (tid == 0) {
    Stat t;
    for (int k = 0; k < 4; ++k) stat_merge(t, sR[k], sS[k]);
    out[r] = StatRec{t.R, 0.f, t.S};
  }
}

// Before a sliced walk: every exchange word's tag at 0 and every status at TV_OK
// (a slice that gives up raises it to TV_EHIP with an atomic max).
__global__ __launch_bounds__(256) void mss_clear_kernel(int B, uint64_t* __restrict__ xrec,
                                                        int32_t* __restrict__ status) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < (size_t)B * kXWords) xrec[i] = 0ull;
  if (i < (size_t)B) status[i] = TV_OK;
}

// The walk of one sequence.  NS == 1: one workgroup per sequence (grid B),
// everything below without exchanges.  NS > 1: NS workgroups per sequence, each
// owning a contiguous range of chunks of every row (its vocabulary slice); the
// row statistics, residual sums, caught values and the draw's slice totals
// are exchanged at each reduction (see exchange), and the slice holding the
// drawn token writes the outputs.
// Sliced walk (256 threads): three waves per SIMD at least (the register budget
// that lets three of its workgroups share a CU), so its grid of up to 768
// workgroups is resident at once and no slice waits on a peer that cannot start.
// (Three per unit measured faster than two, with 11 instead of 8 slices per
// sequence on 64 sequences, and than four, whose budget spills.)
template <bool BF16, int NTH>
__global__ __launch_bounds__(NTH, NTH == kThreadsSliced ? 3 : 1) void mss_kernel(int n, int V, int vec, const void* __restrict__ logits,
                                                  const void* __restrict__ ssm, const int32_t* __restrict__ tokens,
                                                  const int32_t* __restrict__ parent,
                                                  const float* __restrict__ u_acc, const float* __restrict__ u_smp,
                                                  float* __restrict__ ws, int Vpad, const StatRec* __restrict__ pre,
                                                  int NS, uint64_t* __restrict__ xrec, int spin,
                                                  int32_t* __restrict__ path_out, int32_t* __restrict__ plen_out,
                                                  int32_t* __restrict__ bonus, int32_t* __restrict__ status) {
  constexpr int NW = NTH / 64;
  constexpr int CH = NTH * kEPT;  // elements per chunk
  __shared__ Shared<NW> S;
  // sequence b, slice s; with NS > 1 consecutive logical ids (a sequence's
  // slices) are placed on one XCD, so their exchanges stay close
  int b = blockIdx.x, s = 0;
  if (NS > 1) {
    const int nwg = gridDim.x, wg = blockIdx.x;
    const int perx = nwg >> 3, rem = nwg & 7, xcd = wg & 7;
    const int lid = xcd * perx + min(xcd, rem) + (wg >> 3);
    b = lid / NS;
    s = lid % NS;
  }
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const size_t es = BF16 ? 2 : 4;
  const char* lbase = (const char*)logits + (size_t)b * n * V * es;
  const char* sbase = (const char*)ssm + (size_t)b * n * V * es;
  float* const rbase = ws + (size_t)b * 2 * Vpad;  // two residual rows: rbase + ib * Vpad
  const int nch = (V + CH - 1) / CH;
  const int nfull = vec ? V / CH : 0;  // chunks wholly inside the row, read with vector loads
  const int cps = (nch + NS - 1) / NS;
  const int c0 = min(nch, s * cps), c1 = min(nch, c0 + cps);  // this slice's chunks
  const int cf = min(c1, nfull);
  uint64_t* const rec = NS > 1 ? xrec + (size_t)b * 2 * NS * kXW : nullptr;
  int xr = 0;  // exchanges so far
  constexpr int kU = NTH == kThreadsSliced ? kGroupSliced<BF16> : kGroup<BF16>;
  int32_t* pr = path_out + (size_t)b * n;

  // ---- load and check the tree: parents before children, tokens inside the vocabulary
  int bad = 0;
  if (tid < n) {
    const int p = parent[(size_t)b * n + tid];
    const int t = tokens[(size_t)b * n + tid];
    S.par[tid] = p;
    S.tok[tid] = t;
    S.uacc[tid] = u_acc[(size_t)b * n + tid];
    bad = tid == 0 ? p != -1 : (p < 0 || p >= tid || t < 0 || t >= V);
  }
  bad = __syncthreads_or(bad);
  if (bad) {  // every slice sees the same tree and writes the same values
    if (tid < n) pr[tid] = -1;
    if (tid == 0) {
      plen_out[b] = 0;
      bonus[b] = -1;
      if (status) status[b] = TV_EINVAL;
    }
    return;
  }
  // a slice that gave up on its peers: the sequence's status goes to TV_EHIP
  // (outputs then unspecified) and the walk ends
  auto give_up = [&]() {
    if (tid == 0) atomicMax(status + b, TV_EHIP);
  };

  int slot = 0;
  int cur = 0, len = 1;
  if (tid == 0) S.path[0] = 0;
  for (;;) {
    // ---- children of cur in node-id order (ballot over node ids)
    // (each child writes itself at its rank: the children of lower waves, then
    // those of lower lanes in its own wave)
    const bool isc = tid < n && tid > cur && S.par[tid] == cur;
    const unsigned long long bl = __ballot(isc);
    if (tid < 256 && lane == 0) S.ball[wv] = bl;
    lds_sync();  // LDS only: residual stores of the last node may still drain
    int k = 0, below = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int cnt = __builtin_popcountll(S.ball[w]);
      below += w < wv ? cnt : 0;
      k += cnt;
    }
    if (isc) S.child[below + __builtin_popcountll(bl & ((1ull << lane) - 1))] = tid;
    lds_sync();  // S.child visible
    const char* lrow = lbase + (size_t)cur * V * es;
    const int c1st = k > 0 ? S.child[0] : -1;
    const char* srow = c1st >= 0 && !pre ? sbase + (size_t)c1st * V * es : nullptr;
    // the two logits the first child's acceptance test reads, loaded now so their
    // latency hides behind the entry pass (the next child's, behind each residual pass)
    uint32_t lx = 0, qxl = 0;
    if (c1st >= 0) {
      const int x0 = S.tok[c1st];
      lx = load1raw<BF16>(lrow, x0);
      qxl = load1raw<BF16>(sbase + (size_t)c1st * V * es, x0);
    }

    // ---- node entry: statistics of the LLM row and the first child's SSM row,
    // precomputed or in one pass (over this slice, then exchanged)
    Stat sl, sq;
    if (pre) {
      const StatRec a = pre[((size_t)b * n + cur) * 2];
      sl = Stat{a.R, a.S};
      if (c1st >= 0) {
        const StatRec q = pre[((size_t)b * n + c1st) * 2 + 1];
        sq = Stat{q.R, q.S};
      }
    } else {
      // full chunks in groups of kU, every load of a group in flight before any
      // is used; a last, partial group loads in-range chunks in the missing
      // places and skips them (the group bound is uniform)
      int c = c0;
      for (; c < cf; c += kU) {
        Raw<BF16> a[kU], q[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) a[u].load(lrow, min(c + u, cf - 1) * CH + tid * kEPT);
        if (srow) {
#pragma unroll
          for (int u = 0; u < kU; ++u) q[u].load(srow, min(c + u, cf - 1) * CH + tid * kEPT);
          stat_add_group<BF16, kU>(sq, q, cf - c);
        }
        stat_add_group<BF16, kU>(sl, a, cf - c);
      }
      c = max(c0, cf);
      for (; c < c1; ++c) {
        const int e0 = c * CH + tid * kEPT;
        float v[kEPT];
        load8<BF16>(lrow, e0, V, vec, v);
        stat_add8(sl, v);
        if (srow) {
          load8<BF16>(srow, e0, V, vec, v);
          stat_add8(sq, v);
        }
      }
      double unused = 0.0;
      block_reduce<NW, true>(S, slot, sl, sq, unused);
      if (NS > 1) {
        const double mine[kXRec] = {sl.R, sl.S, sq.R, sq.S, 0.0, 0.0, 0.0, 0.0};
        if (!exchange<NW>(S, mine, rec, NS, s, xr++, spin)) return give_up();
        xmerge_stat2(S, NS, 0, 1, 2, 3, sl, sq);
      }
    }

    // ---- children in order
    bool from_logits = true;  // the current distribution is softmax of lrow (else rb[ib] / T)
    int ib = 0;
    double T = 1.0;
    double pnext = 0.0;  // p at the next child's token, when not from logits
    int accepted = -1;
    for (int i = 0; i < k; ++i) {
      const int c = S.child[i];
      const char* crow = sbase + (size_t)c * V * es;
      const double px = from_logits ? (double)ex(use1<BF16>(lx), -sl.R) / sl.S : pnext;
      const double qx = (double)ex(use1<BF16>(qxl), -sq.R) / sq.S;
      if ((double)S.uacc[c] * qx < px) {
        accepted = c;
        break;
      }
      // rejected: residual r = max(0, p - q_c) into the other workspace row, its
      // sum, and the next child's SSM maximum
      const int cn = i + 1 < k ? S.child[i + 1] : -1;
      const char* nrow = cn >= 0 && !pre ? sbase + (size_t)cn * V * es : nullptr;
      const int xn = cn >= 0 ? S.tok[cn] : -1;
      if (cn >= 0) {  // the next test's SSM logit (its p comes from the residual pass)
        qxl = load1raw<BF16>(sbase + (size_t)cn * V * es, xn);
        lx = load1raw<BF16>(lrow, xn);
      }
      const float* rin = rbase + (size_t)ib * Vpad;
      float* rout = rbase + (size_t)(ib ^ 1) * Vpad;
      Resid R{-sl.R, 0.f, 0.f, -sq.R, 0.f, 0.f, rout, xn, S.cap_prev + (i & 1), S.cap_r + (i & 1)};
      split2(from_logits ? 1.0 / sl.S : 1.0 / T, R.sp_hi, R.sp_lo);
      split2(1.0 / sq.S, R.sq_hi, R.sq_lo);
      double tsum = 0.0;
      Stat sn, unused;  // the next child's SSM row
      // the pass, specialised on where p comes from (raw logits or the residual row)
      auto resid_pass = [&](auto fl) {
        constexpr bool FL = decltype(fl)::value;
        using PRaw = Raw<FL ? BF16 : false>;
        const void* prow = FL ? (const void*)lrow : (const void*)rin;
        int ch = c0;
        // three rows in flight here, so a smaller group for one workgroup per
        // sequence; the sliced walk keeps its group (a slice's chunks at once)
        constexpr int kR = NTH == kThreadsSliced ? kGroupSliced<BF16> : (BF16 ? 4 : 2);
        for (; ch < cf; ch += kR) {  // partial last group as in the entry pass
          PRaw pq[kR];  // the current distribution: raw logits or residual
          Raw<BF16> qq[kR], nq[kR];
#pragma unroll
          for (int u = 0; u < kR; ++u) pq[u].load(prow, min(ch + u, cf - 1) * CH + tid * kEPT);
#pragma unroll
          for (int u = 0; u < kR; ++u) qq[u].load(crow, min(ch + u, cf - 1) * CH + tid * kEPT);
          if (nrow) {
#pragma unroll
            for (int u = 0; u < kR; ++u) nq[u].load(nrow, min(ch + u, cf - 1) * CH + tid * kEPT);
            stat_add_group<BF16, kR>(sn, nq, cf - ch);
          }
#pragma unroll
          for (int u = 0; u < kR; ++u) {
            if (ch + u >= cf) break;
            float pv[kEPT], qv[kEPT];
            pq[u].unpack(pv);
            qq[u].unpack(qv);
            tsum += (double)R.template chunk<FL>((ch + u) * CH + tid * kEPT, pv, qv);
          }
        }
        for (ch = max(c0, cf); ch < c1; ++ch) {
          const int e0 = ch * CH + tid * kEPT;
          float pv[kEPT], qv[kEPT];
          if constexpr (FL) {
            load8<BF16>(lrow, e0, V, vec, pv);
          } else {
            Raw<false> r1;
            r1.load(rin, e0);
            r1.unpack(pv);
          }
          load8<BF16>(crow, e0, V, vec, qv);
          tsum += (double)R.template chunk<FL>(e0, pv, qv);
          if (nrow) {
            load8<BF16>(nrow, e0, V, vec, qv);
            stat_add8(sn, qv);
          }
        }
      };
      if (from_logits)
        resid_pass(BoolC<true>{});
      else
        resid_pass(BoolC<false>{});
      block_reduce<NW, false>(S, slot, sn, unused, tsum);
      float capp = S.cap_prev[i & 1], capr = S.cap_r[i & 1];  // caught by the thread owning xn
      if (NS > 1) {
        const bool own = xn >= c0 * CH && xn < c1 * CH;
        const double mine[kXRec] = {sn.R, sn.S, tsum, own ? (double)capp : 0.0, own ? (double)capr : 0.0,
                                    own ? 1.0 : 0.0, 0.0, 0.0};
        if (!exchange<NW>(S, mine, rec, NS, s, xr++, spin)) return give_up();
        sn = xmerge_stat(S, NS, 0, 1);
        tsum = xsum(S, NS, 2);
        {  // the caught values come from the one slice that owns the next child's token
          const int lane = threadIdx.x & 63;
          const unsigned long long ow = __ballot(lane < NS && S.xr[lane][5] != 0.0);
          if (ow) {
            const int t = 63 - __builtin_clzll(ow);
            capp = (float)S.xr[t][3], capr = (float)S.xr[t][4];
          }
        }
      }
      if (tsum > 0.0) {
        pnext = cn >= 0 ? (double)capr / tsum : 0.0;
        from_logits = false;
        ib ^= 1;
        T = tsum;
      } else {
        pnext = cn >= 0 ? (double)capp : 0.0;
      }
      if (pre && cn >= 0) {
        const StatRec q = pre[((size_t)b * n + cn) * 2 + 1];
        sn = Stat{q.R, q.S};
      }
      sq = sn;
    }
    if (accepted >= 0) {
      if (tid == 0) S.path[len] = accepted;
      ++len;
      cur = accepted;
      continue;
    }

    // ---- final draw from the current distribution (unnormalised values v)
    const float* rin = rbase + (size_t)ib * Vpad;
    {
      int ch = c0;
      for (; ch < cf; ch += kU) {  // partial last group as in the entry pass
        Raw<BF16> lq[kU];
        Raw<false> rq[kU];
        if (from_logits) {
#pragma unroll
          for (int u = 0; u < kU; ++u) lq[u].load(lrow, min(ch + u, cf - 1) * CH + tid * kEPT);
        } else {
#pragma unroll
          for (int u = 0; u < kU; ++u) rq[u].load(rin, min(ch + u, cf - 1) * CH + tid * kEPT);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          if (ch + u >= cf) break;
          float v[kEPT];
          if (from_logits) {
            lq[u].unpack(v);
#pragma unroll
            for (int j = 0; j < kEPT; ++j) v[j] = ex(v[j], -sl.R);
          } else {
            rq[u].unpack(v);
          }
          seg_store<NW>(S, ch + u, v);
        }
      }
      for (ch = max(c0, cf); ch < c1; ++ch) {
        const int e0 = ch * CH + tid * kEPT;
        float v[kEPT];
        if (from_logits) {
          load8<BF16>(lrow, e0, V, vec, v);
#pragma unroll
          for (int j = 0; j < kEPT; ++j) v[j] = ex(v[j], -sl.R);
        } else {
          Raw<false> r1;
          r1.load(rin, e0);
          r1.unpack(v);
        }
        seg_store<NW>(S, ch, v);
      }
    }
    __syncthreads();
    // the slice's total mass (segments [sg0, sg1) in order), then with NS > 1 the
    // slices' totals: the first slice whose running total passes u * total owns
    // the draw (the last slice with mass, if rounding leaves none)
    const int sg0 = c0 * NW, sg1 = c1 * NW;
    if (wv == 0) {
      double tot = 0.0;
      for (int s0 = sg0; s0 < sg1; s0 += 64) {
        tot += wave_sum(s0 + lane < sg1 ? S.segd[s0 + lane] : 0.0);
      }
      if (lane == 0) S.xtot = tot;
    }
    __syncthreads();
    const float u = u_smp[(size_t)b * n + cur];
    double target = (double)u * S.xtot, run0 = 0.0;
    int owner = 0;
    if (NS > 1) {
      const double mine[kXRec] = {S.xtot, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
      if (!exchange<NW>(S, mine, rec, NS, s, xr++, spin)) return give_up();
      double grand = 0.0;
      for (int t = 0; t < NS; ++t) grand += S.xr[t][0];
      target = (double)u * grand;
      owner = -1;
      int lastm = 0;
      double prefix = 0.0, pre_last = 0.0;
      for (int t = 0; t < NS; ++t) {
        const double tt = S.xr[t][0];
        if (owner < 0 && prefix + tt > target) owner = t, run0 = prefix;
        if (tt > 0.0) lastm = t, pre_last = prefix;
        prefix += tt;
      }
      if (owner < 0) owner = lastm, run0 = pre_last;
    }
    if (s != owner) return;
    if (wv == 0) {
      double run = run0;
      int seg = -1;
      for (int s0 = sg0; s0 < sg1 && seg < 0; s0 += 64) {
        const double x = s0 + lane < sg1 ? S.segd[s0 + lane] : 0.0;
        double inc = x;  // inclusive prefix over the lanes
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const double y = __shfl_up(inc, o);
          if (lane >= o) inc += y;
        }
        const unsigned long long hit = __ballot(run + inc > target);
        if (hit) {
          const int l = __builtin_ctzll(hit);
          seg = s0 + l;
          run += __shfl(inc - x, l);  // mass before the chosen segment
        } else {
          run += __shfl(inc, 63);
        }
      }
      int y = -1;
      if (seg >= 0) {
        // the segment's 512 elements: lane l holds elements seg_base + l*8 .. +8
        const int ch = seg / NW, w = seg % NW;
        const int e0 = ch * CH + (w * 64 + lane) * kEPT;
        float v[kEPT];
        if (from_logits) {
          load8<BF16>(lrow, e0, V, vec, v);
#pragma unroll
          for (int j = 0; j < kEPT; ++j) v[j] = ex(v[j], -sl.R);
        } else {
#pragma unroll
          for (int j = 0; j < kEPT; ++j) v[j] = rin[e0 + j];
        }
        double ls = 0.0;
#pragma unroll
        for (int j = 0; j < kEPT; ++j) ls += (double)v[j];
        double inc = ls;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const double t = __shfl_up(inc, o);
          if (lane >= o) inc += t;
        }
        double acc = run + (inc - ls);
        int mine = -1, lastpos = -1;
#pragma unroll
        for (int j = 0; j < kEPT; ++j) {
          acc += (double)v[j];
          if (mine < 0 && acc > target) mine = e0 + j;
          if (v[j] > 0.f && e0 + j < V) lastpos = e0 + j;
        }
        const unsigned long long hit = __ballot(mine >= 0);
        if (hit) {
          y = __shfl(mine, __builtin_ctzll(hit));
        } else {  // the segment sum passed the target but the element sums (another order) did not
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) lastpos = max(lastpos, __shfl_xor(lastpos, o));
          y = lastpos;
        }
      }
      if (y < 0) {
        // rounding left u * total at or past the end (of this slice, the last
        // one with mass): the last element with mass
        int last = -1;
        for (int ch = c1 - 1; ch >= c0 && last < 0; --ch) {
          for (int part = 0; part < NW && last < 0; ++part) {
            const int e0 = ch * CH + ((NW - 1 - part) * 64 + lane) * kEPT;
            float v[kEPT];
            if (from_logits) {
              load8<BF16>(lrow, e0, V, vec, v);
#pragma unroll
              for (int j = 0; j < kEPT; ++j) v[j] = ex(v[j], -sl.R);
            } else {
#pragma unroll
              for (int j = 0; j < kEPT; ++j) v[j] = rin[e0 + j];
            }
            int mine = -1;
#pragma unroll
            for (int j = 0; j < kEPT; ++j) mine = v[j] > 0.f && e0 + j < V ? e0 + j : mine;
            int best = mine;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) best = max(best, __shfl_xor(best, o));
            last = best;
          }
        }
        y = last;
      }
      if (lane == 0) S.result = y;
    }
    __syncthreads();
    if (tid < n) pr[tid] = tid < len ? S.path[tid] : -1;
    if (tid == 0) {
      plen_out[b] = len;
      bonus[b] = S.result;
      if (status && NS == 1) status[b] = TV_OK;  // sliced: set to TV_OK before the walk
    }
    return;
  }
}

// Polls of one exchange word before a slice gives up (the host may lower it to
// exercise the give-up path; 0 makes every slice give up at its first exchange).
std::atomic<int> g_spin{kSpinMax};

}  // namespace

int mss_set_poll_limit(int polls) { return g_spin.exchange(polls); }

// Workspace: two fp32 residual rows per sequence, the precomputed row statistics,
// and for the sliced walk two slots of exchange records (kMaxNS slices) per
// sequence.
size_t mss_workspace_bytes(int B, int n, int V) {
  const size_t vpad = (size_t)(V + kChunk - 1) / kChunk * kChunk;
  const size_t rows = (size_t)B * 2 * vpad * sizeof(float);
  const size_t stats = ((size_t)B * n * 2 * sizeof(StatRec) + 255) & ~(size_t)255;
  return rows + stats + (size_t)B * 2 * kMaxNS * kXW * sizeof(uint64_t);
}

int mss_precompute(int B, int n, int V, int bf16, int mode) {
  if (mode != 0) return mode == 2;
  // every row read once in parallel, against the walk's serial passes over the
  // rows it visits: worth it while all rows together stay small
  return (double)B * n * V * (bf16 ? 2 : 4) * 2 <= (double)(1u << 30);
}

// Slices per sequence for the sliced walk: as many as keep the whole grid
// resident at once (the workgroups of the sliced kernel that fit on one CU, as
// the runtime reports for the current device, times its CUs) and give every
// slice at least one chunk; 1 when that is a single slice (or the query fails).
int mss_slices(int B, int V, int bf16) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 1;
  const hipError_t e =
      bf16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mss_kernel<true, kThreadsSliced>, kThreadsSliced, 0)
           : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, mss_kernel<false, kThreadsSliced>, kThreadsSliced, 0);
  if (e != hipSuccess || per_cu < 1 || cus < 1) return 1;
  const int nch = (V + kThreadsSliced * kEPT - 1) / (kThreadsSliced * kEPT);
  const long long resident = (long long)per_cu * cus;
  int ns = (int)min((long long)min(kMaxNS, nch), resident / max(B, 1));
  if (ns < 2) return 1;
  const int cps = (nch + ns - 1) / ns;
  return (nch + cps - 1) / cps;  // no empty slice
}

hipError_t launch_mss(int B, int n, int V, int bf16, int mode, const void* logits, const void* ssm,
                      const int32_t* tokens, const int32_t* parent, const float* u_acc, const float* u_smp,
                      float* ws, int32_t* path, int32_t* plen, int32_t* bonus, int32_t* status, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const int vpad = (V + kChunk - 1) / kChunk * kChunk;
  const int vec = ((size_t)V * (bf16 ? 2 : 4)) % 16 == 0;
  char* base = (char*)ws + (size_t)B * 2 * vpad * sizeof(float);
  StatRec* pre = nullptr;
  const int pc = mss_precompute(B, n, V, bf16, mode);
  uint64_t* xrec = (uint64_t*)(base + (((size_t)B * n * 2 * sizeof(StatRec) + 255) & ~(size_t)255));
  // modes 0, 2 and 3 spread each walk over vocabulary slices (with precomputed
  // statistics the slices exchange only at residual passes and the draw)
  const int ns = (status != nullptr && mode != 1) ? mss_slices(B, V, bf16) : 1;
  if (pc) {
    pre = (StatRec*)base;
    uint64_t* clr = ns > 1 ? xrec : nullptr;  // the statistics pass also clears the exchange area
    if (bf16)
      hipLaunchKernelGGL(row_stats_kernel<true>, dim3(B * n * 2), dim3(256), 0, s, n, V, vec, logits, ssm, pre, B,
                         clr, status);
    else
      hipLaunchKernelGGL(row_stats_kernel<false>, dim3(B * n * 2), dim3(256), 0, s, n, V, vec, logits, ssm, pre, B,
                         clr, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ns > 1) {
    const int spin = g_spin.load();
    if (!pc) {
      const size_t words = (size_t)B * kXWords;
      hipLaunchKernelGGL(mss_clear_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, B, xrec,
                         status);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (bf16)
      hipLaunchKernelGGL((mss_kernel<true, kThreadsSliced>), dim3(B * ns), dim3(kThreadsSliced), 0, s, n, V, vec,
                         logits, ssm, tokens, parent, u_acc, u_smp, ws, vpad, pre, ns, xrec, spin, path, plen,
                         bonus, status);
    else
      hipLaunchKernelGGL((mss_kernel<false, kThreadsSliced>), dim3(B * ns), dim3(kThreadsSliced), 0, s, n, V, vec,
                         logits, ssm, tokens, parent, u_acc, u_smp, ws, vpad, pre, ns, xrec, spin, path, plen,
                         bonus, status);
    return hipGetLastError();
  }
  if (bf16)
    hipLaunchKernelGGL((mss_kernel<true, kThreads>), dim3(B), dim3(kThreads), 0, s, n, V, vec, logits, ssm, tokens,
                       parent, u_acc, u_smp, ws, vpad, pre, 1, nullptr, 0, path, plen, bonus, status);
  else
    hipLaunchKernelGGL((mss_kernel<false, kThreads>), dim3(B), dim3(kThreads), 0, s, n, V, vec, logits, ssm, tokens,
                       parent, u_acc, u_smp, ws, vpad, pre, 1, nullptr, 0, path, plen, bonus, status);
  return hipGetLastError();
}

}  // namespace tv
