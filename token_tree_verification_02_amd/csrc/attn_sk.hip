// Tree attention for bf16 or fp16 inputs with many query rows per KV head (GQA groups
// times tree nodes > 128): a persistent, load-balanced variant of the fused
// prefix + tree kernel.
//
// What is computed is the same as in the other bf16 kernel (SpecInfer explainer,
// token-tree structure section, attention equation; kernel-fusion section,
// precomputed topology mask): node u attends in one softmax to every cached
// prefix token of its sequence and to the tree nodes of S_u.
//
// Work decomposition.  The unit of work is a 64-key tile of one item, an item
// being one (sequence, KV head).  An item's tiles are its prefix tiles followed
// by its tree tiles.  All items' tiles form one list, in (sequence, KV head)
// order, and the list is cut into NV equal ranges; each range belongs to one
// "virtual workgroup" (rsplit real workgroups when the rows of an item need
// more than one workgroup, each taking a 256-row slice over the same tiles).  A
// range may start or end inside an item: such a piece writes an unnormalised
// partial (running max, sum, O) into a slot of its workgroup, and a merge pass
// combines the pieces of every item split that way.  Items that a range covers
// whole are written directly.  Ragged prefix lengths therefore cost no idle
// compute units.  The host does not know the prefix lengths, so every
// workgroup derives the tile list from them on the device (two workgroup scans
// over the sequences) before it starts its range.
//
// Inside a workgroup: 8 waves (two per SIMD), each owning one 32-row MFMA
// column block of query rows, so a workgroup covers 256 rows of an item and
// reads each of its KV tiles from HBM once for all of them; every K or V operand
// read from LDS feeds one v_mfma_f32_32x32x16_bf16.  The KV tiles stream HBM ->
// LDS through an S-stage ring with global_load_lds_dwordx4 and hand-placed
// vmcnt waits (one LDS-only barrier per tile).  Full prefix tiles and masked tiles (the ragged last
// prefix tile, the tree tiles) run separate code, so the common case carries no
// per-score selects.  Per score the softmax costs one FMA, one exp2, half a
// max3, half a bf16 pack and half a dot2: the row sums are taken from the
// bf16-rounded probabilities that also feed the PV product.
#include <float.h>

#include <type_traits>

#include "attn_bf16_common.h"

namespace tv {

namespace {

using namespace attn;

constexpr int kTK = 64;  // keys per tile
constexpr int kShadowValu = 4;  // vector instructions scheduled after each product of a shadowed block
constexpr float kSumCap = 256.f;  // 2^kTau: a lane's block sum above this triggers a rescale
constexpr int kSkQB = 1;  // 32-row query blocks per wave (256 rows per workgroup)

__device__ __attribute__((aligned(4096))) uint4 sk_zero_page[256];


// Scheduling record in the workspace (int32), written by one workgroup of the
// attention kernel for the merge pass:
//   [0] total tiles T, [1] tiles per virtual workgroup, [2] NV, [3] unused,
//   [4 .. 4+B]   exclusive prefix sum of tiles over sequences (B+1 entries).
__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

struct SkArgs {
  int32_t* sched;
  uint16_t* po;  // [2*NV][rsplit][RW][D] a piece's O / (sum * scale), fp16
  float* pml;    // [2*NV][rsplit][RW][4]  (max in the log2 domain, sum, scale, unused)
  int rsplit, NV, cap;
};

// Position in the tile list: item (b, g), tile `off` within the item.
struct Cursor {
  int b, g, off, L, tpre, titem;
};

__device__ __forceinline__ void cursor_seq(Cursor& c, const AS4 int32_t* plen, int cap, int ttree) {
  c.L = clamp_len(plen[c.b], cap);
  c.tpre = (c.L + kTK - 1) / kTK;
  c.titem = c.tpre + ttree;
}

__device__ __forceinline__ void cursor_next(Cursor& c, const AS4 int32_t* plen, int B, int Hkv, int cap, int ttree) {
  if (++c.off < c.titem) return;
  c.off = 0;
  if (++c.g < Hkv) return;
  c.g = 0;
  if (++c.b < B) cursor_seq(c, plen, cap, ttree);
}

// The tile list, derived from the prefix lengths by every workgroup with the
// same integer arithmetic (the host does not know the lengths): T tiles in all,
// `per` tiles per range, and the cursor of tile r0 = v * per, the first of range
// v.  A workgroup passing rec != nullptr also writes the scheduling record.
// NT threads, all of which call this; returns false (uniformly) for an empty range.
template <int NT>
__device__ __forceinline__ bool sk_plan(const int32_t* __restrict__ plen, int B, int cap, int ttree, int Hkv, int NV,
                                        int v, int32_t* rec, int& T_out, int& per_out, Cursor& c) {
  __shared__ int part[NT / 64];
  __shared__ int hit[3];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  auto tiles = [&](int b) { return b < B ? ((clamp_len(plen[b], cap) + kTK - 1) / kTK + ttree) * Hkv : 0; };
  if (B <= NT) {
    // one pass (a batch of at most NT sequences): each thread's sequence, one
    // inclusive scan over the workgroup gives the offsets and the total, then the
    // sequence holding tile r0 reports the cursor
    const int b = tid;
    const int t = tiles(b);
    int x = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) part[wv] = x;
    __syncthreads();
    int off = 0, T = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      off += w < wv ? part[w] : 0;
      T += part[w];
    }
    const int ex = off + x - t;  // tiles before sequence b
    const int per = (T + NV - 1) / NV;
    const long long r0 = (long long)v * per;
    T_out = T;
    per_out = per;
    if (rec != nullptr) {
      if (tid == 0) rec[0] = T, rec[1] = per, rec[2] = NV, rec[3] = 0, rec[4 + B] = T;
      if (b < B) rec[4 + b] = ex;
    }
    if (r0 >= T) return false;  // uniform
    if (b < B && ex <= r0 && r0 < ex + t) {
      const int tb = t / Hkv, r = (int)(r0 - ex);
      hit[0] = b;
      hit[1] = r / tb;
      hit[2] = r % tb;
    }
    __syncthreads();
    c.b = hit[0];
    c.g = hit[1];
    c.off = hit[2];
    return true;
  }
  // larger batches: pass 1, the total
  int T = 0;
  for (int base = 0; base < B; base += NT) {
    int x = tiles(base + tid);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    if (lane == 0) part[wv] = x;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) T += part[w];
    __syncthreads();
  }
  const int per = (T + NV - 1) / NV;
  const long long r0 = (long long)v * per;
  T_out = T;
  per_out = per;
  if (rec != nullptr && tid == 0) {
    rec[0] = T;
    rec[1] = per;
    rec[2] = NV;
    rec[3] = 0;
    rec[4 + B] = T;
  }
  if (r0 >= T) return false;
  // pass 2: exclusive prefix sum over the sequences; the one holding tile r0
  // gives the cursor (the recording workgroup goes through all of them)
  int carry = 0;
  for (int base = 0; base < B; base += NT) {
    const int b = base + tid;
    const int t = tiles(b);
    int x = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) part[wv] = x;
    __syncthreads();
    int off = carry, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      off += w < wv ? part[w] : 0;
      tot += part[w];
    }
    const int ex = off + x - t;  // tiles before sequence b
    if (b < B) {
      if (rec != nullptr) rec[4 + b] = ex;
      if (ex <= r0 && r0 < ex + t) {
        const int tb = t / Hkv, r = (int)(r0 - ex);
        hit[0] = b;
        hit[1] = r / tb;
        hit[2] = r % tb;
      }
    }
    carry += tot;
    __syncthreads();
    if (rec == nullptr && carry > r0) break;  // uniform: every thread holds the same carry
  }
  c.b = hit[0];
  c.g = hit[1];
  c.off = hit[2];
  return true;
}

// 64-bit word `w` (< 4) of a node's mask, from registers.
__device__ __forceinline__ uint64_t pick_word(const uint64_t (&m)[4], int w) {
  return w == 0 ? m[0] : (w == 1 ? m[1] : (w == 2 ? m[2] : m[3]));
}

// Scores of a 32-key block past the tile's valid keys, or (tree tiles) of keys
// that are not ancestors of the lane's node, become -inf.  The lane holds key
// 16*(r>>3) + 8*hh + (r&7) of the block.
__device__ __forceinline__ void sk_mask(f32x16& s, int kb, int lim, bool tree, uint64_t bits, int hh) {
  const int nv = lim - 32 * kb;  // valid keys of the block (lim is uniform)
  if (!tree && nv >= 32) return;  // e.g. a segment's first tile: nothing to mask
  // one keep bit per key of the block, then per score a sign-extended bit field
  // selects the score or -inf (two VALU per score)
  uint32_t keep = nv >= 32 ? ~0u : (nv <= 0 ? 0u : (1u << nv) - 1u);
  if (tree) keep &= (uint32_t)(bits >> (32 * kb));
  keep >>= 8 * hh;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int pos = 16 * (r >> 3) + (r & 7);
    const uint32_t m = (uint32_t)((int)(keep << (31 - pos)) >> 31);  // all ones iff the key is kept
    s[r] = __uint_as_float((__float_as_uint(s[r]) & m) | (0xff800000u & ~m));
  }
}

// Maximum of the lane's 16 scores and its partner's (lane ^ 32): the column max.
__device__ __forceinline__ float sk_colmax(const f32x16& s) {
  float mx = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) mx = fmaxf(fmaxf(mx, s[r]), s[r + 1]);
  mx = fmaxf(mx, s[15]);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// Probabilities of 16 scores against the running max (log2 domain), rounded to
// the 16-bit type (the PV operand); their sum is added to l with a 16-bit dot
// product.
template <class E>
__device__ __forceinline__ void sk_probs(const f32x16& s, typename E::V8 (&P)[2], float& l, float sl2, float msub) {
  const typename E::V2 ones = {E::cvt(1.0f), E::cvt(1.0f)};
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      typename E::V2 pr;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h2 + e], sl2, -msub));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h2 + e + 1], sl2, -msub));
      pr[0] = E::cvt(p0);
      pr[1] = E::cvt(p1);
      l = E::dot2(pr, ones, l);
      P[h2][e] = pr[0];
      P[h2][e + 1] = pr[1];
    }
}

// Running-max update for one query block (log2 domain): the accumulators are
// rescaled only when the block max exceeds the running max by more than kTau.
template <int D>
__device__ __forceinline__ void sk_rescale(f32x16 (&Oq)[D / 32], float& m_run, float& lsum, float mx) {
  const float m_new = fmaxf(m_run, mx);
  const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
  lsum *= alpha;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) Oq[db][r] *= alpha;
    __builtin_amdgcn_sched_barrier(0);  // bounds the registers in flight
  }
  m_run = m_new;
}

// O^T += V^T P^T for one 32-key block: each V operand (two transposing LDS
// reads) feeds all QB query blocks.
template <class E, int D, int QB>
__device__ __forceinline__ void sk_pv(const char AS3* Vr, int kb, const typename E::V8 (&P)[QB][2],
                                      f32x16 (&O)[QB][D / 32],
                                      const uint32_t (&vofs)[D / 32]) {
  constexpr int DB = D / 32, ROWB = 2 * D;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    typename E::V8 vop[DB];  // the half block's operand reads first, then its products
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const char AS3* vp = Vr + (kb * 32 + 16 * half) * ROWB + vofs[db];
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 AS3*)vp);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 AS3*)(vp + 4 * ROWB));
      vop[db] = __builtin_bit_cast(typename E::V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        O[qb][db] = E::mfma(vop[db], P[qb][half], O[qb][db]);
  }
}

// S^T = K Q^T for one 32-key block and all QB query blocks (each K operand read
// once for all of them).
template <class E, int D, int QB>
__device__ __forceinline__ void sk_qk(const char AS3* Kr, int kb, const typename E::V8 (&qop)[QB][D / 16],
                                      const uint32_t (&kofs)[D / 16], f32x16 (&Sa)[QB]) {
  constexpr int SD = D / 16, ROWB = 2 * D;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) Sa[qb][r] = 0.f;
  // all operand reads of the block first (they pipeline in the LDS), then the
  // products: the scheduler may not pair each read with its product
  typename E::V8 kop[SD];
#pragma unroll
  for (int sd = 0; sd < SD; ++sd) kop[sd] = *(const typename E::V8 AS3*)(Kr + kb * 32 * ROWB + kofs[sd]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int sd = 0; sd < SD; ++sd)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      Sa[qb] = E::mfma(kop[sd], qop[qb][sd], Sa[qb]);
}

// One 64-key tile for one wave holding one 32-row query block.  MASKED: key
// validity from `lim` (keys of the tile that exist) and, for tree tiles, the
// ancestor bits of each query's node.  Both key blocks' QK products are issued
// first, then per block max -> (rare) rescale -> softmax -> PV.
// Full tiles place each block's softmax in the shadow of the other block's
// products: issued in bursts, a wave's products stall its issue while the matrix
// core drains them, and its softmax then runs with the matrix core idle unless
// the other wave on the SIMD happens to be in the opposite phase.  So block 0's
// probabilities are emitted with block 1's QK products and block 1's with block
// 0's PV products, and the scheduler alternates one product with up to
// kShadowValu vector instructions (VALU or transcendental; 4 measured best
// among 2 to 6).  The arithmetic and its order are those of one block after
// the other.
// refill: the ring's DMA for a later tile, issued once block 0's QK products are
// in the matrix core (its scalar address work then overlaps them; issued right
// after the barrier it delayed the first products, issued after block 1's
// products it delayed the PV products).
// slt: the score scale (log2 domain).
template <class E, int D, int QB, bool MASKED, class RF>
__device__ __forceinline__ void sk_tile(const char AS3* Kr, const char AS3* Vr,
                                        const typename E::V8 (&qop)[QB][D / 16],
                                        f32x16 (&O)[QB][D / 32], float (&m_run)[QB], float (&lsum)[QB],
                                        const uint32_t (&kofs)[D / 16], const uint32_t (&vofs)[D / 32], float slt,
                                        int lim, bool tree, const uint64_t (&bits)[QB], int hh, RF&& refill) {
  static_assert(QB == 1, "one query block per wave");
  if constexpr (!MASKED) {
    // Full prefix tile with the reference max already set (the first tile of a
    // segment takes the masked path): the probabilities are taken against the
    // reference directly, and the block's maximum is only computed, with a
    // rescale, when a lane's sum of 16 probabilities exceeds 2^kTau, i.e.
    // whenever some probability might (the same bound the masked path keeps).
    constexpr int SD = D / 16, DB = D / 32, ROWB = 2 * D;
    f32x16 S0[1], S1;
    sk_qk<E, D, 1>(Kr, 0, qop, kofs, S0);
    refill();
    typename E::V8 P0[1][2], P1[1][2];
    float lb0 = 0.f, lb1 = 0.f;
    {  // block 1's QK products, block 0's probabilities in their shadow
      typename E::V8 kop[SD];
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) kop[sd] = *(const typename E::V8 AS3*)(Kr + 32 * ROWB + kofs[sd]);
#pragma unroll
      for (int r = 0; r < 16; ++r) S1[r] = 0.f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) S1 = E::mfma(kop[sd], qop[0][sd], S1);
      sk_probs<E>(S0[0], P0[0], lb0, slt, m_run[0]);
#pragma unroll
      for (int i = 0; i < SD; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x402, kShadowValu, 0);  // then VALU / transcendental
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (__builtin_expect(__any(lb0 > kSumCap), 0)) {
      sk_rescale<D>(O[0], m_run[0], lsum[0], sk_colmax(S0[0]) * slt);
      lb0 = 0.f;
      sk_probs<E>(S0[0], P0[0], lb0, slt, m_run[0]);
    }
    lsum[0] += lb0;
    {  // block 0's PV products, block 1's probabilities in their shadow
      typename E::V8 vop[2][DB];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const char AS3* vp = Vr + (16 * half) * ROWB + vofs[db];
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 AS3*)vp);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 AS3*)(vp + 4 * ROWB));
          vop[half][db] = __builtin_bit_cast(typename E::V8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int db = 0; db < DB; ++db) O[0][db] = E::mfma(vop[half][db], P0[0][half], O[0][db]);
      sk_probs<E>(S1, P1[0], lb1, slt, m_run[0]);
#pragma unroll
      for (int i = 0; i < 2 * DB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x402, kShadowValu, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (__builtin_expect(__any(lb1 > kSumCap), 0)) {
      sk_rescale<D>(O[0], m_run[0], lsum[0], sk_colmax(S1) * slt);
      lb1 = 0.f;
      sk_probs<E>(S1, P1[0], lb1, slt, m_run[0]);
    }
    lsum[0] += lb1;
    sk_pv<E, D, 1>(Vr, 1, P1, O, vofs);
    return;
  }
  f32x16 Sa[2][1];
  sk_qk<E, D, 1>(Kr, 0, qop, kofs, Sa[0]);
  refill();
  sk_qk<E, D, 1>(Kr, 1, qop, kofs, Sa[1]);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    if constexpr (MASKED) sk_mask(Sa[kb][0], kb, lim, tree, bits[0], hh);
    const float mx = sk_colmax(Sa[kb][0]) * slt;  // scale > 0 commutes with max
    if (__builtin_expect(__any(mx > m_run[0] + kTau), 0)) sk_rescale<D>(O[0], m_run[0], lsum[0], mx);
    typename E::V8 P[1][2];
    const float msub = (m_run[0] == -INFINITY) ? 0.f : m_run[0];
    sk_probs<E>(Sa[kb][0], P[0], lsum[0], slt, msub);
    sk_pv<E, D, 1>(Vr, kb, P, O, vofs);
  }
}

// NT: every tile is read by exactly one workgroup (one row slice per item), so the
// full prefix tiles stream non-temporal; with several row slices the later ones
// find the tiles in cache, so they are read normally.
template <bool F16, bool NT, int D, int QB, int RB, int S>
__global__ __launch_bounds__(64 * RB) void attn_sk_kernel(AttnArgs a, SkArgs k) {
  using E = Elt<F16>;
  constexpr int RW = 32 * QB * RB;          // query rows per workgroup
  constexpr int ROWB = 2 * D;               // bytes per token row
  constexpr int REG = kTK * ROWB;           // K (or V) region of a stage
  constexpr int STAGE = 2 * REG;
  constexpr int LINES = STAGE / 1024;       // 1 KB DMA lines per tile
  constexpr int HL = LINES / 2;             // lines of the K region
  constexpr int LPW = LINES / RB;           // DMA instructions per wave per tile
  constexpr int RPL = 1024 / ROWB;          // token rows per line
  constexpr int GPR = D / 8;                // 16-byte granules per row
  constexpr int SD = D / 16, DB = D / 32;
  constexpr int WAITN = (S - 2) * LPW;      // loads a wave may leave in flight
  constexpr int NID = LPW / 2;              // paged: distinct blocks among a wave's K (= V) lines
  static_assert(HL % RB == 0 && LPW * (S - 2) < 64 && LPW % 2 == 0, "pipeline shape");
  __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int rb = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int n = a.n, G = a.G, Hkv = a.Hkv, rows = n * G, B = a.B;
  const int ttree = (n + kTK - 1) / kTK;

  // XCD-aware order: consecutive logical ids (the row slices of one range, then
  // neighbouring ranges) land on the same XCD and share its L2.
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int perx = nwg >> 3, rem = nwg & 7, xcd = wg & 7;
  const int lid = xcd * perx + min(xcd, rem) + (wg >> 3);
  const int rs = lid % k.rsplit, v = lid / k.rsplit;

  const AS4 int32_t* plen = (const AS4 int32_t*)a.plen;
  int T, per;
  Cursor ic;
  if (!sk_plan<64 * RB>(a.plen, B, k.cap, ttree, Hkv, k.NV, v, lid == 0 ? k.sched : nullptr, T, per, ic))
    return;  // empty range (uniform per workgroup)
  const int r0 = v * per;
  const int ntiles = min(T - r0, per);
  cursor_seq(ic, plen, k.cap, ttree);
  Cursor cc = ic;

  const char* kc = (const char*)a.kc;
  const char* vc = (const char*)a.vc;
  const char* ktr = (const char*)a.kt;
  const char* vtr = (const char*)a.vt;
  const char* zero = (const char*)sk_zero_page;
  const char* zsrc = zero + lane * 16;
  const uint32_t ring = (uint32_t)(uintptr_t)(AS3 void*)smem;
  const AS4 int32_t* btc = (const AS4 int32_t*)a.bt;
  auto dma_full = [](const void* sbase, uint32_t voff, uint32_t lds_line) {
    if constexpr (NT)
      dma16s_nt(sbase, voff, lds_line);
    else
      dma16s(sbase, voff, lds_line);
  };

  // per-lane DMA geometry: line q*RB + rb of the tile belongs to this wave; the
  // lane's token row within the tile and its source granule (swizzled) follow
  // from q alone, so only the byte offsets of full tiles are kept.
  auto lrow_of = [=](int ln, int q) {
    const int line = q * RB + rb;
    return (q * RB >= HL ? line - HL : line) * RPL + ln / GPR;
  };
  auto gran_of = [=](int ln, int q) {
    const int lrow = lrow_of(ln, q), pg = ln % GPR;
    return q * RB >= HL ? (pg ^ vswz<D>(lrow)) : (pg ^ kswz<D>(lrow));
  };
  uint32_t voff[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    const int lrow = lrow_of(lane, q);
    const int key = q * RB >= HL ? lrow : perm_row(lrow);
    voff[q] = (uint32_t)(((a.paged ? (key & 15) : key) * D + gran_of(lane, q) * 8) * 2);
  }
  // Paged cache: the wave's K lines t < NID and V lines NID + t cover the same
  // token rows, so a tile needs NID block ids per wave: block kq[t] of the tile's
  // four.  They are loaded one tile ahead of their DMA (load_ids), so the
  // scalar-load latency never sits between the barrier and the tile's compute.
  int kq[NID];
#pragma unroll
  for (int t = 0; t < NID; ++t) kq[t] = ((t * RB + rb) * RPL) >> 4;
  const int max_blocks = a.max_blocks, num_blocks = a.num_blocks;
  auto load_ids = [&](const Cursor& c, int (&ids)[NID]) {
#pragma unroll
    for (int t = 0; t < NID; ++t) ids[t] = -1;
    if (!a.paged || c.b >= B || c.off >= c.tpre) return;
    const AS4 int32_t* row = btc + (size_t)c.b * max_blocks;
#pragma unroll
    for (int t = 0; t < NID; ++t) {
      const int bi = c.off * (kTK / TV_PAGE) + kq[t];
      ids[t] = bi < max_blocks ? row[bi] : -1;
    }
  };

  // DMA of this wave's lines of the bf16 tile at cursor c to LDS address gbase
  // (!live: zeros); ids: the tile's block ids from load_ids (paged prefix tiles)
  auto issue = [=](const Cursor& c, bool live, uint32_t gbase, const int (&ids)[NID]) {
    // an opaque copy of the lane id keeps the compiler from hoisting the
    // per-line geometry of the rare paths out of the loop (it would hold dozens
    // of registers for them)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (!live) {
#pragma unroll
      for (int q = 0; q < LPW; ++q) dma16(zsrc, gbase + (q * RB + rb) * 1024);
      return;
    }
    const int b = c.b, g = c.g;
    if (c.off >= c.tpre) {  // tree tile
      const int tstart = (c.off - c.tpre) * kTK;
#pragma unroll
      for (int q = 0; q < LPW; ++q) {
        const bool isv = q * RB >= HL;
        const int vv = tstart + (isv ? lrow_of(ln, q) : perm_row(lrow_of(ln, q)));
        const char* src = (isv ? vtr : ktr) + ((((size_t)b * n + vv) * Hkv + g) * D + gran_of(ln, q) * 8) * 2;
        dma16(vv < n ? src : zsrc, gbase + (q * RB + rb) * 1024);
      }
      return;
    }
    const int tstart = c.off * kTK;
    const bool full = tstart + kTK <= c.L;
    if (a.paged) {
      size_t boff[NID];  // byte offset of (block, KV head) in either cache; ~0 for a bad id
#pragma unroll
      for (int t = 0; t < NID; ++t)
        boff[t] = (ids[t] >= 0 && ids[t] < num_blocks) ? ((size_t)ids[t] * Hkv + g) * (TV_PAGE * D * 2) : ~(size_t)0;
#pragma unroll
      for (int q = 0; q < LPW; ++q) {
        const bool isv = q >= NID;
        const int line = q * RB + rb;
        const size_t bo = boff[q % NID];
        const bool bok = bo != ~(size_t)0;
        const char* lbase = (isv ? vc : kc) + bo;
        if (full) {
          dma_full(bok ? lbase : zero, voff[q], gbase + line * 1024);
        } else {
          const int j = tstart + (isv ? lrow_of(ln, q) : perm_row(lrow_of(ln, q)));
          dma16(bok && j < c.L ? lbase + voff[q] : zsrc, gbase + line * 1024);
        }
      }
    } else {
      const size_t rowbase = ((size_t)b * Hkv + g) * a.Lmax + tstart;
      const char* kb = kc + rowbase * D * 2;
      const char* vb = vc + rowbase * D * 2;
#pragma unroll
      for (int q = 0; q < LPW; ++q) {
        const bool isv = q * RB >= HL;
        const int line = q * RB + rb;
        if (full) {
          dma_full(isv ? vb : kb, voff[q], gbase + line * 1024);
        } else {
          const int j = tstart + (isv ? lrow_of(ln, q) : perm_row(lrow_of(ln, q)));
          dma16(j < c.L ? (isv ? vb : kb) + voff[q] : zsrc, gbase + line * 1024);
        }
      }
    }
  };

  // per-lane LDS read offsets
  uint32_t kofs[SD], vofs[DB];
#pragma unroll
  for (int sd = 0; sd < SD; ++sd) kofs[sd] = col * ROWB + (((2 * sd + hh) ^ kswz<D>(col)) << 4);
  {
    const int l16 = lane & 15, mhalf = (lane >> 4) & 1;
    const int vr = 8 * hh + (l16 >> 2);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int lg = 4 * db + 2 * mhalf + ((lane & 3) >> 1);
      vofs[db] = vr * ROWB + ((lg ^ vswz<D>(vr)) << 4) + ((lane & 1) << 3);
    }
  }

  const int rowbase = rs * RW + 32 * QB * rb;  // first query row of this wave within an item
  const float sl2 = a.scale_log2;

  // prologue: S-1 tiles in flight, then the block ids of the next tile
  int ids[NID];
#pragma unroll
  for (int i = 0; i < S - 1; ++i) {
    const bool live = i < ntiles;
    load_ids(ic, ids);
    issue(ic, live, ring + i * STAGE, ids);
    if (live) cursor_next(ic, plen, B, Hkv, k.cap, ttree);
  }
  load_ids(ic, ids);

  // Segments: the part of one item inside this range.  Queries, masks and
  // accumulators are set up before a segment's tile loop and written out after
  // it, so the loop itself touches the accumulators only through the MFMAs
  // (and the rare rescale).
  int it = 0;
  for (int seg = 0; it < ntiles; ++seg) {
    const bool seg_whole = cc.off == 0;
    const int seg_len = min(cc.titem - cc.off, ntiles - it);
    const bool item_end = cc.off + seg_len == cc.titem;
    typename E::V8 qop[QB][SD];
    uint64_t mw[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = rowbase + 32 * qb + col;
      const bool ok = row < rows;
      const int u = ok ? row / G : 0, gi = ok ? row % G : 0;
      const uint16_t* qp = (const uint16_t*)a.q + ((size_t)(cc.b * n + u) * a.Hq + cc.g * G + gi) * D;
#pragma unroll
      for (int sd = 0; sd < SD; ++sd) {
        u32x4 x = {0, 0, 0, 0};
        if (ok) x = *(const u32x4*)(qp + 16 * sd + 8 * hh);
        qop[qb][sd] = __builtin_bit_cast(typename E::V8, x);
      }
      const uint64_t* mp = a.mask + ((size_t)cc.b * n + u) * a.W;
#pragma unroll
      for (int w = 0; w < 4; ++w) mw[qb][w] = (ok && w < a.W) ? mp[w] : 0ull;
    }
    wait_vmcnt<0>();  // queries and masks are in registers (drains the ring once per segment)
    f32x16 O[QB][DB];
    float m_run[QB], lsum[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      m_run[qb] = -INFINITY;
      lsum[qb] = 0.f;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[qb][db][r] = 0.f;

    // One tile iteration: wait for the tile, free the stage of the previous one,
    // compute, refilling the ring from inside the tile (after its first products).
    // The full prefix tiles of the segment run first in a loop without any masking
    // code, then the masked ones (the ragged last prefix tile and the tree tiles)
    // in a second loop.
    auto step = [&](auto masked_c, int j) {
      constexpr bool MASKED = decltype(masked_c)::value;
      wait_vmcnt<WAITN>();  // this wave's lines of tile `it` have landed
      lds_barrier();        // ... everyone's, and everyone left tile it-1
      auto refill = [&]() {
        const bool live = it + S - 1 < ntiles;
        issue(ic, live, ring + ((it + S - 1) % S) * STAGE, ids);
        if (live) {
          cursor_next(ic, plen, B, Hkv, k.cap, ttree);
          load_ids(ic, ids);  // consumed by the next tile's issue
        }
      };
      const int off = cc.off + j;
      const int st = it % S;
      const char AS3* Kr = (const char AS3*)smem + st * STAGE;
      const char AS3* Vr = Kr + REG;
      uint64_t bits[QB];
      int lim = kTK;
      bool tree = false;
      if constexpr (MASKED) {
        tree = off >= cc.tpre;
        const int tstart = tree ? (off - cc.tpre) * kTK : off * kTK;
        lim = tree ? n - tstart : cc.L - tstart;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) bits[qb] = tree ? pick_word(mw[qb], tstart >> 6) : 0ull;
      } else {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) bits[qb] = 0ull;
      }
      sk_tile<E, D, QB, MASKED>(Kr, Vr, qop, O, m_run, lsum, kofs, vofs, sl2, lim, tree, bits, hh, refill);
      ++it;
    };
    // full prefix tiles come first; the segment's first tile always takes the
    // masked path, which sets the reference max the full-tile path builds on
    const int nfull = max(0, min(seg_len, cc.L / kTK - cc.off));
    step(std::integral_constant<bool, true>(), 0);
    for (int j = 1; j < nfull; ++j) step(std::integral_constant<bool, false>(), j);
    for (int j = max(nfull, 1); j < seg_len; ++j) step(std::integral_constant<bool, true>(), j);

    // write the segment out: whole items directly, pieces into this range's slots
    const bool whole = seg_whole && item_end;
    const int slot = 2 * v + (seg == 0 ? 0 : 1);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lp = lsum[qb];
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lp), __float_as_uint(lp), false, false);
      const float ltot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const int row = rowbase + 32 * qb + col;
      if (row >= rows) continue;
      const int u = row / G, gi = row % G, h = cc.g * G + gi;
      if (whole) {
        const float inv = 1.f / ltot;
        uint16_t* op = (uint16_t*)a.out + ((size_t)(cc.b * n + u) * a.Hq + h) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int d0 = 32 * db + 8 * rq + 4 * hh;
            uint2 w;
            w.x = E::bits(O[qb][db][4 * rq] * inv) | (E::bits(O[qb][db][4 * rq + 1] * inv) << 16);
            w.y = E::bits(O[qb][db][4 * rq + 2] * inv) | (E::bits(O[qb][db][4 * rq + 3] * inv) << 16);
            *(uint2*)(op + d0) = w;
          }
        if (a.lse != nullptr && hh == 0)
          a.lse[(size_t)(cc.b * n + u) * a.Hq + h] = (m_run[qb] + __log2f(ltot)) * kLn2;
      } else {
        // a piece: O over its own sum is a weighted mean of value entries; it is
        // stored in fp16 times a power of two that puts the row's largest entry in
        // [2^14, 2^15), so every entry keeps fp16's relative precision (2^-12)
        // whatever the values' range, in half the bytes of fp32.  The merge
        // weights the piece by its sum and undoes the scale; a row with no key in
        // the piece has sum 0 and weight 0.
        const size_t pidx = ((size_t)slot * k.rsplit + rs) * RW + (row - rs * RW);
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        float amax = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(O[qb][db][r]));
        {
          const auto ms = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
          amax = fmaxf(__uint_as_float(ms[0]), __uint_as_float(ms[1])) * inv;
        }
        // amax < 2^(ex + 15); the floor keeps 2^-ex finite for rows of near-zero values
        const int ex = amax > 0.f ? max(__builtin_amdgcn_frexp_expf(amax) - 15, -96) : 0;
        const float sc = __builtin_amdgcn_ldexpf(inv, -ex);
        uint16_t* wo = k.po + pidx * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int d0 = 32 * db + 8 * rq + 4 * hh;
            uint2 w;
            w.x = Elt<true>::bits(O[qb][db][4 * rq] * sc) | (Elt<true>::bits(O[qb][db][4 * rq + 1] * sc) << 16);
            w.y = Elt<true>::bits(O[qb][db][4 * rq + 2] * sc) | (Elt<true>::bits(O[qb][db][4 * rq + 3] * sc) << 16);
            *(uint2*)(wo + d0) = w;
          }
        if (hh == 0) *(float4*)(k.pml + 4 * pidx) = make_float4(m_run[qb], ltot, __builtin_amdgcn_ldexpf(1.f, ex), 0.f);
      }
    }
    // on to the next item
    cc.off = 0;
    if (++cc.g == Hkv) {
      cc.g = 0;
      if (++cc.b < B) cursor_seq(cc, plen, k.cap, ttree);
    }
  }
  wait_vmcnt<0>();  // trailing zero-page loads land before the workgroup's LDS is released
}

// Combines the pieces of items that were split between ranges, and reports bad
// prefix lengths and block ids.  One workgroup per (item, row slice, 64 rows).
// The kernel is a short chain of memory round trips, so each phase issues all of
// a thread's loads before it uses any: the block ids of the status check in groups
// of 8 per thread, then the pieces' (max, sum, scale) records and values for all of
// the thread's rows (both pieces at once for an item split in two).
template <bool F16>
__global__ __launch_bounds__(256) void sk_merge_kernel(AttnArgs a, SkArgs k, int RW, int chunks) {
  const int D = a.D, rows = a.n * a.G, Hkv = a.Hkv;
  int t = blockIdx.x;
  const int ch = t % chunks;
  t /= chunks;
  const int rs = t % k.rsplit;
  t /= k.rsplit;
  const int g = t % Hkv, b = t / Hkv;
  const int tid = threadIdx.x;

  if (a.status != nullptr && g == 0 && rs == 0 && ch == 0) {
    const int Lraw = a.plen[b];
    int bad = (Lraw < 0 || Lraw > k.cap);
    if (a.paged) {
      const int L = clamp_len(Lraw, k.cap);
      const int nb = (L + TV_PAGE - 1) / TV_PAGE;
      const int32_t* bt = a.bt + (size_t)b * a.max_blocks;
      for (int i0 = 0; i0 < nb; i0 += 8 * 256) {
        int id[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * 256 + tid;
          id[u] = i < nb ? bt[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) bad |= (id[u] < 0 || id[u] >= a.num_blocks);
      }
    }
    bad = __syncthreads_or(bad);
    if (tid == 0) a.status[b] = bad ? TV_EINVAL : TV_OK;
  }

  const int T = k.sched[0], per = k.sched[1];
  const int cb0 = k.sched[4 + b], cb1 = k.sched[4 + b + 1];
  const int titem = (cb1 - cb0) / Hkv;
  const int s0 = cb0 + g * titem, e0 = s0 + titem;
  const int ws = s0 / per, we = (e0 - 1) / per;
  if (ws == we || T == 0) return;  // one range held the whole item and wrote it

  // thread layout: tpr threads per row (4 values each), rpp rows side by side, so a
  // thread owns rows r0, r0 + rpp, ... of the 64 (8 of them for D = 128, 4 for 64)
  constexpr int NRM = 8;
  const int tpr = D / 4;
  const int rpp = 256 / tpr;
  const int nr = 64 / rpp;
  const int r0 = tid / tpr, d0 = (tid % tpr) * 4;
  auto piece = [&](int w, int j) -> size_t {  // index of this row's piece in range w's slot
    const int slot = (s0 <= (long long)w * per) ? 2 * w : 2 * w + 1;
    return ((size_t)slot * k.rsplit + rs) * RW + (ch * 64 + r0 + j * rpp);
  };
  float M[NRM];
  float4 acc[NRM];
  float lt[NRM];
#pragma unroll
  for (int j = 0; j < NRM; ++j) M[j] = -INFINITY, acc[j] = make_float4(0.f, 0.f, 0.f, 0.f), lt[j] = 0.f;
  auto add = [&](int j, const float4& mls, const uint2& oc) {  // one piece into row j
    if (mls.x == -INFINITY) return;                             // no attended key in this piece
    const float wl = exp2f(mls.x - M[j]) * mls.y;
    const float wo = wl * mls.z;
    acc[j].x += wo * f16_to_f32((uint16_t)oc.x);
    acc[j].y += wo * f16_to_f32((uint16_t)(oc.x >> 16));
    acc[j].z += wo * f16_to_f32((uint16_t)oc.y);
    acc[j].w += wo * f16_to_f32((uint16_t)(oc.y >> 16));
    lt[j] += wl;
  };
  if (we == ws + 1) {
    // two pieces (the usual split): both pieces' records and values for all rows in
    // one round of loads
    float4 ma[NRM], mb[NRM];  // max, sum, scale
    uint2 oa[NRM], ob[NRM];
#pragma unroll
    for (int j = 0; j < NRM; ++j) {
      if (j < nr) {
        const size_t pa = piece(ws, j), pb = piece(we, j);
        ma[j] = *(const float4*)(k.pml + 4 * pa);
        mb[j] = *(const float4*)(k.pml + 4 * pb);
        oa[j] = *(const uint2*)(k.po + pa * D + d0);
        ob[j] = *(const uint2*)(k.po + pb * D + d0);
      }
    }
#pragma unroll
    for (int j = 0; j < NRM; ++j) {
      if (j < nr) {
        M[j] = fmaxf(fmaxf(M[j], ma[j].x), mb[j].x);
        add(j, ma[j], oa[j]);
        add(j, mb[j], ob[j]);
      }
    }
  } else {
    // an item over three or more ranges: the maxima of one piece for all rows, then
    // one piece's records and values for all rows, piece by piece
    for (int w = ws; w <= we; ++w) {
      float mx[NRM];
#pragma unroll
      for (int j = 0; j < NRM; ++j) mx[j] = j < nr ? k.pml[4 * piece(w, j)] : -INFINITY;
#pragma unroll
      for (int j = 0; j < NRM; ++j) M[j] = fmaxf(M[j], mx[j]);
    }
    for (int w = ws; w <= we; ++w) {
      float4 mls[NRM];
      uint2 oc[NRM];
#pragma unroll
      for (int j = 0; j < NRM; ++j) {
        if (j < nr) {
          const size_t pi = piece(w, j);
          mls[j] = *(const float4*)(k.pml + 4 * pi);
          oc[j] = *(const uint2*)(k.po + pi * D + d0);
        }
      }
#pragma unroll
      for (int j = 0; j < NRM; ++j)
        if (j < nr) add(j, mls[j], oc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < NRM; ++j) {
    const int row = rs * RW + ch * 64 + r0 + j * rpp;
    if (j >= nr || row >= rows) continue;
    const float inv = 1.f / lt[j];
    const int u = row / a.G, gi = row % a.G, h = g * a.G + gi;
    const size_t oi = ((size_t)(b * a.n + u) * a.Hq + h) * D + d0;
    using E = Elt<F16>;
    uint2 wv;
    wv.x = E::bits(acc[j].x * inv) | (E::bits(acc[j].y * inv) << 16);
    wv.y = E::bits(acc[j].z * inv) | (E::bits(acc[j].w * inv) << 16);
    *(uint2*)((uint16_t*)a.out + oi) = wv;
    if (a.lse != nullptr && d0 == 0) a.lse[(size_t)(b * a.n + u) * a.Hq + h] = (M[j] + log2f(lt[j])) * kLn2;
  }
}

}  // namespace

size_t sk_sched_bytes(int B) { return (((size_t)B + 5) * sizeof(int32_t) + 255) & ~(size_t)255; }

hipError_t launch_attn_sk(const AttnArgs& a, const AttnPlan& p, void* ws, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  const int NV = p.sk_nv, rsplit = p.rsplit, RW = 256;
  SkArgs k;
  k.sched = (int32_t*)ws;
  const size_t sb = sk_sched_bytes(a.B);
  const size_t slots = (size_t)2 * NV * rsplit * RW;
  k.po = (uint16_t*)((char*)ws + sb);
  k.pml = (float*)((char*)ws + sb + ((slots * a.D * sizeof(uint16_t) + 255) & ~(size_t)255));
  k.rsplit = rsplit;
  k.NV = NV;
  k.cap = p.cap;
  const dim3 grid(NV * rsplit), block(512 / kSkQB);
  constexpr int RB = 8 / kSkQB;
  // an fp8 cache has no many-row plan: the host refuses it for more than 128 query rows
  // per KV head, so it cannot reach this launcher
  if (a.kv_fp8) return hipErrorInvalidConfiguration;
  const bool nt = rsplit == 1;
#define TV_SK_LAUNCH(F16, D)                                                                        \
  do {                                                                                              \
    if (nt)                                                                                         \
      hipLaunchKernelGGL((attn_sk_kernel<F16, true, D, kSkQB, RB, 4>), grid, block, 0, s, a, k);  \
    else                                                                                            \
      hipLaunchKernelGGL((attn_sk_kernel<F16, false, D, kSkQB, RB, 4>), grid, block, 0, s, a, k); \
  } while (0)
  if (a.D == 64 && a.f16)
    TV_SK_LAUNCH(true, 64);
  else if (a.D == 64)
    TV_SK_LAUNCH(false, 64);
  else if (a.f16)
    TV_SK_LAUNCH(true, 128);
  else
    TV_SK_LAUNCH(false, 128);
#undef TV_SK_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int chunks = RW / 64;
  if (a.f16)
    hipLaunchKernelGGL(sk_merge_kernel<true>, dim3(a.B * a.Hkv * rsplit * chunks), dim3(256), 0, s, a, k, RW, chunks);
  else
    hipLaunchKernelGGL(sk_merge_kernel<false>, dim3(a.B * a.Hkv * rsplit * chunks), dim3(256), 0, s, a, k, RW,
                       chunks);
  return hipGetLastError();
}

}  // namespace tv
