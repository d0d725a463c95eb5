// Tree attention for bf16 or fp16 inputs on CDNA4 (gfx950): prefix phase, tree phase and
// their online-softmax combination in one kernel, with MFMA for both contractions.
//
// What is computed (SpecInfer explainer, token-tree structure section, attention
// equation): each node u attends, in one softmax, to every cached prefix token of
// its sequence and to exactly the tree nodes of S_u (the precomputed ancestor
// bitmask of the kernel-fusion section).  The prefix is attended by all nodes
// alike, so one workgroup owns a (sequence, KV head, prefix chunk) and streams that
// KV slice from HBM once for all n*G query rows of the GQA group; the tree keys
// follow in the same tile stream with the mask applied.
//
// Data movement: tiles of K and V (token-major, TK keys x D) go HBM -> LDS with
// global_load_lds_dwordx4 into an S-stage ring, S-1 tiles ahead of the compute,
// with the vmcnt waits placed by hand (one barrier per tile, no staging
// registers).  Full prefix tiles use the scalar-base form of the load with
// per-lane offsets computed once; the last prefix tile and the tree tiles take
// per-lane addresses, and lanes whose key lies past the prefix (or whose block
// id is bad) fetch a zero page, so NaN-filled unused cache slots are never read.
//
// Matrix cores (v_mfma_f32_32x32x16_bf16 or _f16, 64-wide waves), one 32-query block per
// wave:
//   S^T = K * Q^T : A = 32 keys x 16 d (ds_read_b128 from the K tile), B = Q^T in
//                   registers; a lane holds the scores of ONE query for 16 keys,
//                   so the softmax max/sum is lane-local plus one lane^32 swap.
//   O^T = V^T * P^T : A = V^T read with ds_read_b64_tr_b16 (the transposing LDS
//                   read of gfx950) straight from the token-major V tile, B = P^T
//                   from the score registers after rounding to the 16-bit type.
//   The QK^T products of a tile's key blocks run as independent accumulator
//   chains stepped together, so back-to-back MFMAs do not wait on each other;
//   the softmax and PV product then go block by block.
//   K rows sit in LDS with bits 2 and 3 of the row index swapped, which makes the
//   8 score registers a lane hands to the PV product 8 consecutive keys.
// The LDS has 64 banks of 4 bytes.  K and V tiles use 16-byte-granule XOR
// swizzles chosen for their read patterns (16 K rows per ds_read_b128 cycle, 4 V
// rows x 4 granules per ds_read_b64_tr_b16 cycle) so operand reads are
// conflict free.  The running max only moves when a block raises it by more than
// 2^8 (exact: the final normalisation uses the same reference), which removes
// almost all accumulator rescales.
#include <float.h>

#include "attn_bf16_common.h"

namespace tv {

// Zeros: the source of every lane (or line) whose key is not to be read.  4 KB
// covers the per-lane offsets of one 16-token paged block line.
__device__ __attribute__((aligned(4096))) uint4 tv_zero_page[256];

namespace {

using namespace attn;

// A lane's value combined with lane (l ^ 32)'s through the gfx950 lane swap (a
// VALU op): the swap of a register with itself leaves the lower half's values in
// every lane of the first result and the upper half's in the second.
__device__ __forceinline__ float max_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int D, int RB, int KS, int TK, int S, bool FP8 = false>
struct Cfg {
  static constexpr int NT = 64 * RB * KS;      // threads per workgroup
  static constexpr int ROWB = 2 * D;           // bytes per token row in LDS
  static constexpr int REG = TK * ROWB;        // bytes of a K (or V) tile region
  static constexpr int GSTAGE = 2 * REG;       // one group's stage: K region, then V region
  static constexpr int STAGE = KS * GSTAGE;
  static constexpr int RING = S * STAGE;
  static constexpr int LINES = GSTAGE / 1024;  // 1 KB DMA lines per group tile
  static constexpr int HL = LINES / 2;         // lines of the K region
  static constexpr int LPW = LINES / RB;       // DMA instructions per wave per tile
  static constexpr int RPL = 1024 / ROWB;      // token rows per line
  static constexpr int GPR = D / 8;            // 16-byte granules per row
  static constexpr int KB = TK / 32;           // 32-key MFMA blocks per tile
  static constexpr int DB = D / 32;            // 32-row d blocks of O^T
  static constexpr int SD = D / 16;            // k-steps of the QK^T product
  // key-split combine: one LDS slot per lane of every wave (O^T values, max, sum),
  // padded to a multiple of 16 bytes so the slots take 128-bit accesses
  static constexpr int SLOT = DB * 16 + 4;
  static constexpr int MERGE = (KS > 1) ? KS * RB * 64 * SLOT * 4 : 0;
  // fp8 cache: the ring stages fp8 tiles (1 byte per element) and one bf16 tile
  // buffer per group (CUR) holds the converted tile the MFMAs read
  static constexpr int GSTAGE8 = 2 * TK * D;
  static constexpr int STAGE8 = KS * GSTAGE8;
  static constexpr int LINES8 = GSTAGE8 / 1024;
  static constexpr int HL8 = LINES8 / 2;
  static constexpr int LPW8 = LINES8 / RB;
  static constexpr int RPL8 = 1024 / D;  // token rows per fp8 line
  static constexpr int GPR8 = D / 16;    // 16-byte granules per fp8 row
  static constexpr int CUR = KS * GSTAGE;
  static constexpr int USED = FP8 ? S * STAGE8 + CUR : RING;
  static constexpr int LDS = USED > MERGE ? USED : MERGE;
  static constexpr int WAITN = (S - 2) * (FP8 ? LPW8 : LPW);  // loads a wave may leave in flight
  static_assert(HL % RB == 0 && LPW * (S - 2) < 64, "pipeline shape");
  static_assert(!FP8 || (HL8 % RB == 0 && LPW8 * (S - 2) < 64), "fp8 pipeline shape");
  static_assert(TK % 32 == 0 && TK <= 64 && 16 % RPL == 0, "tile");
};

__device__ __forceinline__ uint32_t pick32(uint64_t w0, uint64_t w1, uint64_t w2, uint64_t w3, int half) {
  const int w = half >> 1;
  const uint64_t x = w == 0 ? w0 : (w == 1 ? w1 : (w == 2 ? w2 : w3));
  return (half & 1) ? (uint32_t)(x >> 32) : (uint32_t)x;
}

template <bool F16, bool FP8, int D, int RB, int KS, int TK, int S>
__global__ __launch_bounds__(64 * RB * KS) void attn_bf16_kernel(AttnArgs a, int rsplit, int nchunks,
                                                                 int chunk_len, int cap) {
  using C = Cfg<D, RB, KS, TK, S, FP8>;
  using E = Elt<F16>;
  using V8 = typename E::V8;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
  const int rb = wave % RB, ks = wave / RB;
  const int col = lane & 31, hh = lane >> 5;
  const int n = a.n, G = a.G, Hkv = a.Hkv, rows = n * G;

  // XCD-aware order: consecutive logical ids land on the same XCD (shared L2).
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int per = nwg >> 3, rem = nwg & 7, xcd = wg & 7;
  const int lid = xcd * per + min(xcd, rem) + (wg >> 3);
  const int rs = lid % rsplit;
  int t = lid / rsplit;
  const int c = t % nchunks;
  t /= nchunks;
  const int g = t % Hkv;
  const int b = t / Hkv;

  const int Lraw = a.plen[b];  // its latency overlaps the speculative issue below
  const char* kc = (const char*)a.kc;
  const char* vc = (const char*)a.vc;
  const char* ktr = (const char*)a.kt;
  const char* vtr = (const char*)a.vt;
  const char* zero = (const char*)tv_zero_page;
  // Full prefix tiles: with at most 4 row waves the plan has one row slice, so every
  // tile is read by exactly one workgroup and streams non-temporal (each line is read
  // once); the 8-row-wave plan may split rows over workgroups that share the tiles.
  auto dma_full = [](const void* sbase, uint32_t voff, uint32_t lds_line) {
    if constexpr (RB <= 4)
      dma16s_nt(sbase, voff, lds_line);
    else
      dma16s(sbase, voff, lds_line);
  };
  const uint32_t ring = (uint32_t)(uintptr_t)(AS3 void*)smem;
  const size_t rowbase = ((size_t)b * Hkv + g) * a.Lmax;  // contiguous cache row of token 0

  // ---- per-lane DMA geometry: line q*RB + rb of the group tile belongs to this
  // wave; the first HL lines are the K region, so whether slot q loads K or V is
  // known at compile time.
  int lrow_[C::LPW], gran_[C::LPW];
  uint32_t voff[C::LPW];  // byte offset of this lane's granule from the line's base (full tiles)
#pragma unroll
  for (int q = 0; q < C::LPW; ++q) {
    const bool isv = q * RB >= C::HL;
    const int line = q * RB + rb;
    const int lrow = (isv ? line - C::HL : line) * C::RPL + lane / C::GPR;
    const int pg = lane % C::GPR;
    const int gran = isv ? (pg ^ vswz<D>(lrow)) : (pg ^ kswz<D>(lrow));
    const int key = isv ? lrow : perm_row(lrow);
    lrow_[q] = lrow;
    gran_[q] = gran;
    voff[q] = (uint32_t)(((a.paged ? (key & 15) : key) * D + gran * 8) * 2);
  }

  // Contiguous cache: the first ring tiles of this wave's group are issued as full
  // prefix tiles before the prefix length arrives (their addresses do not depend
  // on it, and each lies inside the cache row of Lmax tokens); the prologue below
  // issues again any that turn out partial, tree tiles or past the end, which
  // overwrites the same LDS lines (a wave's DMA lines land in issue order).  Not in
  // the workgroups that check the sequence's status (they use the ring's first
  // word as a flag first), nor with an fp8 cache.
  const bool spec = !FP8 && !a.paged && !(a.status != nullptr && c == 0 && rs == 0 && g == 0);
  auto spec_tile = [&](int i) { return spec && c * chunk_len + (i * KS + ks) * TK + TK <= cap; };
#pragma unroll
  for (int i = 0; i < S - 1; ++i) {
    if (spec_tile(i)) {
      const int tstart = c * chunk_len + (i * KS + ks) * TK;
      const char* kb = kc + (rowbase + tstart) * D * 2;
      const char* vb = vc + (rowbase + tstart) * D * 2;
      const uint32_t gbase = ring + i * C::STAGE + ks * C::GSTAGE;
#pragma unroll
      for (int q = 0; q < C::LPW; ++q)
        dma_full(q * RB >= C::HL ? vb : kb, voff[q], gbase + (q * RB + rb) * 1024);
    }
  }

  const int L = Lraw < 0 ? 0 : (Lraw > cap ? cap : Lraw);
  const AS4 int32_t* btc = (const AS4 int32_t*)a.bt;

  if (a.status != nullptr && c == 0 && rs == 0 && g == 0) {
    int bad = (Lraw < 0 || Lraw > cap);
    if (a.paged) {
      const int nb = (L + TV_PAGE - 1) / TV_PAGE;
      for (int i = tid; i < nb; i += C::NT) {
        const int id = a.bt[(size_t)b * a.max_blocks + i];
        bad |= (id < 0 || id >= a.num_blocks);
      }
    }
    // workgroup OR through the first LDS word (the ring is not in use yet), so
    // the kernel needs no LDS beyond its ring
    int AS3* flag = (int AS3*)smem;
    if (tid == 0) *flag = 0;
    __syncthreads();
    if (bad) *flag = 1;
    __syncthreads();
    bad = *flag;
    __syncthreads();  // read by every thread before the ring is written
    if (tid == 0) a.status[b] = bad ? TV_EINVAL : TV_OK;
  }

  const int k0 = c * chunk_len;
  const int k1 = min(L, k0 + chunk_len);
  const int npre = k1 > k0 ? k1 - k0 : 0;
  const bool has_tree = (c == 0);
  if (npre == 0 && !has_tree) {  // empty chunk (uniform per workgroup)
    wait_vmcnt<0>();              // speculative lines land before the workgroup's LDS is released
    return;
  }
  const int nc_b = L > 0 ? (L + chunk_len - 1) / chunk_len : 1;
  const bool direct = (nc_b == 1);

  const int T_pre = (npre + TK - 1) / TK;
  const int T = T_pre + (has_tree ? (n + TK - 1) / TK : 0);
  const int iters = (T + KS - 1) / KS;


  // ---- issue the DMA lines this wave owns for tile tt of its group into stage st
  auto issue = [=](int tt, int st) {
    // (fp8 cache: only tree tiles come here, into the group's bf16 buffer)
    const uint32_t gbase = FP8 ? ring + S * C::STAGE8 + ks * C::GSTAGE : ring + st * C::STAGE + ks * C::GSTAGE;
    const char* zsrc = zero + lane * 16;
    if (tt >= T) {  // past the end: keep the vmcnt bookkeeping uniform with zero-page loads
#pragma unroll
      for (int q = 0; q < C::LPW; ++q) dma16(zsrc, gbase + (q * RB + rb) * 1024);
      return;
    }
    if (tt >= T_pre) {  // tree tile: token-major K_tree / V_tree rows, per-lane addresses
      const int tstart = (tt - T_pre) * TK;
#pragma unroll
      for (int q = 0; q < C::LPW; ++q) {
        const bool isv = q * RB >= C::HL;
        const int v = tstart + (isv ? lrow_[q] : perm_row(lrow_[q]));
        const char* src = (isv ? vtr : ktr) + ((((size_t)b * n + v) * Hkv + g) * D + gran_[q] * 8) * 2;
        dma16(v < n ? src : zsrc, gbase + (q * RB + rb) * 1024);
      }
      return;
    }
    const int tstart = k0 + tt * TK;
    const bool full = tstart + TK <= k1;
    if (a.paged) {
      // block ids of the tile's 16-token blocks (uniform: scalar loads)
      const int b0 = tstart >> 4;
      const AS4 int32_t* row = btc + (size_t)b * a.max_blocks;
      const int id0 = b0 < a.max_blocks ? row[b0] : -1;
      const int id1 = b0 + 1 < a.max_blocks ? row[b0 + 1] : -1;
      const int id2 = (TK > 32 && b0 + 2 < a.max_blocks) ? row[b0 + 2] : -1;
      const int id3 = (TK > 32 && b0 + 3 < a.max_blocks) ? row[b0 + 3] : -1;
#pragma unroll
      for (int q = 0; q < C::LPW; ++q) {
        const bool isv = q * RB >= C::HL;
        const int line = q * RB + rb;
        const int kq = ((isv ? line - C::HL : line) * C::RPL) >> 4;  // 16-token block of the whole line
        const int blk = kq == 0 ? id0 : (kq == 1 ? id1 : (kq == 2 ? id2 : id3));
        const bool bok = blk >= 0 && blk < a.num_blocks;
        const char* lbase = (isv ? vc : kc) + ((size_t)blk * Hkv + g) * TV_PAGE * D * 2;
        if (full) {
          dma_full(bok ? lbase : zero, voff[q], gbase + line * 1024);
        } else {
          const int j = tstart + (isv ? lrow_[q] : perm_row(lrow_[q]));
          dma16(bok && j < k1 ? lbase + voff[q] : zsrc, gbase + line * 1024);
        }
      }
    } else {
      const char* kb = kc + (rowbase + tstart) * D * 2;
      const char* vb = vc + (rowbase + tstart) * D * 2;
#pragma unroll
      for (int q = 0; q < C::LPW; ++q) {
        const bool isv = q * RB >= C::HL;
        const int line = q * RB + rb;
        if (full) {
          dma_full(isv ? vb : kb, voff[q], gbase + line * 1024);
        } else {
          const int j = tstart + (isv ? lrow_[q] : perm_row(lrow_[q]));
          dma16(j < k1 ? (isv ? vb : kb) + voff[q] : zsrc, gbase + line * 1024);
        }
      }
    }
  };

  // ---- fp8 cache: prefix tiles go through an fp8 ring; each wave converts the
  // lines it loaded into the group's bf16 tile buffer (codes, unscaled), at the
  // positions the bf16 layout above gives each key row and granule
  const uint32_t cur = ring + (FP8 ? S * C::STAGE8 : 0) + ks * C::GSTAGE;  // bf16 tile buffer of the group
  auto issue8 = [=](int tt, int st) {
    const uint32_t gbase = ring + st * C::STAGE8 + ks * C::GSTAGE8;
    const char* zsrc = zero + lane * 16;
    if (tt >= T_pre) {  // past the end, or a tree tile (loaded into the buffer when consumed)
#pragma unroll
      for (int q = 0; q < C::LPW8; ++q) dma16(zsrc, gbase + (q * RB + rb) * 1024);
      return;
    }
    const int tstart = k0 + tt * TK;
    const bool full = tstart + TK <= k1;
    const int gran = lane % C::GPR8;
    int id[4] = {-1, -1, -1, -1};
    if (a.paged) {
      const int b0 = tstart >> 4;
      const AS4 int32_t* row = btc + (size_t)b * a.max_blocks;
#pragma unroll
      for (int i = 0; i < (TK + 15) / 16; ++i) id[i] = b0 + i < a.max_blocks ? row[b0 + i] : -1;
    }
#pragma unroll
    for (int q = 0; q < C::LPW8; ++q) {
      const int line = q * RB + rb;
      const bool isv = line >= C::HL8;
      const int r = (isv ? line - C::HL8 : line) * C::RPL8 + lane / C::GPR8;  // key row within the tile
      const int j = tstart + r;
      const char* src;
      bool ok = full || j < k1;
      if (a.paged) {
        const int blk = id[r >> 4];
        ok = ok && blk >= 0 && blk < a.num_blocks;
        src = (isv ? vc : kc) + (((size_t)blk * Hkv + g) * TV_PAGE + (j & 15)) * D + gran * 16;
      } else {
        src = (isv ? vc : kc) + (rowbase + j) * D + gran * 16;
      }
      dma16(ok ? src : zsrc, gbase + line * 1024);
    }
  };
  auto convert8 = [=](int st) {
    const uint32_t gbase = ring + st * C::STAGE8 + ks * C::GSTAGE8;
    const int gran = lane % C::GPR8;
#pragma unroll
    for (int q = 0; q < C::LPW8; ++q) {
      const int line = q * RB + rb;
      const bool isv = line >= C::HL8;
      const int r = (isv ? line - C::HL8 : line) * C::RPL8 + lane / C::GPR8;
      const u32x4 x = *(const u32x4 AS3*)((const char AS3*)(smem) + (gbase - ring) + line * 1024 + lane * 16);
      u32x4 lo, hi;  // bf16 elements 0..7 and 8..15 of the 16 fp8 codes (exact: E4M3 fits bf16)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t src = x[w];
        // scale 1: the instruction's scale operand acts as a power of two only
        // (an E8M0 block scale), so the per-tensor scales are applied to the
        // scores and probabilities instead
        const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, false);
        const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src, 1.0f, true);
        const uint32_t w0 = __builtin_bit_cast(uint32_t, p0), w1 = __builtin_bit_cast(uint32_t, p1);
        if (w < 2) {
          lo[2 * w] = w0;
          lo[2 * w + 1] = w1;
        } else {
          hi[2 * (w - 2)] = w0;
          hi[2 * (w - 2) + 1] = w1;
        }
      }
      const int lrow = isv ? r : perm_row(r);  // K rows sit at perm_row(key)
      const int sw = isv ? vswz<D>(lrow) : kswz<D>(lrow);
      char AS3* rb0 = (char AS3*)(smem) + (cur - ring) + (isv ? C::REG : 0) + lrow * C::ROWB;
      *(u32x4 AS3*)(rb0 + (((2 * gran) ^ sw) << 4)) = lo;
      *(u32x4 AS3*)(rb0 + (((2 * gran + 1) ^ sw) << 4)) = hi;
    }
  };

  // ---- this lane's query column: operand registers and ancestor mask
  const int qrow = rs * 32 * RB + 32 * rb + col;
  const bool qvalid = qrow < rows;
  V8 qop[C::SD];
  uint64_t mw0 = 0, mw1 = 0, mw2 = 0, mw3 = 0;
  {
    const int u = qvalid ? qrow / G : 0, gi = qvalid ? qrow % G : 0;
    const uint16_t* qp = (const uint16_t*)a.q + ((size_t)(b * n + u) * a.Hq + g * G + gi) * D;
#pragma unroll
    for (int sd = 0; sd < C::SD; ++sd) {
      u32x4 v = {0, 0, 0, 0};
      if (qvalid) v = *(const u32x4*)(qp + 16 * sd + 8 * hh);
      qop[sd] = __builtin_bit_cast(V8, v);
    }
    if (qvalid) {
      const uint64_t* mp = a.mask + ((size_t)b * n + u) * a.W;
      mw0 = mp[0];
      if (a.W > 1) mw1 = mp[1];
      if (a.W > 2) mw2 = mp[2];
      if (a.W > 3) mw3 = mp[3];
    }
  }

  // ---- per-lane LDS read offsets (the key-block and stage parts are added later)
  uint32_t kofs[C::SD], vofs[C::DB];
#pragma unroll
  for (int sd = 0; sd < C::SD; ++sd) kofs[sd] = col * C::ROWB + (((2 * sd + hh) ^ kswz<D>(col)) << 4);
  {
    const int l16 = lane & 15, mhalf = (lane >> 4) & 1;
    const int vr = 8 * hh + (l16 >> 2);  // row within a 16-key half block (multiples of 4 added later)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int lg = 4 * db + 2 * mhalf + ((lane & 3) >> 1);
      vofs[db] = vr * C::ROWB + ((lg ^ vswz<D>(vr)) << 4) + ((lane & 1) << 3);
    }
  }

  f32x16 O[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[db][r] = 0.f;
  float m_run = -INFINITY, lsum = 0.f;
  const float sl2 = a.scale_log2;

  // prologue: S-1 tiles in flight, issued before the query loads have returned
  // so the two latencies overlap; the full wait (which the compiler can see)
  // then leaves no load of its own pending inside the loop
#pragma unroll
  for (int i = 0; i < S - 1; ++i) {
    const int tt = i * KS + ks;
    if constexpr (FP8) {
      issue8(tt, i);
    } else {
      // a speculated tile stands if it is a full prefix tile of this chunk
      if (!(spec_tile(i) && tt < T_pre && k0 + tt * TK + TK <= k1)) issue(tt, i);
    }
  }
  wait_vmcnt<0>();

  for (int it = 0; it < iters; ++it) {
    wait_vmcnt<C::WAITN>();  // this wave's lines of iteration `it` have landed
    // With one wave per key-split group a wave only reads the ring region it
    // filled itself (its own vmcnt wait covers it, and its reads of the stage it
    // refills next were consumed last iteration), so it runs without barriers.
    if constexpr (RB > 1) lds_barrier();  // ... everyone's, and everyone left iteration it-1
    const int tt = it * KS + ks;
    if constexpr (FP8) {
      issue8((it + S - 1) * KS + ks, (it + S - 1) % S);
      if (tt < T) {
        if (tt >= T_pre) {  // tree tile (bf16): straight into the buffer, waited here
          issue(tt, 0);  // the tree branch of issue() takes the buffer as its stage base below
          wait_vmcnt<0>();
        } else {
          convert8(it % S);
        }
      }
      if constexpr (RB > 1) lds_barrier();  // the buffer holds the whole tile
    } else {
      issue((it + S - 1) * KS + ks, (it + S - 1) % S);
    }

    if (tt < T) {
      const int st = it % S;
      const char AS3* Kr = (const char AS3*)(smem) + (FP8 ? cur - ring : st * C::STAGE + ks * C::GSTAGE);
      const char AS3* Vr = Kr + C::REG;
      const bool tree = tt >= T_pre;
      const int tstart = tree ? (tt - T_pre) * TK : k0 + tt * TK;
      const int lim = tree ? n - tstart : k1 - tstart;  // keys of this tile that exist
      const bool full = !tree && lim >= TK;
      // fp8 prefix tiles hold unscaled codes: the key scale joins the score scale
      // and the value scale multiplies the probabilities entering the PV product
      // (the row sum keeps the plain probabilities)
      const float slt = (FP8 && !tree) ? sl2 * a.k_scale : sl2;
      const float vsc = (FP8 && !tree) ? a.v_scale : 1.f;

      // QK^T of the tile's key blocks as independent accumulator chains, stepped
      // together over the head dimension, so consecutive MFMAs never wait on each
      // other and each K operand read has a full step of lead time.  A single
      // 32-key block uses two half-sum chains (even / odd steps) instead.
      f32x16 Sacc[C::KB > 1 ? C::KB : 2];
#pragma unroll
      for (int i = 0; i < (C::KB > 1 ? C::KB : 2); ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) Sacc[i][r] = 0.f;
#pragma unroll
      for (int sd = 0; sd < C::SD; ++sd) {
        if constexpr (C::KB > 1) {
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) {
            const V8 kop = *(const V8 AS3*)(Kr + kb * 32 * C::ROWB + kofs[sd]);
            Sacc[kb] = E::mfma(kop, qop[sd], Sacc[kb]);
          }
        } else {
          const V8 kop = *(const V8 AS3*)(Kr + kofs[sd]);
          Sacc[sd & 1] = E::mfma(kop, qop[sd], Sacc[sd & 1]);
        }
      }
      if constexpr (C::KB == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) Sacc[0][r] += Sacc[1][r];
      }

#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        f32x16 Scur = Sacc[kb];
        // ---- mask (uniform choice of mode per tile) and block max
        float mx = -INFINITY;
        if (full) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, Scur[r]);
        } else if (!tree) {  // last prefix tile: keys past the prefix end
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = kb * 32 + 16 * (r >> 3) + 8 * hh + (r & 7);
            Scur[r] = ko < lim ? Scur[r] : -INFINITY;
            mx = fmaxf(mx, Scur[r]);
          }
        } else {  // tree tile: ancestor bits of this lane's node
          const uint32_t bits = pick32(mw0, mw1, mw2, mw3, (tstart + kb * 32) >> 5) >> (8 * hh);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = kb * 32 + 16 * (r >> 3) + 8 * hh + (r & 7);
            const bool ok = ko < lim && ((bits >> (16 * (r >> 3) + (r & 7))) & 1u);
            Scur[r] = ok ? Scur[r] : -INFINITY;
            mx = fmaxf(mx, Scur[r]);
          }
        }
        mx = max_xor32(mx) * slt;  // scale > 0 commutes with max
        if (__any(mx > m_run + kTau)) {
          const float m_new = fmaxf(m_run, mx);
          const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[db][r] *= alpha;
          m_run = m_new;
        }
        const float msub = (m_run == -INFINITY) ? 0.f : m_run;
        V8 pop[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Scur[r], slt, -msub));
          lsum += p;
          pop[r >> 3][r & 7] = E::cvt(FP8 ? p * vsc : p);
        }
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const char AS3* vp = Vr + (kb * 32 + 16 * half) * C::ROWB + vofs[db];
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 AS3*)vp);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 AS3*)(vp + 4 * C::ROWB));
            const s16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            O[db] = E::mfma(__builtin_bit_cast(V8, v8), pop[half], O[db]);
          }
      }
    }
  }
  wait_vmcnt<0>();  // drain the trailing zero-page loads before LDS is reused or released

  // ---- combine the key-split groups of each query block. Every group leaves its
  // partial output (unnormalised O^T columns, running max, partial sum) in LDS; then
  // the whole workgroup shares the rescale-and-sum and the stores: one work item is
  // 8 consecutive d of one query row, so 16 threads write a row as 16-byte pieces.
  if constexpr (KS > 1) {
    lds_barrier();
    float* mb = (float*)smem;
    {
      float* dst = mb + ((ks * RB + rb) * 64 + lane) * C::SLOT;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *(float4*)(dst + db * 16 + 4 * rq) = make_float4(O[db][4 * rq], O[db][4 * rq + 1], O[db][4 * rq + 2], O[db][4 * rq + 3]);
      *(float2*)(dst + C::DB * 16) = make_float2(m_run, lsum);  // the max is the same on both half-lanes
    }
    lds_barrier();
    constexpr int CPR = D / 8;  // 8-value pieces per row
    for (int it = tid; it < 32 * RB * CPR; it += C::NT) {
      const int rr = it / CPR, ch = it % CPR;
      const int qr = rs * 32 * RB + rr;
      if (qr >= rows) break;  // rows grow with it: every later item is past the end too
      const float* s0 = mb + ((rr >> 5) * 64 + (rr & 31)) * C::SLOT;  // half-lane 0 of group 0
      constexpr int KSTEP = RB * 64 * C::SLOT, HSTEP = 32 * C::SLOT;
      float M = -INFINITY;
#pragma unroll
      for (int k = 0; k < KS; ++k) M = fmaxf(M, s0[k * KSTEP + C::DB * 16]);
      float lt = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const int off = (ch >> 2) * 16 + 4 * (ch & 3);  // O[db][4 rq ..]: db = ch / 4, rq = ch % 4
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const float* sk = s0 + k * KSTEP;
        const float mk = sk[C::DB * 16];
        const float wk = (mk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk - M);
        lt += wk * (sk[C::DB * 16 + 1] + sk[HSTEP + C::DB * 16 + 1]);
        const float4 lo = *(const float4*)(sk + off), hi = *(const float4*)(sk + HSTEP + off);
        acc[0] += wk * lo.x; acc[1] += wk * lo.y; acc[2] += wk * lo.z; acc[3] += wk * lo.w;
        acc[4] += wk * hi.x; acc[5] += wk * hi.y; acc[6] += wk * hi.z; acc[7] += wk * hi.w;
      }
      const int u = qr / G, gi = qr % G, h = g * G + gi;
      if (direct) {
        const float inv = 1.f / lt;
        uint4 w;
        w.x = E::bits(acc[0] * inv) | (E::bits(acc[1] * inv) << 16);
        w.y = E::bits(acc[2] * inv) | (E::bits(acc[3] * inv) << 16);
        w.z = E::bits(acc[4] * inv) | (E::bits(acc[5] * inv) << 16);
        w.w = E::bits(acc[6] * inv) | (E::bits(acc[7] * inv) << 16);
        *(uint4*)((uint16_t*)a.out + ((size_t)(b * n + u) * a.Hq + h) * D + 8 * ch) = w;
        if (a.lse != nullptr && ch == 0) a.lse[(size_t)(b * n + u) * a.Hq + h] = (M + __log2f(lt)) * kLn2;
      } else {
        const size_t pidx = ((size_t)(b * Hkv + g) * nchunks + c) * rows + qr;
        float* wo = a.ws_o + pidx * D + 8 * ch;
        *(float4*)wo = make_float4(acc[0], acc[1], acc[2], acc[3]);
        *(float4*)(wo + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
        if (ch == 0) {
          a.ws_ml[2 * pidx] = M;
          a.ws_ml[2 * pidx + 1] = lt;
        }
      }
    }
    return;
  }

  const float ltot = sum_xor32(lsum);
  if (!qvalid) return;
  const int u = qrow / G, gi = qrow % G, h = g * G + gi;
  if (direct) {
    const float inv = 1.f / ltot;
    uint16_t* op = (uint16_t*)a.out + ((size_t)(b * n + u) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * db + 8 * rq + 4 * hh;
        uint2 w;
        w.x = E::bits(O[db][4 * rq] * inv) | (E::bits(O[db][4 * rq + 1] * inv) << 16);
        w.y = E::bits(O[db][4 * rq + 2] * inv) | (E::bits(O[db][4 * rq + 3] * inv) << 16);
        *(uint2*)(op + d0) = w;
      }
    if (a.lse != nullptr && hh == 0) a.lse[(size_t)(b * n + u) * a.Hq + h] = (m_run + __log2f(ltot)) * kLn2;
  } else {
    const size_t pidx = ((size_t)(b * Hkv + g) * nchunks + c) * rows + qrow;
    float* wo = a.ws_o + pidx * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = 32 * db + 8 * rq + 4 * hh;
        *(float4*)(wo + d0) = make_float4(O[db][4 * rq], O[db][4 * rq + 1], O[db][4 * rq + 2], O[db][4 * rq + 3]);
      }
    if (hh == 0) {
      a.ws_ml[2 * pidx] = m_run;
      a.ws_ml[2 * pidx + 1] = ltot;
    }
  }
}

// KS8, S8, TK8: key-split groups, ring depth and tile keys of the fp8 variant; its
// stages are half the size, so the same LDS holds more groups (waves) or more tiles
template <int D, int RB, int KS, int TK, int S, int KS8, int S8, int TK8 = TK>
hipError_t launch_cfg(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  const int grid = a.B * a.Hkv * p.nchunks * p.rsplit;
  if (grid == 0) return hipSuccess;
  if (a.kv_fp8) {
    if constexpr (RB <= 4)
      hipLaunchKernelGGL((attn_bf16_kernel<false, true, D, RB, KS8, TK8, S8>), dim3(grid), dim3(64 * RB * KS8), 0,
                         s, a, p.rsplit, p.nchunks, p.chunk_len, p.cap);
    else
      return hipErrorInvalidConfiguration;  // the host never plans this
  } else if (a.f16)
    hipLaunchKernelGGL((attn_bf16_kernel<true, false, D, RB, KS, TK, S>), dim3(grid), dim3(64 * RB * KS), 0, s, a, p.rsplit,
                       p.nchunks, p.chunk_len, p.cap);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<false, false, D, RB, KS, TK, S>), dim3(grid), dim3(64 * RB * KS), 0, s, a,
                       p.rsplit, p.nchunks, p.chunk_len, p.cap);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  if (p.rb == 1) return launch_cfg<D, 1, 5, 32, 2, 5, 2>(a, p, s);
  if (p.rb == 2) return launch_cfg<D, 2, 4, 32, 2, 4, 3>(a, p, s);
  if (p.rb == 4) return launch_cfg<D, 4, 2, 32, 4, 2, 3, 64>(a, p, s);
  return launch_cfg<D, 8, 1, 64, 4, 1, 4>(a, p, s);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  return a.D == 64 ? launch_d<64>(a, p, s) : launch_d<128>(a, p, s);
}

}  // namespace tv
