// Tree attention for bf16 inputs on CDNA4 (gfx950): prefix phase, tree phase and
// their online-softmax combination in one kernel, with MFMA for both contractions.
//
// What is computed (SpecInfer explainer, token-tree structure section, attention
// equation): each node u attends, in one softmax, to every cached prefix token of
// its sequence and to exactly the tree nodes of S_u (the precomputed ancestor
// bitmask of the kernel-fusion section).  The prefix is attended by all nodes
// alike, so one workgroup owns a (sequence, KV head, prefix chunk) and streams that
// KV slice from HBM exactly once for all n*G query rows of the GQA group; the
// tree keys follow in the same loop with the mask applied, so no separate
// tree-phase pass or extra partial is needed.
//
// Mapping onto the matrix cores (v_mfma_f32_32x32x16_bf16, 64-wide waves):
//   S^T = K * Q^T : A = 32 keys x 16 d (from LDS), B = Q^T (registers, 32 queries),
//                   so each lane holds the scores of ONE query column for 16 keys
//                   and the softmax max/sum is lane-local plus one lane^32 swap.
//   O^T = V^T * P^T : A = V^T (d x keys, from the d-major V tile in LDS),
//                   B = P^T straight from the score registers after bf16 rounding.
//   K rows are stored in LDS with bits 2 and 3 of the row index swapped, which
//   makes the 8 score registers a lane hands to the PV product cover 8
//   consecutive keys, so the matching V operand is one 16-byte LDS read.
// Both tiles use 16-byte-granule XOR swizzles so the MFMA operand reads and the
// tile writes are bank-conflict free.  Global loads are register-staged into a
// double-buffered LDS ring (one barrier per tile).  The running max is only moved
// when a tile raises it by more than 2^8 (exact: the final normalisation uses the
// same reference), which removes almost all accumulator rescales.
#include <float.h>

#include "tv_internal.h"

namespace tv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kTau = 8.0f;  // lazy-rescale threshold in the log2 domain

__device__ __forceinline__ int perm_row(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

template <int D, int RB, int KS, int TK>
struct Cfg {
  static constexpr int NT = 64 * RB * KS;         // threads per workgroup
  static constexpr int TKT = TK * KS;             // keys per tile
  static constexpr int KSLAB = TK * D * 2;        // bytes of one wave's K slab  [TK][D]
  static constexpr int VSLAB = D * TK * 2;        // bytes of one wave's V slab  [D][TK]
  static constexpr int STAGE = KS * (KSLAB + VSLAB);
  static constexpr int CH = TKT * D / 8;          // 16-byte chunks in a K (or V) tile
  static constexpr int PER = (CH + NT - 1) / NT;  // chunks per thread
  static constexpr int KB = TK / 32;              // 32-key MFMA blocks per wave tile
  static constexpr int DB = D / 32;               // 32-row d blocks of O^T
  static constexpr int SD = D / 16;               // k-steps of the QK^T product
  static constexpr int VG = TK / 8;               // 16-byte granules per V slab row
  static constexpr int MERGE = (KS > 1) ? (KS - 1) * RB * 64 * 66 * 4 : 0;
  static constexpr int LDS = (2 * STAGE > MERGE) ? 2 * STAGE : MERGE;
  static_assert(TK % 32 == 0 && VG >= 4, "tile");
};

__device__ __forceinline__ uint64_t pick(uint64_t a0, uint64_t a1, uint64_t a2, uint64_t a3, int w) {
  return w == 0 ? a0 : (w == 1 ? a1 : (w == 2 ? a2 : a3));
}

template <int D, int RB, int KS, int TK>
__global__ __launch_bounds__(64 * RB * KS) void attn_bf16_kernel(AttnArgs a, int rsplit, int nchunks,
                                                                 int chunk_len, int cap) {
  using C = Cfg<D, RB, KS, TK>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  const int Lraw = a.plen[b];
  const int L = Lraw < 0 ? 0 : (Lraw > cap ? cap : Lraw);

  if (a.status != nullptr && c == 0 && rs == 0 && g == 0) {
    int bad = (Lraw < 0 || Lraw > cap);
    if (a.paged) {
      const int nb = (L + TV_PAGE - 1) / TV_PAGE;
      for (int i = tid; i < nb; i += C::NT) {
        const int id = a.bt[(size_t)b * a.max_blocks + i];
        bad |= (id < 0 || id >= a.num_blocks);
      }
    }
    bad = __syncthreads_or(bad);
    if (tid == 0) a.status[b] = bad ? TV_EINVAL : TV_OK;
  }

  const int k0 = c * chunk_len;
  const int k1 = min(L, k0 + chunk_len);
  const int npre = k1 > k0 ? k1 - k0 : 0;
  const bool has_tree = (c == 0);
  if (npre == 0 && !has_tree) return;  // empty chunk (uniform per workgroup)
  const int nc_b = L > 0 ? (L + chunk_len - 1) / chunk_len : 1;
  const bool direct = (nc_b == 1);

  const int T_pre = (npre + C::TKT - 1) / C::TKT;
  const int T_tree = has_tree ? (n + C::TKT - 1) / C::TKT : 0;
  const int T = T_pre + T_tree;

  const uint16_t* __restrict__ kc = (const uint16_t*)a.kc;
  const uint16_t* __restrict__ vc = (const uint16_t*)a.vc;
  const uint16_t* __restrict__ ktr = (const uint16_t*)a.kt;
  const uint16_t* __restrict__ vtr = (const uint16_t*)a.vt;

  // ---- this lane's query column: operand registers and ancestor mask
  const int qrow = rs * 32 * RB + 32 * rb + col;
  const bool qvalid = qrow < rows;
  bf16x8 qop[C::SD];
  uint64_t mw0 = 0, mw1 = 0, mw2 = 0, mw3 = 0;
  {
    const int u = qvalid ? qrow / G : 0, gi = qvalid ? qrow % G : 0;
    const uint16_t* qp = (const uint16_t*)a.q + ((size_t)(b * n + u) * a.Hq + g * G + gi) * D;
#pragma unroll
    for (int sd = 0; sd < C::SD; ++sd) {
      u32x4 v = {0, 0, 0, 0};
      if (qvalid) v = *(const u32x4*)(qp + 16 * sd + 8 * hh);
      qop[sd] = __builtin_bit_cast(bf16x8, v);
    }
    if (qvalid) {
      const uint64_t* mp = a.mask + ((size_t)b * n + u) * a.W;
      mw0 = mp[0];
      if (a.W > 1) mw1 = mp[1];
      if (a.W > 2) mw2 = mp[2];
      if (a.W > 3) mw3 = mp[3];
    }
  }

  u32x4 kreg[C::PER], vreg[C::PER];

  auto kv_base_contig = [&](void) { return (size_t)(b * Hkv + g); };

  auto load_tile = [&](int tt) {
    if (tt < T_pre) {
      const int kt0 = k0 + tt * C::TKT;
#pragma unroll
      for (int i = 0; i < C::PER; ++i) {
        const int ch = tid + i * C::NT;
        u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
        if (ch < C::CH) {
          {  // K: chunk -> (key, 8-wide d granule), 16 consecutive lanes read one 256-byte row
            const int key = ch / (D / 8), dg = ch % (D / 8);
            const int j = kt0 + key;
            if (j < k1) {
              const uint16_t* p = nullptr;
              if (a.paged) {
                const int blk = a.bt[(size_t)b * a.max_blocks + (j >> 4)];
                if (blk >= 0 && blk < a.num_blocks)
                  p = kc + (((size_t)blk * Hkv + g) * TV_PAGE + (j & 15)) * D + dg * 8;
              } else {
                p = kc + (kv_base_contig() * a.Lmax + j) * D + dg * 8;
              }
              if (p) kv = *(const u32x4*)p;
            }
          }
          {  // V (d-major cache): chunk -> (d row, 8-token granule)
            const int d = ch / (C::TKT / 8), kg = ch % (C::TKT / 8);
            const int j0 = kt0 + kg * 8;
            if (j0 < k1) {
              const uint16_t* p = nullptr;
              if (a.paged) {
                const int blk = a.bt[(size_t)b * a.max_blocks + (j0 >> 4)];
                if (blk >= 0 && blk < a.num_blocks)
                  p = vc + (((size_t)blk * Hkv + g) * D + d) * TV_PAGE + (j0 & 15);
              } else {
                p = vc + (kv_base_contig() * D + d) * a.Lmax + j0;
              }
              if (p) {
                vv = *(const u32x4*)p;
                const int valid = k1 - j0;  // tokens past the prefix may hold NaN: select zero
                if (valid < 8) {
#pragma unroll
                  for (int e = 0; e < 8; ++e)
                    if (e >= valid) vv[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
                }
              }
            }
          }
        }
        kreg[i] = kv;
        vreg[i] = vv;
      }
    } else {
      const int v0 = (tt - T_pre) * C::TKT;
#pragma unroll
      for (int i = 0; i < C::PER; ++i) {
        const int ch = tid + i * C::NT;
        u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
        if (ch < C::CH) {
          const int key = ch / (D / 8), dg = ch % (D / 8);
          const int v = v0 + key;
          if (v < n) {
            const size_t off = (((size_t)b * n + v) * Hkv + g) * D + dg * 8;
            kv = *(const u32x4*)(ktr + off);
            vv = *(const u32x4*)(vtr + off);
          }
        }
        kreg[i] = kv;
        vreg[i] = vv;
      }
    }
  };

  auto store_tile = [&](int stage, int tt) {
    char* base = smem + stage * C::STAGE;
    char* vbase = base + KS * C::KSLAB;
#pragma unroll
    for (int i = 0; i < C::PER; ++i) {
      const int ch = tid + i * C::NT;
      if (ch < C::CH) {
        const int key = ch / (D / 8), dg = ch % (D / 8);
        const int slab = key / TK, row = perm_row(key % TK);
        *(u32x4*)(base + slab * C::KSLAB + row * (2 * D) + ((dg ^ (row & 7)) << 4)) = kreg[i];
        if (tt < T_pre) {
          const int d = ch / (C::TKT / 8), kg = ch % (C::TKT / 8);
          const int vs = (kg * 8) / TK, gi = kg % C::VG;
          *(u32x4*)(vbase + vs * C::VSLAB + d * (2 * TK) + ((gi ^ (d & (C::VG - 1))) << 4)) = vreg[i];
        } else {  // tree V arrives token-major: transpose while writing
          const int ik = key % TK;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int d = dg * 8 + e;
            const uint16_t val = (uint16_t)(vreg[i][e >> 1] >> ((e & 1) * 16));
            *(uint16_t*)(vbase + slab * C::VSLAB + d * (2 * TK) + ((((ik >> 3) ^ (d & (C::VG - 1)))) << 4) +
                         (ik & 7) * 2) = val;
          }
        }
      }
    }
  };

  f32x16 O[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[db][r] = 0.f;
  float m_run = -INFINITY, lsum = 0.f;
  const float sl2 = a.scale_log2;

  load_tile(0);
  store_tile(0, 0);
  __syncthreads();

  for (int tt = 0; tt < T; ++tt) {
    if (tt + 1 < T) load_tile(tt + 1);
    {
      const int stage = tt & 1;
      const char* Ks = smem + stage * C::STAGE + ks * C::KSLAB;
      const char* Vs = smem + stage * C::STAGE + KS * C::KSLAB + ks * C::VSLAB;
      f32x16 S[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) S[kb][r] = 0.f;
        const int row = kb * 32 + col;
#pragma unroll
        for (int sd = 0; sd < C::SD; ++sd) {
          const bf16x8 kop = *(const bf16x8*)(Ks + row * (2 * D) + (((2 * sd + hh) ^ (row & 7)) << 4));
          S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[sd], S[kb], 0, 0, 0);
        }
      }
      // scale, mask, tile max
      const bool is_tree = tt >= T_pre;
      const int kbase = is_tree ? (tt - T_pre) * C::TKT + ks * TK : k0 + tt * C::TKT + ks * TK;
      const int kend = is_tree ? n : k1;
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + kb * 32 + 16 * (r >> 3) + 8 * hh + (r & 7);
          bool ok = qvalid && key < kend;
          if (is_tree) ok = ok && ((pick(mw0, mw1, mw2, mw3, key >> 6) >> (key & 63)) & 1);
          const float x = ok ? S[kb][r] * sl2 : -INFINITY;
          S[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
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
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        bf16x8 pop[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(S[kb][r] - msub);
          lsum += p;
          pop[r >> 3][r & 7] = (__bf16)p;
        }
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const int drow = 32 * db + col;
            const int gran = (kb * 4 + half * 2 + hh) ^ (drow & (C::VG - 1));
            const bf16x8 vop = *(const bf16x8*)(Vs + drow * (2 * TK) + (gran << 4));
            O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[half], O[db], 0, 0, 0);
          }
      }
    }
    if (tt + 1 < T) store_tile((tt + 1) & 1, tt + 1);
    __syncthreads();
  }

  // ---- combine the key-split waves of each query block
  if constexpr (KS > 1) {
    float* mb = (float*)smem;
    if (ks > 0) {
      float* dst = mb + (((ks - 1) * RB + rb) * 64 + lane) * 66;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[db * 16 + r] = O[db][r];
      dst[64] = m_run;
      dst[65] = lsum;
    }
    __syncthreads();
    if (ks > 0) return;
#pragma unroll
    for (int k = 1; k < KS; ++k) {
      const float* src = mb + (((k - 1) * RB + rb) * 64 + lane) * 66;
      const float mk = src[64], lk = src[65];
      const float M = fmaxf(m_run, mk);
      const float wa = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
      const float wb = (mk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk - M);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[db][r] = O[db][r] * wa + src[db * 16 + r] * wb;
      lsum = lsum * wa + lk * wb;
      m_run = M;
    }
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
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
        w.x = (uint32_t)f32_to_bf16(O[db][4 * rq] * inv) | ((uint32_t)f32_to_bf16(O[db][4 * rq + 1] * inv) << 16);
        w.y = (uint32_t)f32_to_bf16(O[db][4 * rq + 2] * inv) |
              ((uint32_t)f32_to_bf16(O[db][4 * rq + 3] * inv) << 16);
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

template <int D, int RB, int KS, int TK>
hipError_t launch_cfg(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  const int grid = a.B * a.Hkv * p.nchunks * p.rsplit;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_bf16_kernel<D, RB, KS, TK>), dim3(grid), dim3(64 * RB * KS), 0, s, a, p.rsplit,
                     p.nchunks, p.chunk_len, p.cap);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  if (p.rb == 1) return launch_cfg<D, 1, 4, 32>(a, p, s);
  if (p.rb == 2) return launch_cfg<D, 2, 2, 32>(a, p, s);
  if (p.rb == 4) return launch_cfg<D, 4, 1, 64>(a, p, s);
  return launch_cfg<D, 8, 1, 64>(a, p, s);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, const AttnPlan& p, hipStream_t s) {
  return a.D == 64 ? launch_d<64>(a, p, s) : launch_d<128>(a, p, s);
}

}  // namespace tv
