// Device helpers shared by the bf16 tree-attention kernels (gfx950 only).
#pragma once
#include "tv_internal.h"

namespace tv {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
#define AS3 __attribute__((address_space(3)))
#define AS4 __attribute__((address_space(4)))

constexpr float kTau = 8.0f;  // lazy-rescale threshold in the log2 domain

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The 16-bit element type of q, K, V, out and of the P operand: bf16 or fp16
// (the explainer's implementation points run everything in FP16).  Both use the
// same 16-bit data paths (DMA, LDS layouts, transposing reads); only the matrix
// instruction, the roundings and the row-sum dot product differ.
template <bool F16>
struct Elt;
template <>
struct Elt<false> {
  typedef __bf16 T;
  typedef bf16x8 V8;
  typedef bf16x2 V2;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ T cvt(float x) { return (__bf16)x; }
  static __device__ __forceinline__ uint32_t bits(float x) { return f32_to_bf16(x); }
  static __device__ __forceinline__ float dot2(V2 a, V2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
  }
};
template <>
struct Elt<true> {
  typedef _Float16 T;
  typedef f16x8 V8;
  typedef f16x2 V2;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ T cvt(float x) { return (_Float16)x; }
  static __device__ __forceinline__ uint32_t bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
  static __device__ __forceinline__ float dot2(V2 a, V2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
};

__device__ __forceinline__ int perm_row(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

// Granule swizzles (16-byte granules within a token row of the tile).
template <int D>
__device__ __forceinline__ int kswz(int row) {  // 16 consecutive rows -> 16 distinct bank groups
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int row) {  // 4 consecutive rows x 4 granules -> distinct
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// HBM -> LDS copy of 16 bytes per lane; lane l lands at lds_line + 16*l.  Issued
// through asm so the compiler does not add its own (full) waits around it; the
// kernel waits with explicit vmcnt counts instead.
//
// The LDS address comes from M0.  Two rules of the GFX9 family apply, and the
// compiler cannot apply them inside asm:
//  - an LDS DMA that reads M0 in the cycle after a scalar write of M0 may see the
//    old value, so one wait state (s_nop 0) separates them, as the compiler's own
//    hazard pass does when it emits this pair;
//  - M0 is a register the compiler reserves, so the asm restores the value it
//    found instead of declaring it clobbered.
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_line) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gaddr), "s"(__builtin_amdgcn_readfirstlane(lds_line)));
}
// Same with a wave-uniform 64-bit base and a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_line) {
  const uint64_t b = (uint64_t)sbase;
  const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(ub), "s"(__builtin_amdgcn_readfirstlane(lds_line)));
}

// The same for the streaming prefix tiles: `nt` marks the lines non-temporal (each
// is read once), so they displace less of what the caches hold.
__device__ __forceinline__ void dma16s_nt(const void* sbase, uint32_t voff, uint32_t lds_line) {
  const uint64_t b = (uint64_t)sbase;
  const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(ub), "s"(__builtin_amdgcn_readfirstlane(lds_line)));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that orders LDS accesses only (a full fence would also wait
// for every outstanding HBM load and empty the pipeline).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace attn
}  // namespace tv
