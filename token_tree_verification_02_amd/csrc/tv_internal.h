// Internal declarations shared by the library's HIP translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tree_verify.h"

namespace tv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 bit pattern -> float (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp16 bit pattern -> float (exact)
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// float -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// ------------------------------------------------------------------ cross-lane moves
// DPP controls within each row of 16 lanes (a lane reads its partner's register
// in the same VALU op, no LDS round trip): swap neighbours, swap pairs, take the
// other quad of the half-row (half-row mirror), take the other half of the row
// (row mirror).  Combining a lane's value with its partner's over these four
// steps reduces each row of 16 lanes.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, dpp<CTRL>(__builtin_bit_cast(int, x)));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)dpp<CTRL>((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)dpp<CTRL>((int)(uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// lane l's value, the same in every lane
__device__ __forceinline__ int lane_read(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ float lane_read(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ double lane_read(double x, int l) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// ------------------------------------------------------------------ launch plans
struct AttnPlan {
  int rows;        // n * (Hq/Hkv): query rows per (sequence, KV head)
  int rb;          // 32-row query blocks per workgroup (waves along rows)
  int ks;          // key-split waves per query block
  int tk;          // keys per wave per tile
  int rsplit;      // workgroups along rows
  int nchunks;     // prefix chunks (split-K) per (sequence, KV head)
  int chunk_len;   // prefix tokens per chunk (multiple of the tile)
  int cap;         // cache capacity per sequence in tokens
  int sk_nv;       // > 0: balanced persistent schedule over this many tile ranges
  size_t ws_bytes; // workspace bytes
};

int plan_attention(const tv_attn_desc* d, AttnPlan* p, int num_cus);
// Validates the descriptor and gives the workspace tree_attention needs for it
// (TV_OK, or the status with the message set as for a failed call).
int attention_workspace_bytes(const tv_attn_desc* d, size_t* bytes);
// Sets the calling thread's last-error message; returns `code`.
int fail(int code, const char* fmt, ...);

struct AttnArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* bt;
  const int32_t* plen;
  const void* kt;
  const void* vt;
  const uint64_t* mask;
  void* out;
  float* lse;
  int32_t* status;
  float* ws_o;     // [B][Hkv][nchunks][rows][D] fp32 partial outputs (unnormalised)
  float* ws_ml;    // [B][Hkv][nchunks][rows][2] running max (log2 domain), sum
  int B, n, Hq, Hkv, G, D, W;
  int paged, Lmax, max_blocks, num_blocks;
  int f16;           // 16-bit element type: 0 bf16, 1 fp16
  int kv_fp8;        // prefix cache holds OCP E4M3 codes; value = code * k_scale (v_scale)
  float k_scale, v_scale;
  float scale_log2;  // softmax scale * log2(e)
};

hipError_t launch_attn_bf16(const AttnArgs& a, const AttnPlan& p, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, const AttnPlan& p, hipStream_t s);
size_t sk_sched_bytes(int B);
hipError_t launch_attn_sk(const AttnArgs& a, const AttnPlan& p, void* ws, hipStream_t s);
hipError_t launch_merge(const AttnArgs& a, const AttnPlan& p, int out_dtype, hipStream_t s);
hipError_t launch_tree_build(int B, int n, const int32_t* parent, const int32_t* depth,
                             const int32_t* plen, uint64_t* mask, int32_t* pos, int32_t* status,
                             hipStream_t s);
hipError_t launch_commit(const tv_attn_desc* d, void* kc, void* vc, const int32_t* bt, const int32_t* plen,
                         const void* kt, const void* vt, const int32_t* path, const int32_t* path_len,
                         int32_t* new_len, int32_t* status, hipStream_t s);
size_t mss_workspace_bytes(int B, int n, int V);
int mss_set_poll_limit(int polls);  // returns the previous limit
hipError_t launch_mss(int B, int n, int V, int bf16, int mode, const void* logits, const void* ssm,
                      const int32_t* tokens, const int32_t* parent, const float* u_acc, const float* u_smp,
                      float* ws, int32_t* path, int32_t* plen, int32_t* bonus, int32_t* status, hipStream_t s);
hipError_t launch_expand(int B, int F, int V, int k, int n_max, int bf16, const void* logits, const int32_t* frontier,
                         const int32_t* n_cur, int32_t* parent, int32_t* depth, int32_t* tokens, float* scores,
                         int32_t* n_out, int32_t* status, hipStream_t s);
hipError_t launch_merge_drafts(int B, int M, int Ld, int n_max, const int32_t* drafts, const int32_t* draft_len,
                               const int32_t* root_token, int32_t* parent, int32_t* depth, int32_t* tokens,
                               int32_t* n_out, int32_t* node_of, int32_t* status, hipStream_t s);
hipError_t launch_verify(int B, int n, int V, int dtype, const void* logits, const int32_t* tokens,
                         const int32_t* parent, int32_t* am, int32_t* path, int32_t* plen,
                         int32_t* bonus, hipStream_t s);

}  // namespace tv
