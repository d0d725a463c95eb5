// C ABI of the library: argument validation on the host, launch planning and
// dispatch.  Nothing here allocates device memory; every launch goes to the
// caller's stream.  Host-side checks return before any HIP call, so they also
// work on machines without a GPU.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "tv_internal.h"

namespace {
thread_local std::string g_err;
}  // namespace

namespace tv {
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
}  // namespace tv

namespace {
using tv::fail;

int hip_fail(hipError_t e, const char* what) {
  return fail(TV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute units the launch plan aims to cover (MI355X: 256).  A constant, so the
// plan and the workspace size depend on the descriptor alone.
constexpr int kPlanCUs = 256;
int num_cus() { return kPlanCUs; }

int check_desc(const tv_attn_desc* d) {
  if (!d) return fail(TV_EINVAL, "desc is NULL");
  if (d->B < 0) return fail(TV_EINVAL, "B=%d < 0", d->B);
  if (d->n < 1 || d->n > TV_NMAX) return fail(TV_EINVAL, "n=%d outside [1, %d]", d->n, TV_NMAX);
  if (d->Hq < 1 || d->Hkv < 1) return fail(TV_EINVAL, "Hq=%d, Hkv=%d must be >= 1", d->Hq, d->Hkv);
  if (d->Hq % d->Hkv) return fail(TV_EUNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", d->Hq, d->Hkv);
  if (d->D != 64 && d->D != 128) return fail(TV_EUNSUPPORTED, "head dim %d (supported: 64, 128)", d->D);
  if (d->dtype != TV_F32 && d->dtype != TV_BF16 && d->dtype != TV_F16)
    return fail(TV_EUNSUPPORTED, "dtype %d", d->dtype);
  if (!(d->scale >= 0.f) || isinf(d->scale)) return fail(TV_EINVAL, "scale must be finite and >= 0");
  if (d->paged != 0 && d->paged != 1) return fail(TV_EINVAL, "paged must be 0 or 1");
  if (d->paged) {
    if (d->block_size != TV_PAGE) return fail(TV_EUNSUPPORTED, "block_size %d (supported: %d)", d->block_size, TV_PAGE);
    if (d->max_blocks < 0 || d->max_blocks > (1 << 26)) return fail(TV_EINVAL, "max_blocks=%d", d->max_blocks);
    if (d->num_blocks < 0) return fail(TV_EINVAL, "num_blocks=%d", d->num_blocks);
  } else {
    if (d->Lmax < 0 || d->Lmax % TV_PAGE) return fail(TV_EINVAL, "Lmax=%d must be >= 0 and a multiple of 16", d->Lmax);
  }
  if ((long long)d->Hq * d->n > (1LL << 24)) return fail(TV_EINVAL, "n*Hq too large");
  if (d->kv_dtype != 0 && d->kv_dtype != d->dtype) {
    if (d->kv_dtype != TV_FP8_E4M3) return fail(TV_EUNSUPPORTED, "cache dtype %d", d->kv_dtype);
    if (d->dtype != TV_BF16) return fail(TV_EUNSUPPORTED, "an fp8 cache needs dtype TV_BF16");
    if (!(d->k_scale > 0.f) || !(d->v_scale > 0.f) || isinf(d->k_scale) || isinf(d->v_scale))
      return fail(TV_EINVAL, "fp8 cache scales must be finite and > 0");
    // the many-row (balanced schedule) plan is not offered with an fp8 cache: a long run of
    // back-to-back calls of that variant once stopped making progress, with no cause found
    if ((long long)d->n * (d->Hq / d->Hkv) > 128)
      return fail(TV_EUNSUPPORTED, "an fp8 cache supports at most 128 query rows per KV head (n * Hq / Hkv = %d)",
                  d->n * (d->Hq / d->Hkv));
  }
  return TV_OK;
}

}  // namespace

namespace tv {

// Workgroup shape and prefix split for a descriptor (independent of device data).
int plan_attention(const tv_attn_desc* d, AttnPlan* p, int cus) {
  const int G = d->Hq / d->Hkv;
  p->rows = d->n * G;
  p->cap = d->paged ? d->max_blocks * TV_PAGE : d->Lmax;
  p->ws_bytes = 0;
  p->sk_nv = 0;
  p->rsplit = 1;
  p->nchunks = 1;
  p->chunk_len = p->cap > 0 ? p->cap : TV_PAGE;
  if (d->dtype == TV_F32) {  // one wave per query row, no split
    p->rb = p->ks = 1;
    p->tk = 64;
    return TV_OK;
  }
  const int qb = (p->rows + 31) / 32;
  if (qb <= 1) {
    p->rb = 1, p->ks = 5, p->tk = 32;
  } else if (qb <= 2) {
    p->rb = 2, p->ks = 4, p->tk = 32;
  } else if (qb <= 4) {
    p->rb = 4, p->ks = 2, p->tk = 32;
  } else {
    // many rows per KV head: 256-row workgroups on a balanced schedule of
    // 64-key tiles (the tile count must fit in int32)
    const long long rs = (p->rows + 255) / 256;
    const long long tiles = (long long)d->B * d->Hkv * ((p->cap + 63) / 64 + (d->n + 63) / 64);
    if (tiles < (1LL << 30)) {
      p->rb = 4, p->ks = 1, p->tk = 64;
      p->rsplit = (int)rs;
      p->sk_nv = (int)(rs >= cus ? 1 : cus / rs);
      const size_t slots = (size_t)2 * p->sk_nv * p->rsplit * 256;
      // per slot: a piece's scaled, normalised O in fp16, then (max, sum, scale, -) in fp32
      p->ws_bytes = tv::sk_sched_bytes(d->B) + ((slots * d->D * sizeof(uint16_t) + 255) & ~(size_t)255) +
                    ((slots * 4 * sizeof(float) + 255) & ~(size_t)255);
      return TV_OK;
    }
    p->rb = 8, p->ks = 1, p->tk = 64;
    p->rsplit = (qb + 7) / 8;
  }
  const int tkt = p->tk * p->ks;
  // split long prefixes so the grid covers the chip once (one workgroup per
  // compute unit streams faster than two sharing it, and fewer partial outputs
  // are written and merged), in chunks of at least 1024 tokens so partial outputs
  // stay a small fraction of the KV bytes
  const long long base = (long long)d->B * d->Hkv * p->rsplit;
  const long long target = cus;
  if (base > 0 && base < target && p->cap > 1024) {
    const long long want = (target + base - 1) / base;
    long long cl = (p->cap + want - 1) / want;
    if (cl < 1024) cl = 1024;
    cl = (cl + tkt - 1) / tkt * tkt;
    p->chunk_len = (int)cl;
    p->nchunks = (int)((p->cap + cl - 1) / cl);
  }
  if (p->chunk_len % tkt) p->chunk_len = (p->chunk_len + tkt - 1) / tkt * tkt;
  if (p->nchunks > 1) {
    const size_t parts = (size_t)d->B * d->Hkv * p->nchunks * p->rows;
    const size_t o = parts * d->D * sizeof(float);
    const size_t ml = parts * 2 * sizeof(float);
    p->ws_bytes = ((o + 255) & ~(size_t)255) + ((ml + 255) & ~(size_t)255);
  }
  return TV_OK;
}

int attention_workspace_bytes(const tv_attn_desc* d, size_t* bytes) {
  const int rc = check_desc(d);
  if (rc != TV_OK) return rc;
  AttnPlan p;
  plan_attention(d, &p, num_cus());
  *bytes = p.ws_bytes;
  return TV_OK;
}

}  // namespace tv

extern "C" {

const char* tv_status_string(int s) {
  switch (s) {
    case TV_OK: return "ok";
    case TV_EINVAL: return "invalid argument";
    case TV_ETOPOLOGY: return "invalid tree topology";
    case TV_EUNSUPPORTED: return "unsupported configuration";
    case TV_EWORKSPACE: return "workspace too small";
    case TV_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* tv_last_error(void) { return g_err.c_str(); }

int tv_version(void) { return TV_VERSION; }

int tree_validate_host(int n, const int32_t* parent, const int32_t* depth) {
  if (!parent || !depth) return fail(TV_EINVAL, "null pointer");
  if (n < 1 || n > TV_NMAX) return fail(TV_EINVAL, "n=%d outside [1, %d]", n, TV_NMAX);
  if (parent[0] != -1) return fail(TV_ETOPOLOGY, "node 0 must be the root (parent -1), got %d", parent[0]);
  if (depth[0] != 0) return fail(TV_ETOPOLOGY, "root depth must be 0, got %d", depth[0]);
  for (int u = 1; u < n; ++u) {
    const int p = parent[u];
    if (p < 0 || p >= u) return fail(TV_ETOPOLOGY, "parent[%d]=%d must be in [0, %d)", u, p, u);
    if (depth[u] != depth[p] + 1)
      return fail(TV_ETOPOLOGY, "depth[%d]=%d but its parent %d has depth %d", u, depth[u], p, depth[p]);
  }
  return TV_OK;
}

int tree_build(int B, int n, const int32_t* parent, const int32_t* depth, const int32_t* prefix_len,
               uint64_t* anc_mask, int32_t* pos_ids, int32_t* status, void* stream) {
  if (B < 0) return fail(TV_EINVAL, "B=%d < 0", B);
  if (n < 1 || n > TV_NMAX) return fail(TV_EINVAL, "n=%d outside [1, %d]", n, TV_NMAX);
  if (B == 0) return TV_OK;
  if (!parent || !depth || !prefix_len || !anc_mask || !pos_ids || !status)
    return fail(TV_EINVAL, "null pointer argument");
  hipError_t e = tv::launch_tree_build(B, n, parent, depth, prefix_len, anc_mask, pos_ids, status,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tree_build launch");
  return TV_OK;
}

size_t tree_attention_workspace_size(const tv_attn_desc* desc) {
  size_t b = 0;
  return tv::attention_workspace_bytes(desc, &b) == TV_OK ? b : (size_t)-1;
}

int tree_attention(const tv_attn_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_table, const int32_t* prefix_len, const void* k_tree, const void* v_tree,
                   const uint64_t* anc_mask, void* out, float* lse, int32_t* status, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc != TV_OK) return rc;
  if (desc->B == 0) return TV_OK;
  if (!q || !prefix_len || !k_tree || !v_tree || !anc_mask || !out)
    return fail(TV_EINVAL, "null pointer argument");
  tv::AttnPlan p;
  tv::plan_attention(desc, &p, num_cus());
  if (p.cap > 0 && (!k_cache || !v_cache)) return fail(TV_EINVAL, "null cache pointer");
  if (desc->paged && desc->max_blocks > 0 && !block_table) return fail(TV_EINVAL, "null block_table");
  if (p.ws_bytes > 0 && (!workspace || workspace_bytes < p.ws_bytes))
    return fail(TV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes, workspace_bytes);
  const uintptr_t al = (uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)k_tree |
                       (uintptr_t)v_tree | (uintptr_t)out | (uintptr_t)workspace;
  if (al & 15) return fail(TV_EINVAL, "device pointers must be 16-byte aligned");

  tv::AttnArgs a;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.bt = block_table;
  a.plen = prefix_len;
  a.kt = k_tree;
  a.vt = v_tree;
  a.mask = anc_mask;
  a.out = out;
  a.lse = lse;
  a.status = status;
  a.B = desc->B;
  a.n = desc->n;
  a.Hq = desc->Hq;
  a.Hkv = desc->Hkv;
  a.G = desc->Hq / desc->Hkv;
  a.D = desc->D;
  a.W = (desc->n + 63) / 64;
  a.paged = desc->paged;
  a.Lmax = desc->Lmax;
  a.max_blocks = desc->max_blocks;
  a.num_blocks = desc->num_blocks;
  a.f16 = desc->dtype == TV_F16;
  a.kv_fp8 = desc->kv_dtype == TV_FP8_E4M3;
  a.k_scale = desc->k_scale;
  a.v_scale = desc->v_scale;
  const float scale = desc->scale > 0.f ? desc->scale : 1.f / sqrtf((float)desc->D);
  a.scale_log2 = scale * tv::kLog2e;
  a.ws_o = nullptr;
  a.ws_ml = nullptr;
  if (p.ws_bytes > 0 && p.sk_nv == 0) {
    const size_t parts = (size_t)a.B * a.Hkv * p.nchunks * p.rows;
    const size_t o = (parts * a.D * sizeof(float) + 255) & ~(size_t)255;
    a.ws_o = (float*)workspace;
    a.ws_ml = (float*)((char*)workspace + o);
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (p.sk_nv > 0)
    e = tv::launch_attn_sk(a, p, workspace, s);
  else
    e = desc->dtype != TV_F32 ? tv::launch_attn_bf16(a, p, s) : tv::launch_attn_f32(a, p, s);
  if (e != hipSuccess) return hip_fail(e, "tree_attention launch");
  if (desc->dtype != TV_F32 && p.sk_nv == 0 && p.nchunks > 1) {
    e = tv::launch_merge(a, p, desc->dtype, s);
    if (e != hipSuccess) return hip_fail(e, "tree_attention merge launch");
  }
  return TV_OK;
}

int tree_verify_greedy(int B, int n, int V, int logits_dtype, const void* logits, const int32_t* tokens,
                       const int32_t* parent, int32_t* argmax_out, int32_t* path_out, int32_t* path_len,
                       int32_t* bonus, void* stream) {
  if (B < 0) return fail(TV_EINVAL, "B=%d < 0", B);
  if (n < 1 || n > TV_NMAX) return fail(TV_EINVAL, "n=%d outside [1, %d]", n, TV_NMAX);
  if (V < 1) return fail(TV_EINVAL, "V=%d < 1", V);
  if (logits_dtype != TV_F32 && logits_dtype != TV_BF16 && logits_dtype != TV_F16)
    return fail(TV_EUNSUPPORTED, "logits dtype %d", logits_dtype);
  if ((long long)B * n > 0x7fffffffLL) return fail(TV_EINVAL, "B*n too large");
  if (B == 0) return TV_OK;
  if (!logits || !tokens || !parent || !argmax_out || !path_out || !path_len || !bonus)
    return fail(TV_EINVAL, "null pointer argument");
  hipError_t e = tv::launch_verify(B, n, V, logits_dtype, logits, tokens, parent, argmax_out, path_out,
                                   path_len, bonus, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tree_verify_greedy launch");
  return TV_OK;
}

size_t tree_verify_stochastic_workspace_size(int B, int n, int V) {
  if (B < 0 || n < 1 || n > TV_NMAX || V < 1 || V > TV_MSS_VMAX) return (size_t)-1;
  return tv::mss_workspace_bytes(B, n, V);
}

int tree_verify_stochastic(int B, int n, int V, int logits_dtype, int mode, const void* logits, const void* ssm_logits,
                           const int32_t* tokens, const int32_t* parent, const float* u_accept,
                           const float* u_sample, int32_t* path_out, int32_t* path_len, int32_t* bonus,
                           int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0) return fail(TV_EINVAL, "B=%d < 0", B);
  if (n < 1 || n > TV_NMAX) return fail(TV_EINVAL, "n=%d outside [1, %d]", n, TV_NMAX);
  if (V < 1 || V > TV_MSS_VMAX) return fail(TV_EINVAL, "V=%d outside [1, %d]", V, TV_MSS_VMAX);
  if (logits_dtype != TV_F32 && logits_dtype != TV_BF16)
    return fail(TV_EUNSUPPORTED, "logits dtype %d", logits_dtype);
  if (mode < 0 || mode > 3) return fail(TV_EINVAL, "mode=%d outside [0, 3]", mode);
  if ((long long)B * n * 2 > 0x7fffffffLL) return fail(TV_EINVAL, "B*n too large");
  if (B == 0) return TV_OK;
  if (!logits || !ssm_logits || !tokens || !parent || !u_accept || !u_sample || !path_out || !path_len || !bonus)
    return fail(TV_EINVAL, "null pointer argument");
  const size_t need = tv::mss_workspace_bytes(B, n, V);
  if (!workspace || workspace_bytes < need)
    return fail(TV_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  if (((uintptr_t)logits | (uintptr_t)ssm_logits | (uintptr_t)workspace) & 15)
    return fail(TV_EINVAL, "logits, ssm_logits and workspace must be 16-byte aligned");
  hipError_t e = tv::launch_mss(B, n, V, logits_dtype == TV_BF16, mode, logits, ssm_logits, tokens, parent, u_accept,
                                u_sample, (float*)workspace, path_out, path_len, bonus, status, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tree_verify_stochastic launch");
  return TV_OK;
}

int tree_verify_stochastic_set_poll_limit(int polls, int* previous) {
  if (polls < 0) return fail(TV_EINVAL, "polls=%d < 0", polls);
  const int prev = tv::mss_set_poll_limit(polls);
  if (previous) *previous = prev;
  return TV_OK;
}

int tree_expand_topk(int B, int F, int V, int k, int n_max, int logits_dtype, const void* ssm_logits,
                     const int32_t* frontier, const int32_t* n_cur, int32_t* parent, int32_t* depth, int32_t* tokens,
                     float* scores, int32_t* n_out, int32_t* status, void* stream) {
  if (B < 0) return fail(TV_EINVAL, "B=%d < 0", B);
  if (F < 1 || F > 256) return fail(TV_EINVAL, "F=%d outside [1, 256]", F);
  if (V < 1) return fail(TV_EINVAL, "V=%d < 1", V);
  if (k < 1 || k > TV_TOPK_MAX || k > V) return fail(TV_EINVAL, "k=%d outside [1, min(%d, V)]", k, TV_TOPK_MAX);
  if (n_max < 1 || n_max > TV_NMAX) return fail(TV_EINVAL, "n_max=%d outside [1, %d]", n_max, TV_NMAX);
  if (logits_dtype != TV_F32 && logits_dtype != TV_BF16)
    return fail(TV_EUNSUPPORTED, "logits dtype %d", logits_dtype);
  if ((long long)B * F > 0x7fffffffLL) return fail(TV_EINVAL, "B*F too large");
  if (B == 0) return TV_OK;
  if (!ssm_logits || !frontier || !n_cur || !parent || !depth || !tokens || !n_out || !status)
    return fail(TV_EINVAL, "null pointer argument");
  hipError_t e = tv::launch_expand(B, F, V, k, n_max, logits_dtype == TV_BF16, ssm_logits, frontier, n_cur, parent,
                                   depth, tokens, scores, n_out, status, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tree_expand_topk launch");
  return TV_OK;
}

int tree_merge_drafts(int B, int M, int Ld, int n_max, const int32_t* drafts, const int32_t* draft_len,
                      const int32_t* root_token, int32_t* parent, int32_t* depth, int32_t* tokens, int32_t* n_out,
                      int32_t* node_of, int32_t* status, void* stream) {
  if (B < 0) return fail(TV_EINVAL, "B=%d < 0", B);
  if (M < 1 || M > TV_MERGE_MMAX) return fail(TV_EINVAL, "M=%d outside [1, %d]", M, TV_MERGE_MMAX);
  if (Ld < 1 || Ld >= TV_NMAX) return fail(TV_EINVAL, "Ld=%d outside [1, %d]", Ld, TV_NMAX - 1);
  if (n_max < 1 || n_max > TV_NMAX) return fail(TV_EINVAL, "n_max=%d outside [1, %d]", n_max, TV_NMAX);
  if (B == 0) return TV_OK;
  if (!drafts || !draft_len || !parent || !depth || !tokens || !n_out || !status)
    return fail(TV_EINVAL, "null pointer argument");
  hipError_t e = tv::launch_merge_drafts(B, M, Ld, n_max, drafts, draft_len, root_token, parent, depth, tokens, n_out,
                                         node_of, status, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tree_merge_drafts launch");
  return TV_OK;
}

int tree_commit_kv(const tv_attn_desc* desc, void* k_cache, void* v_cache, const int32_t* block_table,
                   const int32_t* prefix_len, const void* k_tree, const void* v_tree, const int32_t* path,
                   const int32_t* path_len, int32_t* new_prefix_len, int32_t* status, void* stream) {
  int rc = check_desc(desc);
  if (rc != TV_OK) return rc;
  if (desc->kv_dtype == TV_FP8_E4M3) return fail(TV_EUNSUPPORTED, "committing into an fp8 cache");
  if ((long long)desc->B * desc->n > 0x7fffffffLL) return fail(TV_EINVAL, "B*n too large");
  if (desc->B == 0) return TV_OK;
  if (!k_cache || !v_cache || !prefix_len || !k_tree || !v_tree || !path || !path_len || !new_prefix_len)
    return fail(TV_EINVAL, "null pointer argument");
  if (desc->paged && desc->max_blocks > 0 && !block_table) return fail(TV_EINVAL, "null block_table");
  const uintptr_t al = (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)k_tree | (uintptr_t)v_tree;
  if (al & 15) return fail(TV_EINVAL, "device pointers must be 16-byte aligned");
  const uintptr_t a0 = (uintptr_t)prefix_len, a1 = (uintptr_t)new_prefix_len;
  const uintptr_t nb = (uintptr_t)desc->B * sizeof(int32_t);
  if (a0 < a1 + nb && a1 < a0 + nb) return fail(TV_EINVAL, "new_prefix_len overlaps prefix_len");
  hipError_t e = tv::launch_commit(desc, k_cache, v_cache, block_table, prefix_len, k_tree, v_tree, path, path_len,
                                   new_prefix_len, status, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tree_commit_kv launch");
  return TV_OK;
}

}  // extern "C"
