// Host-side checks of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// The library's host layer (argument validation, launch planning, workspace
// sizing, error strings) is linked against stub launchers instead of the HIP
// kernels, so it runs on a machine without a GPU.  Each stub checks the plan it
// is handed against the shapes the kernels assume (rows covered, prefix chunks
// covering the capacity, workspace regions inside the caller's buffer).  The
// driver sweeps pseudo-random descriptors and arguments, valid and invalid,
// through every entry point; the sanitizers report any out-of-bounds access,
// overflow or other undefined behaviour on the way.  Prints "OK <calls>" on
// success; any failed check prints a message and exits non-zero.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "tv_internal.h"

namespace {

int g_checks = 0;
int g_fail_next = 0;             // the next stub launch reports a HIP error
uintptr_t g_ws = 0;              // workspace the driver passed to tree_attention
size_t g_ws_bytes = 0;
const tv_attn_desc* g_desc = nullptr;

#define CHECK(cond, ...)                                       \
  do {                                                         \
    ++g_checks;                                                \
    if (!(cond)) {                                             \
      fprintf(stderr, "check failed at line %d: ", __LINE__);  \
      fprintf(stderr, __VA_ARGS__);                            \
      fprintf(stderr, "\n");                                   \
      exit(2);                                                 \
    }                                                          \
  } while (0)

hipError_t stub() {
  if (g_fail_next) {
    g_fail_next = 0;
    return hipErrorInvalidValue;
  }
  return hipSuccess;
}

bool in_ws(const void* p, size_t bytes) {
  const uintptr_t a = (uintptr_t)p;
  return a >= g_ws && a + bytes <= g_ws + g_ws_bytes;
}

// what every attention plan must satisfy, whatever kernel runs it
void check_plan_common(const tv::AttnArgs& a, const tv::AttnPlan& p) {
  const tv_attn_desc* d = g_desc;
  CHECK(d != nullptr, "launch without a descriptor");
  CHECK(a.B == d->B && a.n == d->n && a.Hq == d->Hq && a.Hkv == d->Hkv && a.D == d->D, "args differ from desc");
  CHECK(a.G == d->Hq / d->Hkv && p.rows == d->n * a.G, "rows %d", p.rows);
  CHECK(a.W == (d->n + 63) / 64 && a.W >= 1 && a.W <= TV_WMAX, "mask words %d", a.W);
  CHECK(p.cap == (d->paged ? d->max_blocks * TV_PAGE : d->Lmax), "capacity %d", p.cap);
  CHECK(p.ws_bytes <= g_ws_bytes, "plan needs %zu workspace bytes, %zu given", p.ws_bytes, g_ws_bytes);
}

}  // namespace

// ---- stub launchers: plan checks, no device work
namespace tv {

size_t sk_sched_bytes(int B) { return (((size_t)B + 5) * sizeof(int32_t) + 255) & ~(size_t)255; }
size_t mss_workspace_bytes(int B, int n, int V) { return (size_t)B * 2 * (size_t)V * sizeof(float) + (size_t)n; }
int mss_set_poll_limit(int polls) {
  static int limit = 1 << 18;
  const int prev = limit;
  limit = polls;
  return prev;
}

hipError_t launch_attn_bf16(const AttnArgs& a, const AttnPlan& p, hipStream_t) {
  check_plan_common(a, p);
  // the kernel table: (row waves, key-split groups, tile keys) by rows per KV head
  const int qb = (p.rows + 31) / 32;
  const int rb = qb <= 1 ? 1 : qb <= 2 ? 2 : qb <= 4 ? 4 : 8;
  CHECK(p.rb == rb, "rb %d for %d rows", p.rb, p.rows);
  CHECK(p.sk_nv == 0, "few-row plan with a tile schedule");
  CHECK(p.rsplit >= 1 && (long long)p.rsplit * 32 * p.rb >= p.rows, "rsplit %d does not cover %d rows", p.rsplit,
        p.rows);
  // plans of at most 4 row waves stream their tiles non-temporal: one row slice, so one reader per tile
  CHECK(p.rb > 4 || p.rsplit == 1, "rb %d with %d row slices", p.rb, p.rsplit);
  CHECK(p.tk == 32 || p.tk == 64, "tile keys %d", p.tk);
  CHECK(p.nchunks >= 1 && p.chunk_len >= p.tk && p.chunk_len % p.tk == 0, "chunks %d x %d", p.nchunks, p.chunk_len);
  CHECK((long long)p.nchunks * p.chunk_len >= p.cap, "chunks do not cover the capacity");
  CHECK(p.cap == 0 || (long long)(p.nchunks - 1) * p.chunk_len < p.cap, "an empty trailing chunk");
  if (p.nchunks > 1) {
    const size_t parts = (size_t)a.B * a.Hkv * p.nchunks * p.rows;
    CHECK(in_ws(a.ws_o, parts * a.D * sizeof(float)), "partial outputs outside the workspace");
    CHECK(in_ws(a.ws_ml, parts * 2 * sizeof(float)), "partial statistics outside the workspace");
  } else {
    CHECK(a.ws_o == nullptr && a.ws_ml == nullptr, "partials without chunks");
  }
  return stub();
}

hipError_t launch_attn_f32(const AttnArgs& a, const AttnPlan& p, hipStream_t) {
  check_plan_common(a, p);
  CHECK(p.rb == 1 && p.ks == 1 && p.nchunks == 1 && p.sk_nv == 0, "fp32 plan");
  return stub();
}

hipError_t launch_attn_sk(const AttnArgs& a, const AttnPlan& p, void* ws, hipStream_t) {
  check_plan_common(a, p);
  CHECK(p.sk_nv >= 1 && p.rsplit >= 1 && (long long)p.rsplit * 256 >= p.rows, "tile schedule %d x %d for %d rows",
        p.sk_nv, p.rsplit, p.rows);
  CHECK((uintptr_t)ws == g_ws && p.ws_bytes > 0, "schedule workspace");
  const size_t slots = (size_t)2 * p.sk_nv * p.rsplit * 256;
  CHECK(p.ws_bytes >= sk_sched_bytes(a.B) + slots * (a.D * sizeof(uint16_t) + 4 * sizeof(float)),
        "schedule workspace too small");
  return stub();
}

hipError_t launch_merge(const AttnArgs& a, const AttnPlan& p, int, hipStream_t) {
  CHECK(p.nchunks > 1 && a.ws_o != nullptr, "merge without chunks");
  return stub();
}

hipError_t launch_tree_build(int B, int n, const int32_t*, const int32_t*, const int32_t*, uint64_t*, int32_t*, int32_t*,
                             hipStream_t) {
  CHECK(B > 0 && n >= 1 && n <= TV_NMAX, "tree_build launch B=%d n=%d", B, n);
  return stub();
}

hipError_t launch_commit(const tv_attn_desc* d, void*, void*, const int32_t*, const int32_t*, const void*, const void*,
                         const int32_t*, const int32_t*, int32_t*, int32_t*, hipStream_t) {
  CHECK(d != nullptr && d->B > 0 && d->n >= 1 && d->n <= TV_NMAX, "commit launch");
  return stub();
}

hipError_t launch_mss(int B, int n, int V, int, int, const void*, const void*, const int32_t*, const int32_t*,
                      const float*, const float*, float*, int32_t*, int32_t*, int32_t*, int32_t*, hipStream_t) {
  CHECK(B > 0 && n >= 1 && n <= TV_NMAX && V >= 1 && V <= TV_MSS_VMAX, "stochastic launch");
  return stub();
}

hipError_t launch_expand(int B, int F, int V, int k, int n_max, int, const void*, const int32_t*, const int32_t*,
                         int32_t*, int32_t*, int32_t*, float*, int32_t*, int32_t*, hipStream_t) {
  CHECK(B > 0 && F >= 1 && V >= 1 && k >= 1 && k <= TV_TOPK_MAX && n_max >= 1 && n_max <= TV_NMAX, "expand launch");
  return stub();
}

hipError_t launch_merge_drafts(int B, int M, int Ld, int n_max, const int32_t*, const int32_t*, const int32_t*, int32_t*,
                               int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, hipStream_t) {
  CHECK(B > 0 && M >= 1 && M <= TV_MERGE_MMAX && Ld >= 0 && n_max >= 1 && n_max <= TV_NMAX, "merge-drafts launch");
  return stub();
}

hipError_t launch_verify(int B, int n, int V, int, const void*, const int32_t*, const int32_t*, int32_t*, int32_t*,
                         int32_t*, int32_t*, hipStream_t) {
  CHECK(B > 0 && n >= 1 && n <= TV_NMAX && V >= 1, "verify launch");
  return stub();
}

}  // namespace tv

// ---- the sweep
namespace {

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint32_t rnd() {  // xorshift64*
  g_rng ^= g_rng >> 12;
  g_rng ^= g_rng << 25;
  g_rng ^= g_rng >> 27;
  return (uint32_t)((g_rng * 2685821657736338717ull) >> 32);
}
int pick(std::initializer_list<int> v) { return v.begin()[rnd() % v.size()]; }
int range(int lo, int hi) { return lo + (int)(rnd() % (uint32_t)(hi - lo + 1)); }

void* P(uintptr_t a) { return (void*)a; }  // a stand-in device address: never dereferenced on the host
const uintptr_t kDev = 0x7f0000000000ull;

void check_status(int rc) {
  CHECK(rc >= TV_OK && rc <= TV_EHIP, "status %d", rc);
  const char* s = tv_status_string(rc);
  CHECK(s != nullptr && strlen(s) > 0, "status string");
  if (rc != TV_OK) CHECK(strlen(tv_last_error()) > 0, "no error detail for status %d", rc);
}

void sweep_attention(int iters) {
  for (int i = 0; i < iters; ++i) {
    tv_attn_desc d;
    memset(&d, 0, sizeof d);
    d.B = pick({-1, 0, 1, 2, 7, 8, 64, 600});
    d.n = pick({-3, 0, 1, 2, 7, 21, 32, 64, 65, 128, 130, 256, 257});
    d.Hkv = pick({0, 1, 2, 8, 32});
    d.Hq = d.Hkv * pick({1, 2, 4, 8}) + (rnd() % 16 == 0 ? 1 : 0);
    d.D = pick({0, 64, 96, 128, 256});
    d.dtype = pick({-1, TV_F32, TV_BF16, TV_F16, TV_FP8_E4M3, 9});
    d.scale = rnd() % 8 == 0 ? -1.f : (rnd() % 2 ? 0.f : 0.0883883f);
    d.paged = pick({0, 0, 1, 1, 2});
    d.block_size = pick({16, 16, 16, 32, 0});
    d.Lmax = pick({0, 16, 1024, 1030, 8192, 32768, -16});
    d.max_blocks = pick({0, 1, 64, 2048, -1});
    d.num_blocks = pick({0, 100, 40960, -5});
    d.kv_dtype = pick({0, 0, 0, TV_FP8_E4M3, TV_F16, 7});
    d.k_scale = rnd() % 6 == 0 ? 0.f : 0.05f;
    d.v_scale = rnd() % 6 == 0 ? -1.f : 0.04f;

    const size_t ws = tree_attention_workspace_size(&d);
    std::vector<char> host_ws(64);  // the workspace is a device buffer; only its address is used on the host
    g_ws = kDev + 0x100000000ull;
    g_ws_bytes = ws == (size_t)-1 ? 0 : ws;
    g_desc = &d;
    const bool valid = ws != (size_t)-1;
    int rc = tree_attention(&d, P(kDev), P(kDev + 0x1000), P(kDev + 0x2000), (const int32_t*)P(kDev + 0x3000),
                            (const int32_t*)P(kDev + 0x4000), P(kDev + 0x5000), P(kDev + 0x6000),
                            (const uint64_t*)P(kDev + 0x7000), P(kDev + 0x8000), (float*)P(kDev + 0x9000),
                            (int32_t*)P(kDev + 0xa000), ws > 0 && valid ? P(g_ws) : nullptr, g_ws_bytes, nullptr);
    check_status(rc);
    CHECK(valid == (rc == TV_OK), "workspace_size and tree_attention disagree on validity (rc %d)", rc);
    if (!valid || d.B == 0) continue;
    if (ws > 0) {  // one byte short, and missing
      rc = tree_attention(&d, P(kDev), P(kDev + 0x1000), P(kDev + 0x2000), (const int32_t*)P(kDev + 0x3000),
                          (const int32_t*)P(kDev + 0x4000), P(kDev + 0x5000), P(kDev + 0x6000),
                          (const uint64_t*)P(kDev + 0x7000), P(kDev + 0x8000), nullptr, nullptr, P(g_ws), ws - 1,
                          nullptr);
      CHECK(rc == TV_EWORKSPACE, "short workspace gave %d", rc);
      rc = tree_attention(&d, P(kDev), P(kDev + 0x1000), P(kDev + 0x2000), (const int32_t*)P(kDev + 0x3000),
                          (const int32_t*)P(kDev + 0x4000), P(kDev + 0x5000), P(kDev + 0x6000),
                          (const uint64_t*)P(kDev + 0x7000), P(kDev + 0x8000), nullptr, nullptr, nullptr, ws,
                          nullptr);
      CHECK(rc == TV_EWORKSPACE, "missing workspace gave %d", rc);
    }
    // misaligned and null pointers
    rc = tree_attention(&d, P(kDev + 4), P(kDev + 0x1000), P(kDev + 0x2000), (const int32_t*)P(kDev + 0x3000),
                        (const int32_t*)P(kDev + 0x4000), P(kDev + 0x5000), P(kDev + 0x6000),
                        (const uint64_t*)P(kDev + 0x7000), P(kDev + 0x8000), nullptr, nullptr,
                        ws > 0 ? P(g_ws) : nullptr, ws, nullptr);
    CHECK(rc == TV_EINVAL, "misaligned q gave %d", rc);
    rc = tree_attention(&d, nullptr, P(kDev + 0x1000), P(kDev + 0x2000), (const int32_t*)P(kDev + 0x3000),
                        (const int32_t*)P(kDev + 0x4000), P(kDev + 0x5000), P(kDev + 0x6000),
                        (const uint64_t*)P(kDev + 0x7000), P(kDev + 0x8000), nullptr, nullptr,
                        ws > 0 ? P(g_ws) : nullptr, ws, nullptr);
    CHECK(rc == TV_EINVAL, "null q gave %d", rc);
    // a launch error comes back as TV_EHIP with the runtime's text
    g_fail_next = 1;
    rc = tree_attention(&d, P(kDev), P(kDev + 0x1000), P(kDev + 0x2000), (const int32_t*)P(kDev + 0x3000),
                        (const int32_t*)P(kDev + 0x4000), P(kDev + 0x5000), P(kDev + 0x6000),
                        (const uint64_t*)P(kDev + 0x7000), P(kDev + 0x8000), nullptr, nullptr,
                        ws > 0 ? P(g_ws) : nullptr, ws, nullptr);
    g_fail_next = 0;
    CHECK(rc == TV_EHIP && strlen(tv_last_error()) > 0, "launch error gave %d", rc);
    (void)host_ws;
  }
  g_desc = nullptr;
}

void sweep_topology(int iters) {
  for (int i = 0; i < iters; ++i) {
    const int n = pick({0, 1, 2, 5, 64, 255, 256, 257});
    std::vector<int32_t> parent(n > 0 ? n : 1), depth(n > 0 ? n : 1);  // exactly n readable entries when n >= 1
    for (int u = 0; u < n; ++u) {
      parent[u] = u == 0 ? -1 : range(0, u - 1);
      depth[u] = u == 0 ? 0 : depth[parent[u]] + 1;
    }
    int expect = (n >= 1 && n <= TV_NMAX) ? TV_OK : TV_EINVAL;
    if (n >= 2 && expect == TV_OK && rnd() % 2) {  // plant one fault
      const int u = range(1, n - 1);
      switch (rnd() % 4) {
        case 0: parent[u] = u; break;
        case 1: parent[u] = n + 5; break;
        case 2: depth[u] += 1; break;
        default: parent[0] = 0; break;
      }
      expect = TV_ETOPOLOGY;
    }
    const int rc = tree_validate_host(n, n >= 1 ? parent.data() : nullptr, n >= 1 ? depth.data() : nullptr);
    check_status(rc);
    CHECK(rc == expect || (expect == TV_OK && rc == TV_OK), "validate n=%d gave %d, expected %d", n, rc, expect);
    CHECK(tree_validate_host(n, nullptr, depth.data()) == TV_EINVAL, "null parent");
  }
}

void sweep_others(int iters) {
  const int32_t* I = (const int32_t*)P(kDev);
  int32_t* O = (int32_t*)P(kDev + 0x10000);
  for (int i = 0; i < iters; ++i) {
    const int B = pick({-1, 0, 1, 8, 64});
    const int n = pick({-1, 0, 1, 21, 256, 257});
    const int V = pick({-1, 0, 1, 1000, 32000, (1 << 20) + 1});
    const int dt = pick({-1, TV_F32, TV_BF16, TV_F16, TV_FP8_E4M3});
    const bool nul = rnd() % 5 == 0;
    check_status(tree_build(B, n, nul ? nullptr : I, I, I, (uint64_t*)O, O, O, nullptr));
    check_status(tree_verify_greedy(B, n, V, dt, nul ? nullptr : P(kDev), I, I, O, O, O, O, nullptr));
    const size_t sws = tree_verify_stochastic_workspace_size(B, n, V);
    check_status(tree_verify_stochastic(B, n, V, dt, pick({-1, 0, 1, 2, 3}), nul ? nullptr : P(kDev), P(kDev), I, I,
                                        (const float*)P(kDev), (const float*)P(kDev), O, O, O, O,
                                        rnd() % 3 ? P(kDev + 0x20000) : nullptr,
                                        rnd() % 4 ? sws : sws / 2, nullptr));
    {
      int prev = -7;
      const int polls = pick({-1, 0, 1, 1 << 18});
      check_status(tree_verify_stochastic_set_poll_limit(polls, rnd() % 2 ? &prev : nullptr));
    }
    check_status(tree_expand_topk(B, pick({-1, 0, 1, 4}), V, pick({0, 1, 4, 16, 17}), pick({0, 1, 64, 256, 300}), dt,
                                  nul ? nullptr : P(kDev), I, I, O, O, O, (float*)O, O, O, nullptr));
    check_status(tree_merge_drafts(B, pick({0, 1, 8, 64, 65}), pick({-1, 0, 8, 255}), pick({0, 1, 256, 257}),
                                   nul ? nullptr : I, I, I, O, O, O, O, O, O, nullptr));
    tv_attn_desc d;
    memset(&d, 0, sizeof d);
    d.B = B;
    d.n = n;
    d.Hq = 32;
    d.Hkv = pick({0, 8, 32});
    d.D = pick({64, 128, 100});
    d.dtype = dt;
    d.paged = pick({0, 1});
    d.block_size = 16;
    d.Lmax = pick({0, 1024, 17});
    d.max_blocks = 64;
    d.num_blocks = 1000;
    check_status(tree_commit_kv(rnd() % 9 ? &d : nullptr, P(kDev), P(kDev), I, I, P(kDev), P(kDev), I, I, O, O,
                                nullptr));
  }
  for (int s = -2; s < 8; ++s) CHECK(tv_status_string(s) != nullptr, "status string %d", s);
  CHECK(tv_version() == TV_VERSION, "version");
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 20000;
  sweep_topology(iters / 4);
  sweep_attention(iters);
  sweep_others(iters / 4);
  printf("OK %d\n", g_checks);
  return 0;
}
