// tree_attention without a workspace argument, for callers that cannot
// allocate device memory (HIP graph capture, tight serving loops, harnesses
// that forbid allocation).  The partial results tree_attention keeps in the
// caller's workspace go to `scratch`, a fixed array in each GPU's memory that
// exists from the code object's load until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory, so
// it is never passed to a kernel: its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and that address
// is what the kernels receive.
#include <mutex>

#include "tv_internal.h"

namespace {

static __device__ __attribute__((aligned(256))) char scratch[TV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch`, per device id

// Device address of the current device's scratch array.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return tv::fail(TV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return tv::fail(TV_EUNSUPPORTED, "device id %d (at most %d devices)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
      return tv::fail(TV_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    if (p == nullptr || ((uintptr_t)p & 255)) return tv::fail(TV_EHIP, "scratch array on device %d misplaced", dev);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return TV_OK;
}

}  // namespace

extern "C" int tree_attention_noalloc(const tv_attn_desc* desc, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_table, const int32_t* prefix_len,
                                      const void* k_tree, const void* v_tree, const uint64_t* anc_mask, void* out,
                                      float* lse, int32_t* status, void* stream) {
  size_t need = 0;
  int rc = tv::attention_workspace_bytes(desc, &need);
  if (rc != TV_OK) return rc;
  if (need > TV_NOALLOC_SCRATCH_BYTES)
    return tv::fail(TV_EWORKSPACE,
                    "this descriptor needs %zu bytes of scratch, more than the %zu tree_attention_noalloc holds "
                    "(tree_attention with a caller workspace has no such limit)",
                    need, (size_t)TV_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0 && desc->B > 0) {
    rc = scratch_address(&ws);
    if (rc != TV_OK) return rc;
  }
  return tree_attention(desc, q, k_cache, v_cache, block_table, prefix_len, k_tree, v_tree, anc_mask, out, lse,
                        status, ws, ws != nullptr ? (size_t)TV_NOALLOC_SCRATCH_BYTES : 0, stream);
}
