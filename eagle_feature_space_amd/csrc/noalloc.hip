// eagle_draft_step_noalloc: the draft step with its workspace in a
// file-scope device array instead of a caller buffer, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array is `scratch` below.  Its name is a host-side stand-in in host
// code, never a device address: the address of each device's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "eagle.h"

namespace {

constexpr size_t kScratchBytes = (size_t)EAGLE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// this device's copy of `scratch` (nullptr on a HIP error)
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" int eagle_draft_step_noalloc(const eagle_head* head, const eagle_kv* kv,
                                        const eagle_tree* tree, int step, const void* f_root,
                                        const void* lmh, const int32_t* ctx_tokens,
                                        float* logits_out, void* feat_out, void* stream) {
  const size_t need = eagle_workspace_bytes(head, kv, tree);
  if (need == 0) return EAGLE_EINVAL;
  if (need > kScratchBytes) return EAGLE_ECAPACITY;
  void* ws = scratch_ptr();
  if (!ws) return EAGLE_EHIP;
  return eagle_draft_step(head, kv, tree, step, f_root, lmh, ctx_tokens, logits_out, feat_out, ws,
                          kScratchBytes, stream);
}
