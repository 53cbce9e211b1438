// vc_draft_attn_noalloc: the draft attention entry point for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops).  The split partials that vc_draft_attn keeps in the caller's
// workspace live here in a file-scope device array instead, one copy per
// GPU, held until the process ends.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>
#include <vector>

#include "launch.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;   // the largest split workspace this entry point serves

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
std::vector<void *> g_ptr;   // per device: the device address of `scratch` (null until first use)

// The device address of this GPU's copy of `scratch`.  Host code never uses
// the array's name as an address: it stands for a host-side shadow.
vc_status scratch_ptr(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return vc::set_error(VC_EHIP, hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_mu);
  if ((int)g_ptr.size() <= dev) g_ptr.resize(dev + 1, nullptr);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return vc::set_error(VC_EHIP, "hipGetSymbolAddress of the draft scratch array failed");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return VC_OK;
}

}  // namespace

extern "C" {

size_t vc_draft_noalloc_max_scratch(void) { return kScratchBytes; }

vc_status vc_draft_attn_noalloc(const vc_draft_args *a, void *stream) {
  if (!a) return vc::set_error(VC_EINVAL, "null argument struct");
  const size_t need = vc_draft_workspace_size(a);
  if (need > kScratchBytes) {
    char m[160];
    snprintf(m, sizeof m, "this call needs %zu bytes of split scratch, above the %zu-byte static array", need,
             kScratchBytes);
    return vc::set_error(VC_EINVAL, m);
  }
  vc_draft_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (need && a->B > 0) {
    const vc_status st = scratch_ptr(&b.workspace);
    if (st != VC_OK) return st;
    b.workspace_bytes = kScratchBytes;
  }
  return vc_draft_attn(&b, stream);
}

}  // extern "C"
