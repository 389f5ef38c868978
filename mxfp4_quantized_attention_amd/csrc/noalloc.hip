// noalloc.hip -- mxattn_fwd for callers that cannot allocate device memory.
//
// mxattn_fwd needs device memory beyond its inputs and output: the quantized
// K and V (codes and E8M0 scales) that the two quantize passes write and the
// fused attention kernel reads.  This entry point keeps them in a file-scope
// device array of the library instead of a caller-provided workspace, so it
// makes no allocation at all (no hipMalloc, no allocating library routine):
// usable under HIP graph capture, in tight serving loops and in harnesses
// that forbid allocation.  The kernels and the workspace layout are those of
// mxattn_fwd, so the results are bit-identical to it.
//
// The array is kNoAllocScratchBytes (256 MiB): every GPU the library runs on
// holds one copy of it until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): the device address of each GPU's copy is looked up once per device
// with hipGetSymbolAddress, with that device current, and used from then on.
// Every call on one GPU shares that GPU's copy, so calls that overlap in time
// on one GPU race; calls must be ordered (one stream, or synchronized).
#include <hip/hip_runtime.h>

#include <mutex>

#include "mxattn.h"

namespace {

constexpr size_t kNoAllocScratchBytes = size_t(256) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// Per-device address of `scratch`, looked up once per device (with that
// device current) and kept for the life of the process.
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

int scratch_on_current_device(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MXQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MXQ_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return MXQ_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MXQ_OK;
}

}  // namespace

extern "C" {

size_t mxattn_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int mxattn_fwd_noalloc(const void* q, const void* k, const void* v, int64_t B, int64_t H, int64_t N, int64_t d,
                       int mode, int pnq, float softmax_scale, void* o, void* stream) {
  const size_t need = mxattn_workspace_bytes(B, H, N, d);
  if (need == 0 || need > kNoAllocScratchBytes) {
    // Bad sizes, or a problem whose K/V operands do not fit the array:
    // mxattn_fwd without a workspace returns the size or argument error, or
    // else MXQ_ERR_WORKSPACE, before anything is enqueued.
    return mxattn_fwd(q, k, v, B, H, N, d, mode, pnq, softmax_scale, o, nullptr, 0, stream);
  }
  void* ws = nullptr;
  const int st = scratch_on_current_device(&ws);
  if (st != MXQ_OK) return st;
  // mxattn_fwd with the array as its workspace: same checks, same kernels,
  // same layout.  Every byte its attention kernel reads is written by its two
  // quantize passes in the same call (the kernel's buffer reads are range
  // checked to this call's regions), so nothing left by an earlier call is
  // read and nothing needs clearing.
  return mxattn_fwd(q, k, v, B, H, N, d, mode, pnq, softmax_scale, o, ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"
