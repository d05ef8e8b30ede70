// ttt_forward_noalloc: the forward pass for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  Its scratch memory is a file-scope device array of
// a fixed size, kNoallocScratchBytes per GPU, instead of a caller workspace.
//
// The array lives in this file's code object, so every GPU the library runs on
// holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the device
// symbol): on the first call on a device, with that device current, its device
// address is looked up once with hipGetSymbolAddress and kept per device; every
// later call on that device passes that address as the workspace of
// ttt_forward.  No call here allocates or frees memory, and none creates a
// stream or an event (a request with several head ranges uses the handle's
// second stream only if an earlier ttt_forward created it).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ttt.h"
#include "ttt_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[ttt::kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

extern "C" int ttt_forward_noalloc(ttt_handle* h, const void* q, const void* k, const void* v, const ttt_weights* W0,
                                   const ttt_eta* eta, int loss, int inner, int chunk, void* o,
                                   const ttt_weights_out* W_out, void* stream) {
  if (!h) return ttt::set_error(nullptr, TTT_ERR_INVALID, "handle is NULL");
  size_t need = 0;
  int rc = ttt_workspace_bytes(h, loss, inner, chunk, &need);
  if (rc != TTT_OK) return rc;
  if (need > ttt::kNoallocScratchBytes)
    return ttt::set_error(h, TTT_ERR_WORKSPACE,
                          "request needs %zu bytes of scratch, more than the %zu bytes ttt_forward_noalloc holds per "
                          "device; use ttt_forward with a caller workspace",
                          need, (size_t)ttt::kNoallocScratchBytes);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ttt::set_error(h, TTT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return ttt::set_error(h, TTT_ERR_UNSUPPORTED, "device index %d out of range", dev);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return ttt::set_error(h, TTT_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                              hipGetErrorString(e));
      g_scratch[dev] = p;
    }
    ws = g_scratch[dev];
  }
  return ttt::forward_no_create(h, q, k, v, W0, eta, loss, inner, chunk, o, W_out, ws, ttt::kNoallocScratchBytes,
                                stream);
}

static_assert(ttt::kNoallocScratchBytes == TTT_NOALLOC_SCRATCH_BYTES, "header and library disagree on the size");
