// attn_noalloc.hip — attn_fwd_noalloc: attn_fwd whose workspace is a fixed
// array in device memory, for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array; in host code its name is only a
// host-side stand-in, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever handed to kernels. Each GPU holds its own copy at its own address.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/attn.h"
#include "attn_internal.hpp"

// The array itself. No kernel names it; the host-side use below is what keeps
// it in the device code object, where the runtime finds it by name.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace attn {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up

// Device address of `scratch` on the current device (looked up on first use).
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

}  // namespace attn

extern "C" int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B,
                                int Hq, int Hkv, int Nq, int Nk, int D, int causal, int window_lo,
                                int pos0, float scale, int mode, int dtype, void* stream) {
  int st = attn::fwd_validate(q, k, v, o, B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, scale,
                              mode, dtype);
  if (st != ATTN_OK) return st;
  // (the split prefill runs only where its workspace fits in the array too)
  const size_t need = attn::fwd_min_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, causal, window_lo,
                                                    pos0, mode, dtype);
  if (need > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_E_TOO_LARGE;
  if (stream != nullptr) {
    int sdev = -1, cur = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess ||
        hipGetDevice(&cur) != hipSuccess)
      return ATTN_E_HIP;
    if (sdev != cur) return ATTN_E_INVALID;
  }
  void* ws = nullptr;
  if (attn::scratch_on_current_device(&ws) != hipSuccess) return ATTN_E_HIP;
  return attn_fwd(q, k, v, o, B, Hq, Hkv, Nq, Nk, D, causal, window_lo, pos0, scale, mode, dtype,
                  ws, ATTN_NOALLOC_SCRATCH_BYTES, stream);
}
