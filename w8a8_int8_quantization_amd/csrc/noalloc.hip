// The one-call W8A8 linear layer with its scratch in a static device array:
// an entry point that allocates nothing, for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops or harnesses
// that forbid allocation).
//
// The scratch (Xq, the row scales, the split-K counters and partial tiles of
// sq_w8a8_linear_dyn's workspace) is `scratch`, a file-scope device array of
// SQ_STATIC_SCRATCH_BYTES that every GPU the library runs on holds until the
// process ends. Host code never uses the array's name as an address: on the
// first call on a device, with that device current, hipGetSymbolAddress gives
// that device's copy, and the address is kept per device. All calls on one
// GPU share its copy, which keeps the last call's contents; the split-K
// counters, the only part that must start at zero, are cleared by each call's
// own quantisation launch.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "sq.h"
#include "sq_launch.hpp"

namespace {

static __device__ __align__(256) unsigned char scratch[SQ_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of the scratch array (looked up once per device).
sq_status device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    sqh::set_last_hip_error((int)e);
    return SQ_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return SQ_ERR_RANGE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      sqh::set_last_hip_error((int)e);
      return SQ_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SQ_OK;
}

}  // namespace

extern "C" sq_status sq_w8a8_linear_dyn_static(const void* x, sq_dtype xt, int64_t ldx, const float* smooth,
                                               const int8_t* wq, const float* w_scale, int64_t m, int64_t n,
                                               int64_t k, void* y, sq_dtype yt, int64_t ldy, sq_stream_t stream) {
  // enum arguments are checked as ints before they are used (a C caller may
  // pass any int; see the C-ABI layer)
  int xv, yv;
  std::memcpy(&xv, &xt, sizeof xv);
  std::memcpy(&yv, &yt, sizeof yv);
  if (xv < (int)SQ_F32 || xv > (int)SQ_I8 || yv < (int)SQ_F32 || yv > (int)SQ_I8) return SQ_ERR_DTYPE;
  // empty problems and bad shapes go straight to the workspace entry point's
  // validation (it needs no scratch for them)
  const size_t need = sq_w8a8_linear_dyn_workspace_size(m, n, k);
  if (need > (size_t)SQ_STATIC_SCRATCH_BYTES) return SQ_ERR_WORKSPACE;
  if (need == 0) return sq_w8a8_linear_dyn(x, xt, ldx, smooth, wq, w_scale, m, n, k, y, yt, ldy, nullptr, 0, stream);
  void* ws = nullptr;
  const sq_status st = device_scratch(&ws);
  if (st != SQ_OK) return st;
  return sq_w8a8_linear_dyn(x, xt, ldx, smooth, wq, w_scale, m, n, k, y, yt, ldy, ws,
                            (size_t)SQ_STATIC_SCRATCH_BYTES, stream);
}
