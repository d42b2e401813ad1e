// fa_bwd_noalloc: the backward for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).  Its
// scratch memory - the per-row -D and LSE*log2(e) that the dQ pass leaves for the
// dK/dV kernel, and the two kernels' work-queue counters - lives in a file-scope
// device array instead of a caller workspace.  Each device holds its own copy of
// the array until the process ends; host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address).  Every call on a device shares that device's array, so calls
// that overlap on one device race; every call clears the counters (with a kernel,
// not a memset) before the kernels that use them run.
#include "fa_mi355x.h"

#include <mutex>

#include "fa_internal.hpp"

namespace fa {

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, looked up once per device with
// that device current; null if the lookup fails.
void* scratch_of_current_device(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = FA_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      *status = FA_ERR_HIP;
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  *status = FA_OK;
  return g_ptr[dev];
}

}  // namespace
}  // namespace fa

extern "C" {

size_t fa_bwd_noalloc_max_scratch_bytes(void) { return FA_NOALLOC_SCRATCH_BYTES; }

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
                   int Nkv, int d, float softmax_scale, int causal, int dtype, void* stream) {
  // Only the separate dQ path: the atomic path's float32 dQ buffer (B*Hq*N_q*d
  // floats) is not a bounded size.  Every check runs before any device call.
  const fa::BwdCall c{q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, d, softmax_scale,
                      causal, dtype};
  size_t need = 0;
  int st = fa::bwd_validate(c, FA_DQ_SEPARATE, &need);
  if (st != FA_OK) return st;
  if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    ws = fa::scratch_of_current_device(&st);
    if (st != FA_OK) return st;
  }
  return fa::bwd_checked(c, FA_DQ_SEPARATE, nullptr, nullptr, ws, need, stream);
}

}  // extern "C"
