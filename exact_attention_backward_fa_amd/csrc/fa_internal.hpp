// Host-side plumbing shared by the C entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Head dims with a kernel instance (every kernel family but the fused atomic one,
// which is built for 64 and 128 only).
constexpr bool head_dim_supported(int d) {
  return d == 32 || d == 64 || d == 96 || d == 128 || d == 256;
}
constexpr bool atomic_head_dim(int d) { return d == 64 || d == 128; }

// Call FN<DT, D, CAUSAL>(args...) for a problem's (dtype, head dim, causal).
#define FA_DISPATCH_D(DT, PB, FN, ...)                                                        \
  switch ((PB).d) {                                                                          \
    case 32: return (PB).causal ? FN<DT, 32, true>(__VA_ARGS__) : FN<DT, 32, false>(__VA_ARGS__); \
    case 64: return (PB).causal ? FN<DT, 64, true>(__VA_ARGS__) : FN<DT, 64, false>(__VA_ARGS__); \
    case 96: return (PB).causal ? FN<DT, 96, true>(__VA_ARGS__) : FN<DT, 96, false>(__VA_ARGS__); \
    case 128:                                                                                \
      return (PB).causal ? FN<DT, 128, true>(__VA_ARGS__) : FN<DT, 128, false>(__VA_ARGS__);   \
    case 256:                                                                                \
      return (PB).causal ? FN<DT, 256, true>(__VA_ARGS__) : FN<DT, 256, false>(__VA_ARGS__);   \
    default:                                                                                 \
      return hipErrorInvalidValue;                                                           \
  }
#define FA_DISPATCH(PB, FN, ...)                        \
  do {                                                  \
    if ((PB).dtype == 0) {                              \
      FA_DISPATCH_D(0, PB, FN, __VA_ARGS__)             \
    } else {                                            \
      FA_DISPATCH_D(1, PB, FN, __VA_ARGS__)             \
    }                                                   \
  } while (0)

// Validated arguments of one call (sizes already checked, pointers device-side).
struct Problem {
  int B, Hq, Hkv, Nq, Nkv, d;
  float scale;
  bool causal;
  int dtype;  // 0 fp16, 1 bf16
};

struct FwdArgs {
  Problem pb;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
};

struct BwdArgs {
  Problem pb;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* ndelta;  // [B*Hq*Nq]      -rowsum(dO o O)
  float* lse2;    // [B*Hq*Nq]      LSE * log2(e), +inf for rows that see no key
  float* dq_acc;  // [B*Hq*Nq*d]    float32 dQ accumulator (atomic path only)
  int* sched;     // [32]           work-queue counters of the dK/dV and dQ kernels (zeroed
                  //                by the preprocess); null: static work split
};

// Arguments of one backward call as the C entry points receive them (unchecked).
struct BwdCall {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Nq, Nkv, d;
  float scale;
  int causal, dtype;
};

// Checks every argument of a backward call on the host (no device call); on
// FA_OK sets *workspace_need to the workspace bytes the call needs.
int bwd_validate(const BwdCall& c, int dq_mode, size_t* workspace_need);
// Checks every argument of a backward call on the host, then enqueues the
// kernels with `workspace` as the scratch memory; returns FA_OK or an FA_ERR_*
// code (nothing is launched or written on error).
int bwd_checked(const BwdCall& c, int dq_mode, void* ev_begin, void* ev_end, void* workspace,
                size_t workspace_bytes, void* stream);
// Workspace bytes of a backward call with this dQ path (0 for invalid arguments).
size_t bwd_workspace_checked(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal, int dtype,
                             int dq_mode);

// Workspace carve-up; every region starts on a 256-byte boundary.
struct WorkspaceLayout {
  size_t ndelta_off, lse2_off, dqacc_off, sched_off, total;
};
WorkspaceLayout workspace_layout(const Problem& pb, bool atomic_dq);

// Kernel launchers (return hipSuccess or the launch error).
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s);
// The forward launcher of one template instance (dtype 0 fp16 / 1 bf16, head dim,
// causal), defined in fa_fwd_kernels.hpp.
template <int DT, int D, bool CAUSAL> hipError_t run_fwd(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_pre(const BwdArgs& a, bool zero_dq_acc, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, bool atomic_dq, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dq_convert(const BwdArgs& a, hipStream_t s);

// Compute units of the current device (cached per device; 0 if it cannot be read).
int device_cu_count();

}  // namespace fa
