// Host-side plumbing shared by the C entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

// Head dims with a kernel instance: every multiple of 32 up to 256 (every kernel
// family but the fused atomic one, which is built for 64 and 128 only).
constexpr bool head_dim_supported(int d) { return d > 0 && d <= 256 && d % 32 == 0; }
constexpr bool atomic_head_dim(int d) { return d == 64 || d == 128; }

// Kernel feature set of an instance: 0 plain attention, 1 with an additive score
// bias (and its gradient), 2 with the bias and dropout of P, 3 with a bias that
// depends on the batch and the key only (a key-padding mask, say) and no gradient
// for it: the plain kernels' shape, the bias entering the score products; 4 with
// dropout and no bias.
enum : int { FT_PLAIN = 0, FT_BIAS = 1, FT_DROPOUT = 2, FT_KEYBIAS = 3, FT_DROP = 4 };
// Head dims with the instances of feature set ft: a bias per (batch, key) at every
// head dim; bias tiles, dBias and dropout at 64 and 128.
constexpr bool feature_head_dim(int ft, int d) {
  return ft == FT_KEYBIAS ? head_dim_supported(d) : (d == 64 || d == 128);
}
// instances that stream 2-D bias tiles through LDS (32-row shape)
constexpr bool tile_bias(int ft) { return ft == FT_BIAS || ft == FT_DROPOUT; }

// Validated arguments of one call (sizes already checked, pointers device-side).
struct Problem {
  int B, Hq, Hkv, Nq, Nkv, d;
  float scale;
  bool causal;
  int dtype;  // 0 fp16, 1 bf16
};

// Optional score bias and dropout of a call (defaults: neither).
struct Extras {
  const void* bias = nullptr;  // element (b, h, i, j) at b*sb + h*sh + i*sq + j; null: zero
  long long bias_sb = 0, bias_sh = 0, bias_sq = 0;
  void* dbias = nullptr;       // [B, Hq, N_q, N_kv] contiguous, or null
  unsigned keep_t = 256;       // dropout: keep iff the element's random byte < keep_t
  unsigned long long seed = 0;
  int ft() const {
    if (keep_t < 256) return (bias || dbias) ? FT_DROPOUT : FT_DROP;
    if (dbias) return FT_BIAS;
    if (bias) return (bias_sh == 0 && bias_sq == 0) ? FT_KEYBIAS : FT_BIAS;
    return FT_PLAIN;
  }
};

struct FwdArgs {
  Problem pb;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  Extras x;
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
                  //                before them); null: static work split
  Extras x;
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
int bwd_validate(const BwdCall& c, int dq_mode, size_t* workspace_need,
                 const Extras* x = nullptr);
// Checks every argument of a backward call on the host, then enqueues the
// kernels with `workspace` as the scratch memory; returns FA_OK or an FA_ERR_*
// code (nothing is launched or written on error).
int bwd_checked(const BwdCall& c, int dq_mode, void* ev_begin, void* ev_end, void* workspace,
                size_t workspace_bytes, void* stream, const Extras* x = nullptr);
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
// causal, feature set), defined in fa_fwd_kernels.hpp.
template <int DT, int D, bool CAUSAL, int FT> hipError_t run_fwd(const FwdArgs& a, hipStream_t s);

// Calls f(dtype, head dim, causal, feature set) - each a std::integral_constant -
// for a problem's instance; hipErrorInvalidValue when none is built.
template <class F>
hipError_t dispatch(const Problem& pb, int ft, F&& f) {
  using std::integral_constant;
  auto by_ft = [&](auto dt, auto d, auto c) -> hipError_t {
    if constexpr (feature_head_dim(FT_BIAS, decltype(d)::value)) {
      if (ft == FT_BIAS) return f(dt, d, c, integral_constant<int, FT_BIAS>());
      if (ft == FT_DROPOUT) return f(dt, d, c, integral_constant<int, FT_DROPOUT>());
      if (ft == FT_DROP) return f(dt, d, c, integral_constant<int, FT_DROP>());
    }
    if constexpr (feature_head_dim(FT_KEYBIAS, decltype(d)::value)) {
      if (ft == FT_KEYBIAS) return f(dt, d, c, integral_constant<int, FT_KEYBIAS>());
    }
    if (ft != FT_PLAIN) return hipErrorInvalidValue;
    return f(dt, d, c, integral_constant<int, FT_PLAIN>());
  };
  auto by_c = [&](auto dt, auto d) -> hipError_t {
    return pb.causal ? by_ft(dt, d, integral_constant<bool, true>())
                     : by_ft(dt, d, integral_constant<bool, false>());
  };
  auto by_d = [&](auto dt) -> hipError_t {
    switch (pb.d) {
      case 32: return by_c(dt, integral_constant<int, 32>());
      case 64: return by_c(dt, integral_constant<int, 64>());
      case 96: return by_c(dt, integral_constant<int, 96>());
      case 128: return by_c(dt, integral_constant<int, 128>());
      case 160: return by_c(dt, integral_constant<int, 160>());
      case 192: return by_c(dt, integral_constant<int, 192>());
      case 224: return by_c(dt, integral_constant<int, 224>());
      case 256: return by_c(dt, integral_constant<int, 256>());
      default: return hipErrorInvalidValue;
    }
  };
  return pb.dtype == 0 ? by_d(integral_constant<int, 0>()) : by_d(integral_constant<int, 1>());
}
// Row preprocess kernel of the atomic dQ path (-D, LSE * log2 e, counters
// cleared, float32 dQ buffer zeroed); on the separate path the dQ pass does the
// row preprocess and launch_sched_clear clears the counters.
hipError_t launch_bwd_pre(const BwdArgs& a, hipStream_t s);
hipError_t launch_sched_clear(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, bool atomic_dq, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dq_convert(const BwdArgs& a, hipStream_t s);
// zeros into the dBias entries the causal mask hides (no-op without dBias or mask)
hipError_t launch_dbias_fill(const BwdArgs& a, hipStream_t s);

// Compute units of the current device (cached per device; 0 if it cannot be read).
int device_cu_count();

}  // namespace fa
