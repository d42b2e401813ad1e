// Kernel parameters and dispatch shared by the backward kernels.
#pragma once

#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* ndelta;  // minus D per query row
  float* lse2;
  float* dq_acc;
  int B, Hq, Hkv, Nq, Nkv, G, off;  // off = Nkv - Nq (bottom-right causal offset)
  float scale, scale_log2;
  size_t rows;  // B * Hq * Nq
};

inline BwdParams make_params(const BwdArgs& a) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<const uint16_t*>(a.o);
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.dq = static_cast<uint16_t*>(a.dq);
  p.dk = static_cast<uint16_t*>(a.dk);
  p.dv = static_cast<uint16_t*>(a.dv);
  p.ndelta = a.ndelta;
  p.lse2 = a.lse2;
  p.dq_acc = a.dq_acc;
  p.B = a.pb.B;
  p.Hq = a.pb.Hq;
  p.Hkv = a.pb.Hkv;
  p.Nq = a.pb.Nq;
  p.Nkv = a.pb.Nkv;
  p.G = a.pb.Hq / a.pb.Hkv;
  p.off = a.pb.Nkv - a.pb.Nq;
  p.scale = a.pb.scale;
  p.scale_log2 = a.pb.scale * kLog2e;
  p.rows = (size_t)a.pb.B * a.pb.Hq * a.pb.Nq;
  return p;
}

// Launchers of one template instance; each is explicitly instantiated in its own
// compilation of fa_bwd_inst.hip.
template <int DT, int D, bool CAUSAL> hipError_t run_pre(const BwdArgs& a, bool zero, hipStream_t s);
template <int DT, int D, bool CAUSAL> hipError_t run_dkdv(const BwdArgs& a, hipStream_t s);
template <int DT, int D, bool CAUSAL> hipError_t run_dq(const BwdArgs& a, hipStream_t s);
template <int DT, int D, bool CAUSAL> hipError_t run_dkdv_atomic(const BwdArgs& a, hipStream_t s);

// Template instance for a problem: dtype (0 fp16, 1 bf16), head dim, causal.
inline int dispatch_key(const Problem& pb) {
  return pb.dtype * 4 + (pb.d == 128 ? 2 : 0) + (pb.causal ? 1 : 0);
}

#define FA_DISPATCH(KEY, FN, ...)                        \
  switch (KEY) {                                         \
    case 0: return FN<0, 64, false>(__VA_ARGS__);        \
    case 1: return FN<0, 64, true>(__VA_ARGS__);         \
    case 2: return FN<0, 128, false>(__VA_ARGS__);       \
    case 3: return FN<0, 128, true>(__VA_ARGS__);        \
    case 4: return FN<1, 64, false>(__VA_ARGS__);        \
    case 5: return FN<1, 64, true>(__VA_ARGS__);         \
    case 6: return FN<1, 128, false>(__VA_ARGS__);       \
    default: return FN<1, 128, true>(__VA_ARGS__);       \
  }

}  // namespace fa
