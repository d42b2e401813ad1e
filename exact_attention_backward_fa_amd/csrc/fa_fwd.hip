// Forward entry point: dispatch of a problem to its instance of the forward kernel
// (fa_fwd_kernels.hpp).
#include "fa_fwd_kernels.hpp"

namespace fa {

template <int DT, int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  const Problem& pb = a.pb;
  FwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.o = static_cast<uint16_t*>(a.o);
  p.lse = a.lse;
  p.B = pb.B;
  p.Hq = pb.Hq;
  p.Hkv = pb.Hkv;
  p.Nq = pb.Nq;
  p.Nkv = pb.Nkv;
  p.G = pb.Hq / pb.Hkv;
  p.off = pb.Nkv - pb.Nq;
  p.scale_log2 = pb.scale * kLog2e;
  const dim3 grid((unsigned)(((pb.Nq + 255) / 256) * pb.Hq * pb.B));
  hipLaunchKernelGGL((fwd_kernel<DT, D, CAUSAL>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if ((size_t)a.pb.B * a.pb.Nq == 0) return hipSuccess;
  const int key = a.pb.dtype * 4 + (a.pb.d == 128 ? 2 : 0) + (a.pb.causal ? 1 : 0);
  switch (key) {
    case 0: return launch_fwd_t<0, 64, false>(a, s);
    case 1: return launch_fwd_t<0, 64, true>(a, s);
    case 2: return launch_fwd_t<0, 128, false>(a, s);
    case 3: return launch_fwd_t<0, 128, true>(a, s);
    case 4: return launch_fwd_t<1, 64, false>(a, s);
    case 5: return launch_fwd_t<1, 64, true>(a, s);
    case 6: return launch_fwd_t<1, 128, false>(a, s);
    default: return launch_fwd_t<1, 128, true>(a, s);
  }
}

}  // namespace fa
