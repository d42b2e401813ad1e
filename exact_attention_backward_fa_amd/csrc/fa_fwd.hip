// Forward entry point: dispatch of a problem to its instance of the forward kernel
// (fa_fwd_kernels.hpp, instantiated one instance per compilation of fa_fwd_inst.hip).
#include "fa_internal.hpp"

namespace fa {

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if ((size_t)a.pb.B * a.pb.Nq == 0) return hipSuccess;
  const int key = a.pb.dtype * 4 + (a.pb.d == 128 ? 2 : 0) + (a.pb.causal ? 1 : 0);
  switch (key) {
    case 0: return run_fwd<0, 64, false>(a, s);
    case 1: return run_fwd<0, 64, true>(a, s);
    case 2: return run_fwd<0, 128, false>(a, s);
    case 3: return run_fwd<0, 128, true>(a, s);
    case 4: return run_fwd<1, 64, false>(a, s);
    case 5: return run_fwd<1, 64, true>(a, s);
    case 6: return run_fwd<1, 128, false>(a, s);
    default: return run_fwd<1, 128, true>(a, s);
  }
}

}  // namespace fa
