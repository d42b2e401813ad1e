// Forward entry point: dispatch of a problem to its instance of the forward kernel
// (fa_fwd_kernels.hpp, instantiated one instance per compilation of fa_fwd_inst.hip).
#include "fa_internal.hpp"

namespace fa {

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if ((size_t)a.pb.B * a.pb.Nq == 0) return hipSuccess;
  FA_DISPATCH(a.pb, run_fwd, a, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
