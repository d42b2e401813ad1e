// Forward entry point: dispatch of a problem to its instance of the forward kernel
// (fa_fwd_kernels.hpp, instantiated one instance per compilation of fa_fwd_inst.hip).
#include "fa_internal.hpp"

namespace fa {

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if ((size_t)a.pb.B * a.pb.Nq == 0) return hipSuccess;
  return dispatch(a.pb, a.x.ft(), [&](auto dt, auto d, auto c, auto ft) {
    return run_fwd<decltype(dt)::value, decltype(d)::value, decltype(c)::value, decltype(ft)::value>(a, s);
  });
}

}  // namespace fa
