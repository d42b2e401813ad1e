// One template instance of the forward kernel, selected by -DFA_DT (0 fp16, 1 bf16),
// -DFA_D (head dim), -DFA_CAUSAL (0 or 1) and -DFA_FT (feature set: 0 plain, 1
// score bias, 2 bias and dropout); the build compiles this file once per instance,
// in parallel.
#include "fa_fwd_kernels.hpp"

namespace fa {

template hipError_t run_fwd<FA_DT, FA_D, FA_CAUSAL != 0, FA_FT>(const FwdArgs&, hipStream_t);

}  // namespace fa
