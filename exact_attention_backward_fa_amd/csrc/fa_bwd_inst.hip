// One template instance of the backward kernels, selected by -DFA_DT (0 fp16,
// 1 bf16), -DFA_D (64 or 128) and -DFA_CAUSAL (0 or 1); the build compiles this
// file once per instance, in parallel.
#include "fa_bwd_atomic.hpp"
#include "fa_bwd_kernels.hpp"

namespace fa {

template hipError_t run_pre<FA_DT, FA_D, FA_CAUSAL != 0>(const BwdArgs&, bool, hipStream_t);
template hipError_t run_dkdv<FA_DT, FA_D, FA_CAUSAL != 0>(const BwdArgs&, hipStream_t);
template hipError_t run_dq<FA_DT, FA_D, FA_CAUSAL != 0>(const BwdArgs&, hipStream_t);
template hipError_t run_dkdv_atomic<FA_DT, FA_D, FA_CAUSAL != 0>(const BwdArgs&, hipStream_t);

}  // namespace fa
