// One template instance of one backward kernel family, selected by -DFA_DT (0 fp16,
// 1 bf16), -DFA_D (head dim), -DFA_CAUSAL (0 or 1), -DFA_FT (feature set: 0 plain,
// 1 score bias, 2 bias and dropout, 3 key bias; dK/dV and dQ pass only) and
// -DFA_KIND (0 row preprocess of the atomic path, 1 dK/dV, 2 dQ pass, 3 fused dK/dV
// with atomic dQ); the build compiles this file once per (instance, kind), in
// parallel.
#if FA_KIND == 3
#include "fa_bwd_atomic.hpp"
#else
#include "fa_bwd_kernels.hpp"
#endif

namespace fa {

#if FA_KIND == 0
template hipError_t run_pre<FA_DT, FA_D, FA_CAUSAL != 0>(const BwdArgs&, hipStream_t);
#elif FA_KIND == 1
template hipError_t run_dkdv<FA_DT, FA_D, FA_CAUSAL != 0, FA_FT>(const BwdArgs&, hipStream_t);
#elif FA_KIND == 2
template hipError_t run_dq<FA_DT, FA_D, FA_CAUSAL != 0, FA_FT>(const BwdArgs&, hipStream_t);
#else
template hipError_t run_dkdv_atomic<FA_DT, FA_D, FA_CAUSAL != 0>(const BwdArgs&, hipStream_t);
#endif

}  // namespace fa
