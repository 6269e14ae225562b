// One translation unit per (element type, Dqk, Dv, kernel family, variants):
// the build compiles this file once for every combination, with INST_T,
// INST_DQK, INST_DV, INST_PART (0 forward, 1 Delta + dQ, 2 dK/dV) and
// INST_VAR (0 plain kernels, 1 kernels that apply bias, soft-capping, sink
// and max logit; for the forward also 2, the kernel for bias and soft-cap,
// 1 being the one for sink and max logit alone) set on the command line.  Keeping the kernel families apart
// also keeps the code generated for one from depending on the others.
#include "attn_kernels.hpp"

#if !defined(INST_T) || !defined(INST_DQK) || !defined(INST_DV) || !defined(INST_PART) || !defined(INST_VAR)
#error "INST_T, INST_DQK, INST_DV, INST_PART and INST_VAR must be defined"
#endif

namespace bps {
#if INST_PART == 0
template hipError_t launch_fwd<INST_T, INST_DQK, INST_DV, INST_VAR>(const FwdArgs&, hipStream_t);
#elif INST_PART == 1
template hipError_t launch_bwd_delta<INST_T, INST_DQK, INST_DV, INST_VAR != 0>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<INST_T, INST_DQK, INST_DV, INST_VAR != 0>(const BwdArgs&, hipStream_t);
#else
template hipError_t launch_bwd_dkdv<INST_T, INST_DQK, INST_DV, INST_VAR != 0>(const BwdArgs&, hipStream_t);
#endif
}  // namespace bps
