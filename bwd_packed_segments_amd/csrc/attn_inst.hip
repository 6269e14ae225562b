// One translation unit per (element type, Dqk, Dv): the build compiles this
// file once for every head-dim pair the library supports, with INST_T,
// INST_DQK and INST_DV set on the command line, so the instantiations build
// in parallel.
#include "attn_kernels.hpp"

#if !defined(INST_T) || !defined(INST_DQK) || !defined(INST_DV)
#error "INST_T, INST_DQK and INST_DV must be defined"
#endif

namespace bps {
template hipError_t launch_fwd<INST_T, INST_DQK, INST_DV>(const FwdArgs&, hipStream_t);
template hipError_t launch_bwd_delta<INST_T, INST_DQK, INST_DV>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dkdv<INST_T, INST_DQK, INST_DV>(const BwdArgs&, hipStream_t);
template hipError_t launch_bwd_dq<INST_T, INST_DQK, INST_DV>(const BwdArgs&, hipStream_t);
}  // namespace bps
