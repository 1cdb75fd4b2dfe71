// gemm_inst.hip - one instantiation of the GEMM's launcher (and so of its
// kernels) for the operand formats MXQ_FA x MXQ_FB and the mode
// MXQ_PRECISE, given on the compiler's command line.  The build compiles
// this file once per format pair and mode, in parallel.
#include "gemm_kernel.h"

#if !defined(MXQ_FA) || !defined(MXQ_FB) || !defined(MXQ_PRECISE)
#error "MXQ_FA, MXQ_FB and MXQ_PRECISE must be defined"
#endif

namespace mxq {
template hipError_t launch_t<MXQ_FA, MXQ_FB, (MXQ_PRECISE != 0)>(const GemmArgs&, hipStream_t);
#if MXQ_PRECISE == 0 && MXQ_FA != 2 && MXQ_FB != 2
// FP8 x FP8: also the up-projection with the SwiGLU + MX epilogue
template hipError_t launch_swiglu_t<MXQ_FA, MXQ_FB>(const GemmArgs&, hipStream_t);
#endif
}  // namespace mxq
