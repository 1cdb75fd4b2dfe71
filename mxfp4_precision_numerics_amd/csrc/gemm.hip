// gemm.hip - dispatch of the scaled GEMM on its operand formats and mode to
// the launchers that gemm_inst.hip instantiates (kernels in gemm_kernel.h).
#include "common.h"
#include "launch.h"

namespace mxq {

hipError_t launch_scaled_gemm(const GemmArgs& a, hipStream_t st) {
    if (a.precise) {
        switch (a.fa * 3 + a.fb) {
        case E4M3 * 3 + E4M3: return launch_t<E4M3, E4M3, true>(a, st);
        case E4M3 * 3 + E5M2: return launch_t<E4M3, E5M2, true>(a, st);
        case E5M2 * 3 + E4M3: return launch_t<E5M2, E4M3, true>(a, st);
        case E5M2 * 3 + E5M2: return launch_t<E5M2, E5M2, true>(a, st);
        }
        return hipErrorInvalidValue;
    }
    switch (a.fa * 3 + a.fb) {
    case E4M3 * 3 + E4M3: return launch_t<E4M3, E4M3, false>(a, st);
    case E4M3 * 3 + E5M2: return launch_t<E4M3, E5M2, false>(a, st);
    case E4M3 * 3 + E2M1: return launch_t<E4M3, E2M1, false>(a, st);
    case E5M2 * 3 + E4M3: return launch_t<E5M2, E4M3, false>(a, st);
    case E5M2 * 3 + E5M2: return launch_t<E5M2, E5M2, false>(a, st);
    case E5M2 * 3 + E2M1: return launch_t<E5M2, E2M1, false>(a, st);
    case E2M1 * 3 + E4M3: return launch_t<E2M1, E4M3, false>(a, st);
    case E2M1 * 3 + E5M2: return launch_t<E2M1, E5M2, false>(a, st);
    case E2M1 * 3 + E2M1: return launch_t<E2M1, E2M1, false>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_grouped_swiglu(const GemmArgs& a, hipStream_t st) {
    switch (a.fa * 3 + a.fb) {
    case E4M3 * 3 + E4M3: return launch_swiglu_t<E4M3, E4M3>(a, st);
    case E4M3 * 3 + E5M2: return launch_swiglu_t<E4M3, E5M2>(a, st);
    case E5M2 * 3 + E4M3: return launch_swiglu_t<E5M2, E4M3>(a, st);
    case E5M2 * 3 + E5M2: return launch_swiglu_t<E5M2, E5M2>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace mxq
