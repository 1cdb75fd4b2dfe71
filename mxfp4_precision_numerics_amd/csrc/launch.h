// launch.h - internal launchers behind the C ABI (arguments already
// validated on the host by mxq_api.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

hipError_t launch_quantize_per_tensor(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int fmt,
                                      float* history, int hist_len, float* amax_out, float* scale_out,
                                      float* scale_inv_out, uint8_t* q_row, uint8_t* q_col, hipStream_t st);

hipError_t launch_quantize_mx(const void* x, int src, int64_t rows, int64_t cols, int64_t ld, int fmt, uint8_t* q_row,
                              uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, hipStream_t st);

hipError_t launch_swiglu_quantize_mx(const void* gu, int src, int64_t rows, int64_t inter, int64_t ld, int fmt,
                                     uint8_t* q, uint8_t* s, hipStream_t st);

hipError_t launch_repack_fp4_to_fp8(const uint8_t* q4, const uint8_t* s4, const int32_t* idx, int64_t src_rows,
                                    int64_t rows, int64_t cols, uint8_t* q8, uint8_t* s8, hipStream_t st);
hipError_t launch_fp4_row_to_fp8_col(const uint8_t* q4, const uint8_t* s4, int64_t rows, int64_t cols, uint8_t* q8,
                                     uint8_t* s8, hipStream_t st);

// Dense (group_off == nullptr) or grouped scaled GEMM.
struct GemmArgs {
    const uint8_t* A;
    const void* sA;
    const uint8_t* B;
    const void* sB;
    void* C;
    const int64_t* group_off;  // device [G+1] or nullptr
    int64_t G;
    int64_t M, N, K;  // M = total rows for the grouped form
    int64_t ldc;
    int64_t b_group_stride;  // bytes between consecutive B_g
    int64_t sb_group_stride; // bytes between consecutive sB_g (0 for per-tensor)
    int fa, fb, ma, mb, out;  // out: 0 fp32, 1 bf16
    int precise;              // exact products (FP8 x FP8 only; E2M1 x E2M1 is exact natively)
    // Expert-MLP epilogue (C unused): B_g = [gate rows 0..inter-1; up rows
    // inter..2 inter-1], N = 2 inter; each output row's h = silu(gate) * up
    // is MX block-32 quantized to q_out [M, inter] with scales s_out
    // [M, inter/32] in format hfmt.
    int swiglu;
    int hfmt;
    int64_t inter;
    uint8_t* q_out;
    uint8_t* s_out;
};
hipError_t launch_scaled_gemm(const GemmArgs& a, hipStream_t st);
// Grouped up-projection with the SwiGLU + MX epilogue (a.swiglu set).
hipError_t launch_grouped_swiglu(const GemmArgs& a, hipStream_t st);
// The launcher for one operand-format pair and mode (gemm_kernel.h;
// instantiated by gemm_inst.hip).
template <int FA, int FB, bool PRECISE>
hipError_t launch_t(const GemmArgs& a, hipStream_t st);
// The grouped GEMM with the SwiGLU + MX epilogue, FP8 operands.
template <int FA, int FB>
hipError_t launch_swiglu_t(const GemmArgs& a, hipStream_t st);

}  // namespace mxq
