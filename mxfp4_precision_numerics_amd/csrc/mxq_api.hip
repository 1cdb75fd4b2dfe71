// mxq_api.hip - the extern "C" entry points declared in include/mxq.h.
// Every argument is validated on the host before any HIP call; the launchers
// in the kernel files run only on arguments that passed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxq.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
int hip_status(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_ERR_HIP; }

constexpr int64_t MAX_GRID_Y = 65535;
constexpr int64_t MAX_GRID_X = 0x7FFFFFFF;

bool valid_fmt(int f) { return f == MXQ_E4M3 || f == MXQ_E5M2 || f == MXQ_E2M1; }
bool valid_mode(int m) { return m == MXQ_SCALE_TENSOR || m == MXQ_SCALE_BLK32 || m == MXQ_SCALE_BLK128; }

}  // namespace

extern "C" {

int mxq_abi_version(void) { return MXQ_ABI_VERSION; }

const char* mxq_status_string(int status) {
    switch (status) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "a required pointer is NULL";
    case MXQ_ERR_SHAPE: return "invalid size or divisibility";
    case MXQ_ERR_ALIGN: return "pointer or row pitch not 16-byte aligned";
    case MXQ_ERR_FORMAT: return "unsupported format, scale mode or source type";
    case MXQ_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
    }
}

int mxq_quantize_per_tensor(const void* x, int src, int64_t rows, int64_t cols, int64_t ld_x, int fmt,
                            float* amax_history, int history_len, float* amax_out, float* scale_out,
                            float* scale_inv_out, uint8_t* q_row, uint8_t* q_col, void* stream) {
    if (src != MXQ_SRC_F32 && src != MXQ_SRC_BF16) return MXQ_ERR_FORMAT;
    if (fmt != MXQ_E4M3 && fmt != MXQ_E5M2) return MXQ_ERR_FORMAT;
    if (rows < 0 || cols < 0 || history_len < 0 || history_len > 1024) return MXQ_ERR_SHAPE;
    if (cols % 16 != 0 || ld_x < cols) return MXQ_ERR_SHAPE;
    if (q_col && rows % 16 != 0) return MXQ_ERR_SHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || !amax_out || !scale_out || (!q_row && !q_col)) return MXQ_ERR_NULL;
    if (history_len > 0 && !amax_history) return MXQ_ERR_NULL;
    if ((rows + 127) / 128 > MAX_GRID_Y) return MXQ_ERR_SHAPE;
    const int64_t esz = src == MXQ_SRC_BF16 ? 2 : 4;
    if (!aligned16(x) || (ld_x * esz) % 16 != 0) return MXQ_ERR_ALIGN;
    if ((q_row && !aligned16(q_row)) || (q_col && !aligned16(q_col))) return MXQ_ERR_ALIGN;
    if (!aligned4(amax_out) || !aligned4(scale_out) || (scale_inv_out && !aligned4(scale_inv_out)) ||
        (amax_history && !aligned4(amax_history)))
        return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_quantize_per_tensor(x, src, rows, cols, ld_x, fmt, amax_history, history_len,
                                                      amax_out, scale_out, scale_inv_out, q_row, q_col,
                                                      as_stream(stream)));
}

int mxq_quantize_mx(const void* x, int src, int64_t rows, int64_t cols, int64_t ld_x, int fmt, uint8_t* q_row,
                    uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, void* stream) {
    if (src != MXQ_SRC_F32 && src != MXQ_SRC_BF16) return MXQ_ERR_FORMAT;
    if (!valid_fmt(fmt)) return MXQ_ERR_FORMAT;
    if (q_col && fmt == MXQ_E2M1) return MXQ_ERR_FORMAT;
    if (rows < 0 || cols < 0) return MXQ_ERR_SHAPE;
    if (cols % 32 != 0 || ld_x < cols) return MXQ_ERR_SHAPE;
    if (q_col && rows % 32 != 0) return MXQ_ERR_SHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!x || (!q_row && !q_col)) return MXQ_ERR_NULL;
    if ((q_row && !s_row) || (q_col && !s_col)) return MXQ_ERR_NULL;
    if (q_col && (rows + 127) / 128 > MAX_GRID_Y) return MXQ_ERR_SHAPE;
    if (!q_col && rows * (cols / 8) / 512 + 1 > MAX_GRID_X) return MXQ_ERR_SHAPE;  // 512 vectors per block
    const int64_t esz = src == MXQ_SRC_BF16 ? 2 : 4;
    if (!aligned16(x) || (ld_x * esz) % 16 != 0) return MXQ_ERR_ALIGN;
    if ((q_row && !aligned16(q_row)) || (s_row && !aligned16(s_row)) || (q_col && !aligned16(q_col)) ||
        (s_col && !aligned16(s_col)))
        return MXQ_ERR_ALIGN;
    return hip_status(
        mxq::launch_quantize_mx(x, src, rows, cols, ld_x, fmt, q_row, s_row, q_col, s_col, as_stream(stream)));
}

int mxq_repack_fp4_to_fp8(const uint8_t* q4, const uint8_t* s4, const int32_t* gather_idx, int64_t src_rows,
                          int64_t rows, int64_t cols, uint8_t* q8, uint8_t* s8, void* stream) {
    if (rows < 0 || cols < 0 || src_rows < 0) return MXQ_ERR_SHAPE;
    if (cols % 128 != 0) return MXQ_ERR_SHAPE;
    if (!gather_idx && rows > src_rows) return MXQ_ERR_SHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!q4 || !s4 || !q8 || !s8) return MXQ_ERR_NULL;
    if (rows * (cols / 128) * 4 / 256 + 1 > MAX_GRID_X) return MXQ_ERR_SHAPE;  // one 32-block per lane
    if (!aligned16(q4) || !aligned16(s4) || !aligned16(q8) || !aligned16(s8) ||
        (gather_idx && !aligned4(gather_idx)))
        return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_repack_fp4_to_fp8(q4, s4, gather_idx, src_rows, rows, cols, q8, s8,
                                                    as_stream(stream)));
}

int mxq_fp4_row_to_fp8_col(const uint8_t* q4, const uint8_t* s4, int64_t rows, int64_t cols, uint8_t* q8,
                           uint8_t* s8, void* stream) {
    if (rows < 0 || cols < 0) return MXQ_ERR_SHAPE;
    if (rows % 32 != 0 || cols % 32 != 0) return MXQ_ERR_SHAPE;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!q4 || !s4 || !q8 || !s8) return MXQ_ERR_NULL;
    if (!aligned16(q4) || !aligned16(q8)) return MXQ_ERR_ALIGN;
    if (((rows + 127) / 128) * ((cols + 255) / 256) > MAX_GRID_X) return MXQ_ERR_SHAPE;  // one block per tile
    return hip_status(mxq::launch_fp4_row_to_fp8_col(q4, s4, rows, cols, q8, s8, as_stream(stream)));
}

int mxq_swiglu_quantize_mx(const void* gu, int src, int64_t rows, int64_t inter, int64_t ld, int fmt, uint8_t* q,
                           uint8_t* s, void* stream) {
    if (src != MXQ_SRC_F32 && src != MXQ_SRC_BF16) return MXQ_ERR_FORMAT;
    if (fmt != MXQ_E4M3 && fmt != MXQ_E5M2) return MXQ_ERR_FORMAT;
    if (rows < 0 || inter < 0) return MXQ_ERR_SHAPE;
    if (inter % 32 != 0 || ld < 2 * inter) return MXQ_ERR_SHAPE;
    if (rows == 0 || inter == 0) return MXQ_OK;
    if (!gu || !q || !s) return MXQ_ERR_NULL;
    if (rows * (inter / 8) / 512 + 1 > MAX_GRID_X) return MXQ_ERR_SHAPE;  // 512 vectors per block
    const int64_t esz = src == MXQ_SRC_BF16 ? 2 : 4;
    if (!aligned16(gu) || (ld * esz) % 16 != 0 || !aligned16(q)) return MXQ_ERR_ALIGN;
    return hip_status(mxq::launch_swiglu_quantize_mx(gu, src, rows, inter, ld, fmt, q, s, as_stream(stream)));
}

// The GEMM kernel addresses each operand (per group) and its scale array
// with 32-bit byte offsets.
static bool below_4gib(int64_t rows, int64_t K, int fmt, int mode) {
    const int64_t lim = (int64_t)1 << 32;
    const int64_t ld = fmt == MXQ_E2M1 ? K / 2 : K;
    if (rows > 0 && ld > (lim - 1) / rows) return false;
    return mode == MXQ_SCALE_TENSOR || rows * (K / 32) < lim;
}

// Formats, modes and K: checked for every call, zero-size ones included.
static int check_formats(int fa, int ma, int fb, int mb, int64_t K, int out) {
    if (!valid_fmt(fa) || !valid_fmt(fb) || !valid_mode(ma) || !valid_mode(mb)) return MXQ_ERR_FORMAT;
    const int kind = out & ~MXQ_OUT_PRECISE;
    if (kind != MXQ_OUT_F32 && kind != MXQ_OUT_BF16) return MXQ_ERR_FORMAT;
    // the precise mode takes FP8 x FP8 (E2M1 x E2M1 is exact natively); mixed FP8 x FP4 is refused
    if ((out & MXQ_OUT_PRECISE) && ((fa == MXQ_E2M1) != (fb == MXQ_E2M1))) return MXQ_ERR_FORMAT;
    if (K <= 0 || K % 128 != 0) return MXQ_ERR_SHAPE;
    return MXQ_OK;
}

// Operand pointers: checked once the problem is known to be non-empty.
static int check_pointers(const uint8_t* A, const void* sA, const uint8_t* B, const void* sB, void* C) {
    if (!A || !B || !sA || !sB || !C) return MXQ_ERR_NULL;
    if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return MXQ_ERR_ALIGN;
    if (!aligned4(sA) || !aligned4(sB)) return MXQ_ERR_ALIGN;
    return MXQ_OK;
}

int mxq_scaled_gemm(const uint8_t* A, int fa, const void* sA, int ma, const uint8_t* B, int fb, const void* sB,
                    int mb, int64_t M, int64_t N, int64_t K, void* C, int out, int64_t ldc, void* stream) {
    if (M < 0 || N < 0) return MXQ_ERR_SHAPE;
    int st = check_formats(fa, ma, fb, mb, K, out);
    if (st != MXQ_OK) return st;
    if (ldc < N) return MXQ_ERR_SHAPE;
    if ((ldc * ((out & ~MXQ_OUT_PRECISE) == MXQ_OUT_F32 ? 4 : 2)) % 16 != 0) return MXQ_ERR_ALIGN;
    if (M == 0 || N == 0) return MXQ_OK;
    st = check_pointers(A, sA, B, sB, C);
    if (st != MXQ_OK) return st;
    if (((M + 127) / 128) * ((N + 127) / 128) > MAX_GRID_X) return MXQ_ERR_SHAPE;
    if (!below_4gib(M, K, fa, ma) || !below_4gib(N, K, fb, mb)) return MXQ_ERR_SHAPE;
    mxq::GemmArgs a{};
    a.A = A; a.sA = sA; a.B = B; a.sB = sB; a.C = C;
    a.group_off = nullptr; a.G = 0;
    a.M = M; a.N = N; a.K = K; a.ldc = ldc;
    a.fa = fa; a.fb = fb; a.ma = ma; a.mb = mb; a.out = out & ~MXQ_OUT_PRECISE;
    a.precise = (out & MXQ_OUT_PRECISE) && fa != MXQ_E2M1;
    return hip_status(mxq::launch_scaled_gemm(a, as_stream(stream)));
}

int mxq_grouped_scaled_gemm(const uint8_t* A, int fa, const void* sA, int ma, const uint8_t* B, int fb,
                            const void* sB, int mb, const int64_t* group_off, int64_t G, int64_t total_rows,
                            int64_t N, int64_t K, void* C, int out, void* stream) {
    if (G < 0 || G > 4096 || total_rows < 0 || N < 0) return MXQ_ERR_SHAPE;
    int st = check_formats(fa, ma, fb, mb, K, out);
    if (st != MXQ_OK) return st;
    if ((N * ((out & ~MXQ_OUT_PRECISE) == MXQ_OUT_F32 ? 4 : 2)) % 16 != 0) return MXQ_ERR_ALIGN;
    if (G == 0 || total_rows == 0 || N == 0) return MXQ_OK;
    st = check_pointers(A, sA, B, sB, C);
    if (st != MXQ_OK) return st;
    if (!group_off) return MXQ_ERR_NULL;
    if (!aligned4(group_off)) return MXQ_ERR_ALIGN;
    if (((total_rows + 127) / 128 + G + 7) * ((N + 127) / 128) > MAX_GRID_X) return MXQ_ERR_SHAPE;
    if (!below_4gib(total_rows, K, fa, ma) || !below_4gib(N, K, fb, mb)) return MXQ_ERR_SHAPE;
    mxq::GemmArgs a{};
    a.A = A; a.sA = sA; a.B = B; a.sB = sB; a.C = C;
    a.group_off = group_off; a.G = G;
    a.M = total_rows; a.N = N; a.K = K; a.ldc = N;
    a.b_group_stride = N * (fb == MXQ_E2M1 ? K / 2 : K);
    a.sb_group_stride = mb == MXQ_SCALE_BLK32 ? N * (K / 32) : (mb == MXQ_SCALE_BLK128 ? N * (K / 128) : 0);
    a.fa = fa; a.fb = fb; a.ma = ma; a.mb = mb; a.out = out & ~MXQ_OUT_PRECISE;
    a.precise = (out & MXQ_OUT_PRECISE) && fa != MXQ_E2M1;
    return hip_status(mxq::launch_scaled_gemm(a, as_stream(stream)));
}

int mxq_grouped_gemm_swiglu_quantize_mx(const uint8_t* A, int fa, const void* sA, int ma, const uint8_t* B, int fb,
                                        const void* sB, int mb, const int64_t* group_off, int64_t G,
                                        int64_t total_rows, int64_t inter, int64_t K, int hfmt, uint8_t* q_out,
                                        uint8_t* s_out, void* stream) {
    if (G < 0 || G > 4096 || total_rows < 0 || inter < 0) return MXQ_ERR_SHAPE;
    if (fa == MXQ_E2M1 || fb == MXQ_E2M1) return MXQ_ERR_FORMAT;
    if (hfmt != MXQ_E4M3 && hfmt != MXQ_E5M2) return MXQ_ERR_FORMAT;
    // the operand checks of the plain GEMM, with q_out in the place of C
    int st = check_formats(fa, ma, fb, mb, K, MXQ_OUT_F32);
    if (st != MXQ_OK) return st;
    if (inter % 128 != 0) return MXQ_ERR_SHAPE;
    if (G == 0 || total_rows == 0 || inter == 0) return MXQ_OK;
    st = check_pointers(A, sA, B, sB, q_out);
    if (st != MXQ_OK) return st;
    if (!group_off || !s_out) return MXQ_ERR_NULL;
    if (!aligned4(group_off)) return MXQ_ERR_ALIGN;
    const int64_t N = 2 * inter;
    if (((total_rows + 127) / 128 + G + 7) * ((N + 127) / 128) > MAX_GRID_X) return MXQ_ERR_SHAPE;
    if (!below_4gib(total_rows, K, fa, ma) || !below_4gib(N, K, fb, mb)) return MXQ_ERR_SHAPE;
    mxq::GemmArgs a{};
    a.A = A; a.sA = sA; a.B = B; a.sB = sB; a.C = nullptr;
    a.group_off = group_off; a.G = G;
    a.M = total_rows; a.N = N; a.K = K; a.ldc = N;
    a.b_group_stride = N * K;
    a.sb_group_stride = mb == MXQ_SCALE_BLK32 ? N * (K / 32) : (mb == MXQ_SCALE_BLK128 ? N * (K / 128) : 0);
    a.fa = fa; a.fb = fb; a.ma = ma; a.mb = mb; a.out = MXQ_OUT_F32;
    a.swiglu = 1; a.hfmt = hfmt; a.inter = inter; a.q_out = q_out; a.s_out = s_out;
    return hip_status(mxq::launch_grouped_swiglu(a, as_stream(stream)));
}

}  // extern "C"
