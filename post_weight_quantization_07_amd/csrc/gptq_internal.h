// Host-side interfaces between the C ABI (abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gptq {

// ---------------------------------------------------------------- hessian --
struct HessPlan {
  int tile;          // output tile edge
  int stage_tokens;  // tokens per LDS stage
  int nt;            // tiles per edge
  int n_tiles;       // upper-triangular tiles
  int n_split;       // token slices
  int64_t split_len; // tokens per slice (multiple of stage_tokens)
  size_t partial_bytes;
  size_t ws_bytes;
};
HessPlan hessian_plan(int64_t d_in, int64_t n_tokens, bool bf16, int n_cu);
hipError_t hessian_launch(const HessPlan& plan, float* S, int64_t d_in, const void* X, bool bf16,
                          int64_t n_tokens, int64_t ldx, void* ws, hipStream_t stream);

// ---------------------------------------------------------------- prepare --
constexpr int kPanel = 128;  // Cholesky panel / diagonal block width

struct PrepLayout {
  size_t off_hr, off_t, off_diag, off_lambda, ws_bytes;
};
PrepLayout prepare_layout(int64_t d_in);
hipError_t prepare_launch(float* S_to_H, int64_t d_in, int64_t n_total, float damp, bool desc_act,
                          float* U, int32_t* perm, int32_t* info, void* ws, hipStream_t stream);

// ------------------------------------------------------------------- gemm --
// C[M,N] = alpha * op(A)[M,K] * op(B)[K,N] + beta * C, row-major fp32 on MFMA.
// transB: B is given as [N, K] row-major.  lower_tiles: only compute tiles whose
// first row >= first column (block-lower part; used by the Cholesky update).
// tri: 0 dense; 1 B is lower-triangular (a tile skips k < its first column);
// 2 A is lower-triangular (a tile skips k past its last row).
// Batched over blockIdx.z with element strides sA, sB, sC.
hipError_t gemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const float* A, int64_t lda,
                    int64_t sA, const float* B, int64_t ldb, int64_t sB, bool transB, float beta,
                    float* C, int64_t ldc, int64_t sC, int batch, bool lower_tiles, int tri,
                    hipStream_t stream);

// --------------------------------------------------------------- quantize --
struct QuantLayout {
  size_t off_wp, off_err, ws_bytes;
};
QuantLayout quant_layout(int64_t d_out, int64_t d_in);
hipError_t quantize_launch(const void* W, bool w_bf16, int64_t d_out, int64_t d_in, const float* U,
                           const int32_t* perm, int bits, int group_size, bool sym, bool static_groups,
                           uint8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx, float* Q,
                           float* row_loss, void* ws, hipStream_t stream, bool identity);

// ------------------------------------------------------------------- pack --
hipError_t pack_launch(const uint8_t* codes, int64_t d_out, int64_t d_in, int bits, int32_t* qweight,
                       hipStream_t stream);

// ---------------------------------------------------------------- dequant --
size_t dequant_workspace_bytes(int64_t m, int64_t d_in, int64_t d_out);
hipError_t dequant_matmul_launch(const void* x, bool x_bf16, int64_t m, int64_t d_in, const int32_t* qweight,
                                 const float* scales, const int32_t* zeros, const int32_t* g_idx, int bits,
                                 int64_t d_out, int n_groups, float* y, void* ws, hipStream_t stream);
hipError_t dequant_order_launch(const int32_t* qweight, const int32_t* g_idx, int bits, int64_t d_in, int64_t d_out,
                                int32_t* qweight_out, int32_t* g_idx_out, int32_t* order, hipStream_t stream);
size_t dequant_ordered_workspace_bytes(int64_t m, int64_t d_in, int64_t d_out);
hipError_t dequant_matmul_ordered_launch(const void* x, bool x_bf16, int64_t m, int64_t d_in, const int32_t* qweight,
                                         const float* scales, const int32_t* zeros, const int32_t* g_idx,
                                         const int32_t* order, int bits, int64_t d_out, int n_groups, float* y,
                                         void* ws, hipStream_t stream);

}  // namespace gptq
