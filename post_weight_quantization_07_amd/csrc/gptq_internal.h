// Host-side interfaces between the C ABI (abi.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gptq {

// ---------------------------------------------------------- phase timing --
// A measurement aid (phase_timing.cpp): while switched on, each instrumented
// launch records a HIP event before and after itself on its stream.
enum Phase {
  kPhHessian = 0, kPhHessReduce, kPhPrepElem, kPhPanel, kPhCholUpdate, kPhTrtri,
  kPhQuantElem, kPhSweep, kPhUpdate, kPhPack, kNumPhases
};
bool phase_timing_on();
void phase_mark(int phase, bool begin, hipStream_t st);
hipError_t phase_timing_set(bool on);
hipError_t phase_timing_read(float* ms, int32_t* launches, int n);
const char* phase_name(int phase);
struct PhaseScope {
  int phase;
  hipStream_t st;
  PhaseScope(int p, hipStream_t s) : phase(p), st(s) { phase_mark(p, true, s); }
  ~PhaseScope() { phase_mark(phase, false, st); }
  PhaseScope(const PhaseScope&) = delete;
  PhaseScope& operator=(const PhaseScope&) = delete;
};

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
  bool planes;       // fp32 X as three bf16 planes on the bf16 matrix cores
  int64_t chunk;     // planes: tokens split per pass
  size_t planes_off; // planes: offset of the plane buffer in the workspace
};
HessPlan hessian_plan(int64_t d_in, int64_t n_tokens, bool bf16, int n_cu);
hipError_t hessian_launch(const HessPlan& plan, float* S, int64_t d_in, const void* X, bool bf16,
                          int64_t n_tokens, int64_t ldx, void* ws, hipStream_t stream);

// ---------------------------------------------------------------- prepare --
constexpr int kPanel = 128;  // Cholesky panel / diagonal block width

struct PrepLayout {
  size_t off_hr, off_t, off_diag, off_dinv, off_lambda, off_p, off_qa, off_qb, ws_bytes;
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

// fp32 product on the bf16 matrix cores (gemm_x3.hip): C[M,N] += alpha * A B
// with A given as three bf16 planes over [M][K] (plane stride sA) and B as
// three planes of its transpose over [N][K] (plane stride sB), each the exact
// split x = hi + mid + lo of the fp32 values; six part products.  Planes use
// the blocked panel layout below (rows padded to 128, K multiple of 16).
// split3_t writes the planes of the transpose of a row-major fp32 block
// src[K][N] (row stride ld), plane stride x3_plane_elems(N, K).
//
// Blocked panel layout: element (r, k) of a plane of K columns sits at
// x3_offset(r, k, K): blocks of 128 rows x 16 k, 4 KB contiguous, row-major
// inside a block, blocks ordered by row block, then k block.
__host__ __device__ inline int64_t x3_offset(int64_t r, int64_t k, int64_t K) {
  return ((r >> 7) * (K >> 4) + (k >> 4)) * 2048 + (r & 127) * 16 + (k & 15);
}
__host__ __device__ inline int64_t x3_plane_elems(int64_t rows, int64_t K) { return ((rows + 127) >> 7) * 128 * K; }
// ldk: width of the planes' layout when the product uses only their first K
// columns (0: K).  lower: square C, only tiles on or below the diagonal, and
// nothing written above the 64-block diagonal (the Cholesky update).
// tri: 1 B lower-triangular (each tile skips k below its first column), 2 A
// lower-triangular (each tile skips k past its last row); K a multiple of 64
// and the zero parts of the 64- or 128-tiles on the diagonal stored as zeros.
// beta0: C = alpha A B without reading C.  batch: blockIdx.y, with element
// strides bA, bB (of the planes) and bC.
hipError_t gemm_x3(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t* A, int64_t sA, const uint16_t* Bt,
                   int64_t sB, float* C, int64_t ldc, hipStream_t stream, int64_t ldk = 0, bool lower = false,
                   int tri = 0, bool beta0 = false, int batch = 1, int64_t bA = 0, int64_t bB = 0, int64_t bC = 0);
hipError_t split3_t(const float* src, int64_t ld, int64_t K, int64_t N, uint16_t* out, hipStream_t stream,
                    int batch = 1, int64_t bsrc = 0, int64_t bout = 0);
// split3_rows writes the planes of a row-major block src[R][K] itself (no
// transpose), plane stride x3_plane_elems(R, K).
hipError_t split3_rows(const float* src, int64_t ld, int64_t R, int64_t K, uint16_t* out, hipStream_t stream,
                       int batch = 1, int64_t bsrc = 0, int64_t bout = 0);

// --------------------------------------------------------------- quantize --
struct QuantLayout {
  size_t off_wp, off_err, ws_bytes;
  size_t off_ea, off_bt;  // one launch per group: error planes, transposed U planes
};
// one sweep launch per group of columns: groups inside a block or parameters
// fixed before the sweep
bool group_launch(int group_size, bool static_groups);
// groups of 1024 columns, whose products past the group run on the bf16
// matrix cores (error and U planes in the workspace)
bool quant_planes(int group_size, bool static_groups);
QuantLayout quant_layout(int64_t d_out, int64_t d_in, bool planes);
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
// bytes of partial sums one call of the product writes (0: a single K slice)
size_t dequant_partial_bytes(int64_t m, int64_t d_in, int64_t d_out, bool x_bf16, int bits);
// the library's fixed scratch buffer (device address of the current device's copy)
constexpr size_t kDequantScratchBytes = size_t{16} << 20;
hipError_t dequant_scratch(void** out);
hipError_t dequant_matmul_ordered_launch(const void* x, bool x_bf16, int64_t m, int64_t d_in, const int32_t* qweight,
                                         const float* scales, const int32_t* zeros, const int32_t* g_idx,
                                         const int32_t* order, int bits, int64_t d_out, int n_groups, float* y,
                                         void* ws, hipStream_t stream);

}  // namespace gptq
