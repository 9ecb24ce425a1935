// fp32 GEMM on gfx950 matrix cores (v_mfma_f32_16x16x4_f32).
//
// C[M,N] = alpha * A[M,K] * op(B)[K,N] + beta * C, all row-major.  op(B) is B
// ([K,N]) or, with transB, the transpose of a [N,K] matrix.  Used by the
// Cholesky trailing update, the triangular inverse and the GPTQ lazy-batch
// update W[:, j+B:] -= Err * U[j:j+B, j+B:] (GPTQ 实战 ch.5, section 5.1.8).
//
// 64x64 or 128x128 output tile per 256-thread workgroup (2x2 waves), k-stage
// of 16.  LDS holds both operands k-major ([k][m] and [k][n]); stages are
// double-buffered with the next stage's global loads in registers.
// Requirements (checked by the callers): K, N, lda, ldb, ldc multiples of 4 and
// 16-byte aligned base pointers; M arbitrary.
#include "gptq_common.h"
#include "gptq_internal.h"

namespace gptq {
namespace {

constexpr int kBK = 16;

struct GemmParams {
  int64_t M, N, K;
  float alpha, beta;
  const float* A;
  int64_t lda, sA;
  const float* B;
  int64_t ldb, sB;
  float* C;
  int64_t ldc, sC;
  int lower_tiles;
};

// BM x BN output tile, 2x2 waves of (BM/2) x (BN/2), MFMA 16x16x4.  LDS rows
// hold BM (or BN) floats plus 16 of padding, so the four k-rows one operand
// load touches fall in distinct bank groups.
template <bool TRANS_B, int BM, int BN>
__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(GemmParams p) {
  constexpr int PA = BM + 16, PB = BN + 16;
  constexpr int NI = BM / 32, NJ = BN / 32;       // 16x16 tiles per wave
  constexpr int LA = BM * kBK / 4 / 256;           // float4 loads per thread (A)
  constexpr int LB = BN * kBK / 4 / 256;           // float4 loads per thread (B)
  __shared__ __attribute__((aligned(16))) float As[2][kBK * PA];
  __shared__ __attribute__((aligned(16))) float Bs[2][kBK * PB];
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * BN;
  if (m0 >= p.M) return;
  if (p.lower_tiles && n0 > m0 + BM - 1) return;
  const float* A = p.A + blockIdx.z * p.sA;
  const float* B = p.B + blockIdx.z * p.sB;
  float* C = p.C + blockIdx.z * p.sC;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x4_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // k-major sources (A, transposed B): float4 along k, row = tid % R, k-quad by tid / R
  auto load_kmajor = [&](const float* src, int64_t ld, int64_t rows, int64_t r0, int64_t k0, int R, int u) {
    const int r = tid % R, kq = tid / R + (256 / R) * u;
    const int64_t gr = r0 + r, gk = k0 + 4 * kq;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (gr < rows && gk < p.K) v = *reinterpret_cast<const f32x4_t*>(src + gr * ld + gk);
    return v;
  };
  auto store_kmajor = [&](float* dst, int pitch, int R, int u, const f32x4_t& v) {
    const int r = tid % R, kq = tid / R + (256 / R) * u;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[(4 * kq + e) * pitch + r] = v[e];
  };
  // row-major B [K, N]: float4 along n
  auto load_b_rows = [&](int64_t k0, int u) {
    constexpr int Q = BN / 4;
    const int nq = tid % Q, kr = tid / Q + (256 / Q) * u;
    const int64_t gk = k0 + kr, gn = n0 + 4 * nq;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (gk < p.K && gn < p.N) v = *reinterpret_cast<const f32x4_t*>(B + gk * p.ldb + gn);
    return v;
  };
  auto store_b_rows = [&](float* dst, int u, const f32x4_t& v) {
    constexpr int Q = BN / 4;
    const int nq = tid % Q, kr = tid / Q + (256 / Q) * u;
    *reinterpret_cast<f32x4_t*>(dst + kr * PB + 4 * nq) = v;
  };

  f32x4_t ra[LA], rb[LB];
  auto load_stage = [&](int64_t k0) {
#pragma unroll
    for (int u = 0; u < LA; ++u) ra[u] = load_kmajor(A, p.lda, p.M, m0, k0, BM, u);
#pragma unroll
    for (int u = 0; u < LB; ++u) rb[u] = TRANS_B ? load_kmajor(B, p.ldb, p.N, n0, k0, BN, u) : load_b_rows(k0, u);
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < LA; ++u) store_kmajor(As[buf], PA, BM, u, ra[u]);
#pragma unroll
    for (int u = 0; u < LB; ++u) {
      if (TRANS_B)
        store_kmajor(Bs[buf], PB, BN, u, rb[u]);
      else
        store_b_rows(Bs[buf], u, rb[u]);
    }
  };

  const int nstage = static_cast<int>((p.K + kBK - 1) / kBK);
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int s = 0; s < nstage; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nstage;
    if (more) load_stage(static_cast<int64_t>(s + 1) * kBK);
    const float* as = As[cur];
    const float* bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 4) {
      const int kr = kk + (lane >> 4);
      float a[NI], b[NJ];
#pragma unroll
      for (int i = 0; i < NI; ++i) a[i] = as[kr * PA + wm * (BM / 2) + 16 * i + (lane & 15)];
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[j] = bs[kr * PB + wn * (BN / 2) + 16 * j + (lane & 15)];
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) store_stage(cur ^ 1);
    __syncthreads();
  }
  // epilogue: element (i, j, r) -> row 16 i + 4 (lane >> 4) + r, col 16 j + (lane & 15) of the wave block
#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t n = n0 + wn * (BN / 2) + 16 * j + (lane & 15);
      if (n >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * (BM / 2) + 16 * i + 4 * (lane >> 4) + r;
        if (m < p.M) {
          float* c = C + m * p.ldc + n;
          const float v = p.alpha * acc[i][j][r];
          *c = (p.beta == 0.f) ? v : v + p.beta * *c;
        }
      }
    }
  }
}

}  // namespace

hipError_t gemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const float* A, int64_t lda,
                    int64_t sA, const float* B, int64_t ldb, int64_t sB, bool transB, float beta,
                    float* C, int64_t ldc, int64_t sC, int batch, bool lower_tiles, bool /*wide_n*/,
                    hipStream_t stream) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  GemmParams p{M, N, K, alpha, beta, A, lda, sA, B, ldb, sB, C, ldc, sC, lower_tiles ? 1 : 0};
  // 64x64 tiles: measured faster than 128x128 on every shape this library
  // issues (more resident workgroups hide the global-load latency better).
  // Lower-tile problems need tiles aligned with their 64-column diagonal blocks.
  const bool big = false;
  if (big) {
    dim3 grid(static_cast<unsigned>((N + 127) / 128), static_cast<unsigned>((M + 127) / 128), static_cast<unsigned>(batch));
    if (transB)
      gemm_f32_kernel<true, 128, 128><<<grid, 256, 0, stream>>>(p);
    else
      gemm_f32_kernel<false, 128, 128><<<grid, 256, 0, stream>>>(p);
  } else {
    dim3 grid(static_cast<unsigned>((N + 63) / 64), static_cast<unsigned>((M + 63) / 64), static_cast<unsigned>(batch));
    if (transB)
      gemm_f32_kernel<true, 64, 64><<<grid, 256, 0, stream>>>(p);
    else
      gemm_f32_kernel<false, 64, 64><<<grid, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace gptq
