// fp32 GEMM on gfx950 matrix cores (v_mfma_f32_16x16x4_f32).
//
// C[M,N] = alpha * A[M,K] * op(B)[K,N] + beta * C, all row-major.  op(B) is B
// ([K,N]) or, with transB, the transpose of a [N,K] matrix.  Used by the
// Cholesky trailing update, the triangular inverse and the GPTQ lazy-batch
// update W[:, j+B:] -= Err * U[j:j+B, j+B:] (GPTQ 实战 ch.5, section 5.1.8).
//
// 64x64 output tile per 256-thread workgroup, 2x2 waves of 32x32, k-stage of
// 16.  LDS holds both operands k-major ([k][m] and [k][n]); rows are padded to
// 80 floats so the four k-rows one MFMA operand load touches fall in distinct
// bank groups, and each wave's transposing stores cover 64 consecutive rows;
// stages are double-buffered with the next stage's global loads in registers.
// Requirements (checked by the callers): K, N, lda, ldb, ldc multiples of 4 and
// 16-byte aligned base pointers; M arbitrary.
#include "gptq_common.h"
#include "gptq_internal.h"

namespace gptq {
namespace {

constexpr int kBM = 64, kBN = 64, kBK = 16, kPitch = 80;

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

template <bool TRANS_B>
__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) float As[2][kBK * kPitch];
  __shared__ __attribute__((aligned(16))) float Bs[2][kBK * kPitch];
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kBN;
  if (m0 >= p.M) return;
  if (p.lower_tiles && n0 > m0 + kBM - 1) return;
  const float* A = p.A + blockIdx.z * p.sA;
  const float* B = p.B + blockIdx.z * p.sB;
  float* C = p.C + blockIdx.z * p.sC;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // loader coordinates: A (and transposed B) read float4 along k: row = lane, k-quad = wave
  const int ar = tid & 63, akq = tid >> 6;
  // non-transposed B reads float4 along n: k-row tid/16, n-quad tid%16
  const int bk = tid >> 4, bnq = tid & 15;

  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto load_a = [&](int64_t k0) {
    const int64_t m = m0 + ar, k = k0 + 4 * akq;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (m < p.M && k < p.K) v = *reinterpret_cast<const f32x4_t*>(A + m * p.lda + k);
    return v;
  };
  auto load_b = [&](int64_t k0) {
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (TRANS_B) {
      const int64_t n = n0 + ar, k = k0 + 4 * akq;
      if (n < p.N && k < p.K) v = *reinterpret_cast<const f32x4_t*>(B + n * p.ldb + k);
    } else {
      const int64_t k = k0 + bk, n = n0 + 4 * bnq;
      if (k < p.K && n < p.N) v = *reinterpret_cast<const f32x4_t*>(B + k * p.ldb + n);
    }
    return v;
  };
  auto store_a = [&](float* s, const f32x4_t& v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) s[(4 * akq + e) * kPitch + ar] = v[e];
  };
  auto store_b = [&](float* s, const f32x4_t& v) {
    if (TRANS_B) {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[(4 * akq + e) * kPitch + ar] = v[e];
    } else {
      *reinterpret_cast<f32x4_t*>(s + bk * kPitch + 4 * bnq) = v;
    }
  };

  const int nstage = static_cast<int>((p.K + kBK - 1) / kBK);
  f32x4_t ra = load_a(0), rb = load_b(0);
  store_a(As[0], ra);
  store_b(Bs[0], rb);
  __syncthreads();
  for (int s = 0; s < nstage; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nstage;
    if (more) {
      ra = load_a(static_cast<int64_t>(s + 1) * kBK);
      rb = load_b(static_cast<int64_t>(s + 1) * kBK);
    }
    const float* as = As[cur];
    const float* bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 4) {
      const int kr = kk + (lane >> 4);
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = as[kr * kPitch + wm * 32 + 16 * i + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = bs[kr * kPitch + wn * 32 + 16 * j + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_a(As[cur ^ 1], ra);
      store_b(Bs[cur ^ 1], rb);
    }
    __syncthreads();
  }
  // epilogue: element (i, j, r) -> row wm*32 + 16 i + 4 (lane >> 4) + r, col wn*32 + 16 j + (lane & 15)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + wn * 32 + 16 * j + (lane & 15);
      if (n >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + wm * 32 + 16 * i + 4 * (lane >> 4) + r;
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
  dim3 grid(static_cast<unsigned>((N + kBN - 1) / kBN), static_cast<unsigned>((M + kBM - 1) / kBM),
            static_cast<unsigned>(batch));
  if (transB)
    gemm_f32_kernel<true><<<grid, 256, 0, stream>>>(p);
  else
    gemm_f32_kernel<false><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace gptq
