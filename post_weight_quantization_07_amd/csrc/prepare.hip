// Hessian finalisation, damping, act-order and the inverse factor U.
//
// GPTQ 实战 ch.5, section 5.1.8: damp H by lambda * mean(diag H) * I, then
// take "Cholesky(inverse(H))" once; its rows are the compensation
// coefficients of the column sweep.  desc_act (AutoGPTQ examples walkthrough,
// section 1.4) orders the columns by descending diag(H).
//
// Route on the GPU.  With J the index reversal, H_p = U^-1 U^-T for the
// upper-triangular U with H_p^-1 = U^T U, hence J U^-1 J is the lower Cholesky
// factor of J H_p J.  So
//     U = J * chol_lower(J H_p J)^-1 * J,
// one Cholesky and one triangular inverse, no explicit inverse of H.  The
// reversal and the act-order permutation are folded into one gather.
//
//   finalize   H = (2/N) S in place, diag(H) saved
//   lambda     lambda = damp * mean(diag H)              (one workgroup, fixed order)
//   order      perm by rank of -diag(H), ties by index   (stable sort by counting)
//   gather     Hr[a][b] = H[p(a)][p(b)] + lambda d_ab, p(a) = perm[n-1-a], lower part
//   panels     right-looking blocked Cholesky of Hr, 64-column panels:
//                panel kernel: factor the 64x64 diagonal block (one wave, rows in
//                registers), then solve the panel rows below against it;
//                trailing update Hr[k+64:, k+64:] -= P P^T on MFMA (lower tiles)
//   diag inv   invert every 64x64 diagonal block of the factor in place
//   trtri      recursive doubling: for neighbouring inverted blocks A^-1, C^-1
//              and the factor block L21 below A, M21 = -C^-1 (L21 A^-1)
//   reverse    U[i][j] = M[n-1-i][n-1-j] for j >= i, 0 below the diagonal
#include "gptq_common.h"
#include "gptq_internal.h"

#include <algorithm>

namespace gptq {
namespace {

constexpr int kNB = kPanel;  // 64

__global__ void finalize_kernel(float* S, int64_t n, float scale, float* diag) {
  const int64_t total = n * n;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float v = S[e] * scale;
    S[e] = v;
    const int64_t r = e / n;
    if (r * n + r == e) diag[r] = v;
  }
}

// lambda = damp * mean(diag): fixed-order tree over 1024 threads.
__global__ __launch_bounds__(1024) void lambda_kernel(const float* diag, int64_t n, float damp,
                                                      float* lambda_out, int32_t* info) {
  __shared__ double part[1024];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) s += static_cast<double>(diag[i]);
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    lambda_out[0] = damp * static_cast<float>(part[0] / static_cast<double>(n));
    info[0] = 0;
  }
}

// perm[rank(i)] = i with rank(i) = #{j : d_j > d_i} + #{j < i : d_j == d_i}.
__global__ __launch_bounds__(256) void order_kernel(const float* diag, int64_t n, int desc_act,
                                                    int32_t* perm) {
  __shared__ float tile[1024];
  const int64_t i = blockIdx.x * 256 + threadIdx.x;
  if (!desc_act) {
    if (i < n) perm[i] = static_cast<int32_t>(i);
    return;
  }
  const float di = (i < n) ? diag[i] : 0.f;
  int64_t rank = 0;
  for (int64_t base = 0; base < n; base += 1024) {
    __syncthreads();
    for (int t = threadIdx.x; t < 1024; t += 256) tile[t] = (base + t < n) ? diag[base + t] : 0.f;
    __syncthreads();
    const int lim = static_cast<int>(std::min<int64_t>(1024, n - base));
    for (int t = 0; t < lim; ++t) {
      const float dj = tile[t];
      rank += (dj > di) || (dj == di && base + t < i);
    }
  }
  if (i < n) perm[rank] = static_cast<int32_t>(i);
}

// Hr[a][b] = H[p(a)][p(b)] (+ lambda on the diagonal) for b <= a, 0 above.
__global__ void gather_kernel(const float* H, int64_t n, const int32_t* perm, const float* lambda,
                              float* Hr) {
  const float lam = lambda[0];
  const int64_t total = n * n;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t a = e / n, b = e - a * n;
    float v = 0.f;
    if (b <= a) {
      const int64_t pa = perm[n - 1 - a], pb = perm[n - 1 - b];
      v = H[pa * n + pb];
      if (a == b) v += lam;
    }
    Hr[e] = v;
  }
}

// Lower Cholesky of the 64x64 block held in L (LDS, pitch 68), blocked by 16
// columns.  Sub-panel b (columns 16 b .. 16 b + 15, all rows) is factored by
// one wave, lane r holding row r's 16 entries in registers; the rank-16 update
// of the lower 16x16 blocks to its right then runs on MFMA, spread over the
// workgroup's four waves.
//
// Sub-panel factor: right-looking, pipelined by one step: at step j column j
// is complete; the step's update of column j + 1 is applied at once (the next
// pivot depends on it, and l[j+1] comes by readlane), and its updates of the
// sub-panel's later columns are applied during step j + 1 from the column
// published in LDS one step earlier, so the LDS round trip overlaps the pivot
// chain.  Every lane scales its column-j entry by 1 / sqrt(pivot): lanes above
// the pivot only ever touch their own upper-triangle entries, which are
// discarded (each sub-panel is written back with zeros above the diagonal,
// also to LTq, the transposed layout of the row solve).  `fail` receives the
// first pivot that is not positive.
template <int b>
GPTQ_DEV void factor_subpanel(float (*L)[68], float (*LTq)[4][16], f32x4_t (*colbuf)[kNB / 4], int lane,
                              int& fail) {
  constexpr int c0 = 16 * b;
  float v[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) v[c] = L[lane][c0 + c];
  float lp = 0.f;
  f32x4_t xp[4], xn[4];  // published column of the previous / current step (sub-panel window)
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const int j = c0 + jj;
    const float piv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[jj]), j));
    if (!(piv > 0.f) && fail < 0) fail = j;
    // hardware square root and reciprocal (about 1 ulp): the pivot chain is the
    // latency-critical path of the factorization
    const float inv = __builtin_amdgcn_rcpf(__builtin_amdgcn_sqrtf(piv));
    const float l = v[jj] * inv;
    v[jj] = l;
    reinterpret_cast<float*>(colbuf[jj & 1])[lane] = l;
    // keep the publication above the reads of this buffer
    asm volatile("" ::: "memory");
    // read the column back now for the next step's update of columns j + 2 ..
#pragma unroll
    for (int q = (jj + 2) >> 2; q < 4; ++q) xn[q] = colbuf[jj & 1][c0 / 4 + q];
    if (jj + 1 < 16) {
      const float lj1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), j + 1));
      v[jj + 1] = fmaf(-l, lj1, v[jj + 1]);
    }
    if (jj >= 1) {
#pragma unroll
      for (int q = (jj + 1) >> 2; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * q + e > jj) v[4 * q + e] = fmaf(-lp, xp[q][e], v[4 * q + e]);
    }
    lp = l;
#pragma unroll
    for (int q = 0; q < 4; ++q) xp[q] = xn[q];
  }
  // the sub-panel's columns are final: write them and their transpose for the
  // row solve (LTq[c][q][u] = L[4u+q][c])
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const float x = (c0 + c <= lane) ? v[c] : 0.f;
    L[lane][c0 + c] = x;
    LTq[c0 + c][lane & 3][lane >> 2] = x;
  }
}

// Rank-16 update after sub-panel b: for the lower 16x16 blocks (I, J),
// b < J <= I <= 3, L[I][J] -= P_I P_J^T with P_I = L[16 I .., 16 b ..].
// v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16], B[l / 16][l % 16]
// and holds D[4 (l / 16) + e][l % 16].  Block t goes to wave t % 4.
template <int b>
GPTQ_DEV void trailing_update(float (*L)[68], int wave, int lane) {
  constexpr int n = 3 - b;  // trailing blocks per edge
  const int m = lane & 15, kq = lane >> 4;
  int t = 0;
#pragma unroll
  for (int i = 0; i < n; ++i) {
#pragma unroll
    for (int jb = 0; jb <= i; ++jb, ++t) {
      if (t % 4 != wave) continue;
      const int I = b + 1 + i, J = b + 1 + jb;
      f32x4_t acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = L[16 * I + 4 * kq + e][16 * J + m];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const float a = -L[16 * I + m][16 * b + 4 * tt + kq];
        const float bb = L[16 * J + m][16 * b + 4 * tt + kq];
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) L[16 * I + 4 * kq + e][16 * J + m] = acc[e];
    }
  }
}

// One launch per panel k: every workgroup factors the 64x64 diagonal block
// (the same arithmetic, so the same result), workgroup 0 stores it, and the
// workgroup then solves 64 panel rows x L^T = p against it.  Each row is
// solved by a quad of lanes, lane q holding columns q, q+4, ..., q+60:
// right-looking substitution (once x_c is known, every later column of the row
// is updated at once) keeps the dependent chain at 64 steps, and x_c reaches
// the other three lanes of the quad through a DPP quad broadcast.
constexpr int kPanelRows = 64;

template <int Q>
GPTQ_DEV float quad_bcast(float v) {
  constexpr int sel = Q | (Q << 2) | (Q << 4) | (Q << 6);
  return __builtin_amdgcn_update_dpp(0.0f, v, sel, 0xf, 0xf, false);
}

template <int C>
GPTQ_DEV void solve_step(float (&sv)[16], float (&xv)[16], const float (*LTq)[4][16], const float* dinv, int q) {
  constexpr int owner = C & 3, u = C >> 2;
  const float xc = quad_bcast<owner>(sv[u] * dinv[C]);
  xv[u] = (q == owner) ? xc : xv[u];
  // column C of L for this lane's columns 4 k + q (zeros above the diagonal)
  const f32x4_t* lt = reinterpret_cast<const f32x4_t*>(&LTq[C][q][0]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f32x4_t l4 = lt[w];
#pragma unroll
    for (int e = 0; e < 4; ++e) sv[4 * w + e] = fmaf(-xc, l4[e], sv[4 * w + e]);
  }
}

template <int... Cs>
GPTQ_DEV void solve_all(float (&sv)[16], float (&xv)[16], const float (*LTq)[4][16], const float* dinv, int q,
                        std::integer_sequence<int, Cs...>) {
  (solve_step<Cs>(sv, xv, LTq, dinv, q), ...);
}

__global__ __launch_bounds__(256, 1) void panel_kernel(float* Hr, int64_t n, int64_t k, int32_t* info) {
  __shared__ __attribute__((aligned(16))) float L[kNB][68];
  __shared__ __attribute__((aligned(16))) float LTq[kNB][4][16];  // LTq[c][q][u] = L[4u+q][c]
  __shared__ f32x4_t colbuf[2][kNB / 4];
  __shared__ float dinv[kNB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = static_cast<int>(std::min<int64_t>(kNB, n - k));
  for (int e = tid; e < kNB * kNB; e += 256) {
    const int r = e >> 6, c = e & 63;
    float v = (r == c) ? 1.f : 0.f;
    if (r < nb && c <= r) v = Hr[(k + r) * n + k + c];
    L[r][c] = v;
  }
  // this thread's panel row (quad q holds columns q, q + 4, ..., q + 60):
  // loaded now, so the load overlaps the factorization
  const int q = tid & 3;
  const int64_t row = k + kNB + static_cast<int64_t>(blockIdx.x) * kPanelRows + (tid >> 2);
  const bool solve = (nb == kNB) && (row < n);
  float sv[16], xv[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    sv[u] = solve ? Hr[row * n + k + 4 * u + q] : 0.f;
    xv[u] = 0.f;
  }
  __syncthreads();
  int fail = -1;
  if (wave == 0) factor_subpanel<0>(L, LTq, colbuf, lane, fail);
  __syncthreads();
  trailing_update<0>(L, wave, lane);
  __syncthreads();
  if (wave == 0) factor_subpanel<1>(L, LTq, colbuf, lane, fail);
  __syncthreads();
  trailing_update<1>(L, wave, lane);
  __syncthreads();
  if (wave == 0) factor_subpanel<2>(L, LTq, colbuf, lane, fail);
  __syncthreads();
  trailing_update<2>(L, wave, lane);
  __syncthreads();
  if (wave == 0) {
    factor_subpanel<3>(L, LTq, colbuf, lane, fail);
    if (lane == 0 && blockIdx.x == 0 && fail >= 0 && fail < nb)
      atomicCAS(info, 0, static_cast<int32_t>(n - (k + fail)));
  }
  __syncthreads();
  if (tid < kNB) dinv[tid] = __builtin_amdgcn_rcpf(L[tid][tid]);
  __syncthreads();
  if (solve) {
    solve_all(sv, xv, LTq, dinv, q, std::make_integer_sequence<int, kNB>{});
    float* dst = Hr + row * n + k;
#pragma unroll
    for (int u = 0; u < 16; ++u) dst[4 * u + q] = xv[u];
  }
  // the factored diagonal block (L stays valid in LDS), after the solve so it
  // does not hold up workgroup 0's rows
  if (blockIdx.x == 0) {
    for (int e = tid; e < nb * nb; e += 256) {
      const int r = e / nb, c = e - r * nb;
      Hr[(k + r) * n + k + c] = L[r][c];
    }
  }
}

// Invert every 64x64 diagonal block of the lower factor in place.  Wave 0,
// lane c computes column c of the inverse by forward substitution.
__global__ __launch_bounds__(256) void diag_inverse_kernel(float* Hr, int64_t n) {
  __shared__ __attribute__((aligned(16))) float L[kNB][68];
  const int64_t k = static_cast<int64_t>(blockIdx.x) * kNB;
  const int nb = static_cast<int>(std::min<int64_t>(kNB, n - k));
  const int tid = threadIdx.x, lane = tid & 63;
  for (int e = tid; e < kNB * kNB; e += 256) {
    const int r = e >> 6, c = e & 63;
    float v = (r == c) ? 1.f : 0.f;
    if (r < nb && c <= r) v = Hr[(k + r) * n + k + c];
    L[r][c] = v;
  }
  __syncthreads();
  if (tid >= 64) return;
  float m[kNB];
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    float s = (i == lane) ? 1.f : 0.f;
#pragma unroll
    for (int t = 0; t < i; ++t) s = fmaf(-L[i][t], m[t], s);
    m[i] = (i >= lane) ? s * __builtin_amdgcn_rcpf(L[i][i]) : 0.f;
  }
  for (int i = 0; i < nb; ++i)
    if (lane < nb) Hr[(k + i) * n + k + lane] = m[i];
}

__global__ void reverse_kernel(const float* M, int64_t n, float* U) {
  const int64_t total = n * n;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t i = e / n, j = e - i * n;
    U[e] = (j >= i) ? M[(n - 1 - i) * n + (n - 1 - j)] : 0.f;
  }
}

int grid_for(int64_t total) {
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 8192)));
}

}  // namespace

PrepLayout prepare_layout(int64_t d) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  PrepLayout L{};
  size_t off = 0;
  L.off_hr = off;
  off += up(static_cast<size_t>(d) * d * sizeof(float));
  L.off_t = off;  // trtri scratch: at most d*d/4 floats
  off += up(static_cast<size_t>(d) * d / 4 * sizeof(float) + 64 * 64 * sizeof(float));
  L.off_diag = off;
  off += up(static_cast<size_t>(d) * sizeof(float));
  L.off_lambda = off;
  off += 256;
  L.ws_bytes = off;
  return L;
}


#define GPTQ_TRY(x)                          \
  do {                                       \
    hipError_t e_ = (x);                     \
    if (e_ != hipSuccess) return e_;         \
  } while (0)

hipError_t prepare_launch(float* S, int64_t n, int64_t n_total, float damp, bool desc_act, float* U,
                          int32_t* perm, int32_t* info, void* ws, hipStream_t st) {
  const PrepLayout lay = prepare_layout(n);
  char* w = static_cast<char*>(ws);
  float* Hr = reinterpret_cast<float*>(w + lay.off_hr);
  float* T = reinterpret_cast<float*>(w + lay.off_t);
  float* diag = reinterpret_cast<float*>(w + lay.off_diag);
  float* lam = reinterpret_cast<float*>(w + lay.off_lambda);
  const int64_t nn = n * n;

  finalize_kernel<<<grid_for(nn), 256, 0, st>>>(S, n, static_cast<float>(2.0 / static_cast<double>(n_total)), diag);
  GPTQ_TRY(hipGetLastError());
  lambda_kernel<<<1, 1024, 0, st>>>(diag, n, damp, lam, info);
  GPTQ_TRY(hipGetLastError());
  order_kernel<<<static_cast<int>((n + 255) / 256), 256, 0, st>>>(diag, n, desc_act ? 1 : 0, perm);
  GPTQ_TRY(hipGetLastError());
  gather_kernel<<<grid_for(nn), 256, 0, st>>>(S, n, perm, lam, Hr);
  GPTQ_TRY(hipGetLastError());

  // blocked right-looking Cholesky of Hr
  for (int64_t k = 0; k < n; k += kNB) {
    const int64_t below = std::max<int64_t>(0, n - k - kNB);
    const int blocks = static_cast<int>(std::max<int64_t>(1, (below + kPanelRows - 1) / kPanelRows));
    panel_kernel<<<blocks, 256, 0, st>>>(Hr, n, k, info);
    GPTQ_TRY(hipGetLastError());
    if (below > 0) {
      const float* P = Hr + (k + kNB) * n + k;
      GPTQ_TRY(gemm_f32(below, below, kNB, -1.f, P, n, 0, P, n, 0, true, 1.f, Hr + (k + kNB) * (n + 1), n,
                        0, 1, true, 0, st));
    }
  }
  // triangular inverse: diagonal blocks, then recursive doubling
  const int64_t nblk = (n + kNB - 1) / kNB;
  diag_inverse_kernel<<<static_cast<int>(nblk), 256, 0, st>>>(Hr, n);
  GPTQ_TRY(hipGetLastError());
  for (int64_t h = 1; h < nblk; h *= 2) {
    const int64_t w_el = h * kNB;           // width of A (elements)
    const int64_t groups_full = n / (2 * w_el);
    // full groups: A and C both h blocks wide
    if (groups_full > 0) {
      const int64_t gs = 2 * w_el * (n + 1);  // stride between groups in Hr
      const float* L21 = Hr + w_el * n;        // rows [w_el, 2 w_el), cols [0, w_el)
      const float* Ainv = Hr;
      const float* Cinv = Hr + w_el * (n + 1);
      GPTQ_TRY(gemm_f32(w_el, w_el, w_el, 1.f, L21, n, gs, Ainv, n, gs, false, 0.f, T, w_el, w_el * w_el,
                        static_cast<int>(groups_full), false, 1, st));
      GPTQ_TRY(gemm_f32(w_el, w_el, w_el, -1.f, Cinv, n, gs, T, w_el, w_el * w_el, false, 0.f,
                        Hr + w_el * n, n, gs, static_cast<int>(groups_full), false, 2, st));
    }
    // ragged last group: A is h blocks wide, C is what remains (< h blocks)
    const int64_t a0 = groups_full * 2 * w_el;
    const int64_t c0 = a0 + w_el;
    if (c0 < n) {
      const int64_t cw = n - c0;
      const float* L21 = Hr + c0 * n + a0;
      const float* Ainv = Hr + a0 * (n + 1);
      const float* Cinv = Hr + c0 * (n + 1);
      GPTQ_TRY(gemm_f32(cw, w_el, w_el, 1.f, L21, n, 0, Ainv, n, 0, false, 0.f, T, w_el, 0, 1, false, 1, st));
      GPTQ_TRY(gemm_f32(cw, w_el, cw, -1.f, Cinv, n, 0, T, w_el, 0, false, 0.f, Hr + c0 * n + a0, n, 0, 1, false,
                        2, st));
    }
  }
  reverse_kernel<<<grid_for(nn), 256, 0, st>>>(Hr, n, U);
  return hipGetLastError();
}

}  // namespace gptq
