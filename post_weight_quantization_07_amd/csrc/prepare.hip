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
//   panels     right-looking blocked Cholesky of Hr, 128-column panels:
//                panel kernel: factor and invert the 128x128 diagonal block in
//                LDS, solve the panel rows below as a product with that
//                inverse, store the inverse in a strip of its own (Dinv);
//                trailing update Hr[k+128:, k+128:] -= P P^T on MFMA (lower tiles)
//   place      every inverted diagonal block from Dinv into Hr (one launch
//              after the last panel)
//   trtri      recursive doubling: for neighbouring inverted blocks A^-1, C^-1
//              and the factor block L21 below A, M21 = -C^-1 (L21 A^-1)
//   reverse    U[i][j] = M[n-1-i][n-1-j] for j >= i, 0 below the diagonal
#include "gptq_common.h"
#include "gptq_internal.h"

#include <algorithm>

namespace gptq {
namespace {

constexpr int kNB = kPanel;  // 128

// The elementwise passes over n x n matrices go row by row (workgroups over
// rows, threads over columns), so no thread divides a flat index.
__global__ void finalize_kernel(float* S, int64_t n, float scale, float* diag) {
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x)
    for (int64_t c = threadIdx.x; c < n; c += blockDim.x) {
      const float v = S[r * n + c] * scale;
      S[r * n + c] = v;
      if (c == r) diag[r] = v;
    }
}

// lambda = damp * mean(diag): fixed-order tree over 1024 threads.  A diagonal
// that is not finite (NaN or an infinity in X) sets info = -1; the panels then
// leave info alone (they only replace a 0).
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
    info[0] = isfinite(part[0]) ? 0 : -1;
  }
}

// perm[rank(i)] = i with rank(i) = #{j : d_j > d_i} + #{j < i : d_j == d_i}.
// A NaN key counts as -infinity (last, ties by index), so the ranks are always
// a permutation of 0 .. n-1 and every perm entry is written.
GPTQ_DEV float order_key(float d) { return (d == d) ? d : -INFINITY; }

__global__ __launch_bounds__(256) void order_kernel(const float* diag, int64_t n, int desc_act,
                                                    int32_t* perm) {
  __shared__ float tile[1024];
  const int64_t i = blockIdx.x * 256 + threadIdx.x;
  if (!desc_act) {
    if (i < n) perm[i] = static_cast<int32_t>(i);
    return;
  }
  const float di = (i < n) ? order_key(diag[i]) : 0.f;
  int64_t rank = 0;
  for (int64_t base = 0; base < n; base += 1024) {
    __syncthreads();
    for (int t = threadIdx.x; t < 1024; t += 256) tile[t] = (base + t < n) ? order_key(diag[base + t]) : 0.f;
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
  for (int64_t a = blockIdx.x; a < n; a += gridDim.x) {
    const int64_t pa = perm[n - 1 - a];
    for (int64_t b = threadIdx.x; b < n; b += blockDim.x) {
      float v = 0.f;
      if (b <= a) {
        v = H[pa * n + perm[n - 1 - b]];
        if (a == b) v += lam;
      }
      Hr[a * n + b] = v;
    }
  }
}

// ------------------------------------------------------------ panel kernel --
// One launch per 128-column panel k.  Every workgroup factors the 128x128
// diagonal block (the same arithmetic, so the same result) and inverts it, on
// LDS: L holds the block and its factor, M its inverse.  The block is taken as
// two 64-column halves (A11 A21 ; A21 A22):
//   L11 = chol(A11);  L21 = A21 L11^-T;  L22 = chol(A22 - L21 L21^T)
//   M = L^-1 = (L11^-1 0 ; -L22^-1 L21 L11^-1  L22^-1)
// The triangular solve of the rows below the block against L is then a
// product with M: X = P M^T, 32 rows per pass.  Workgroup 0 only stores M, the
// diagonal block of the factor's inverse that the recursive-doubling inverse
// uses as its first level, into the strip Dinv (block k / 128, row pitch 128);
// workgroups 1.. solve the rows.  Nothing in the launch writes the diagonal
// block of Hr that every workgroup reads at its start, so the result does not
// depend on how many workgroups are resident at once (the grid may exceed the
// CUs available to it, one workgroup per CU by LDS).
constexpr int kLP = kNB + 4;    // LDS row pitch (floats)
constexpr int kChunk = 32;      // panel rows solved per pass
constexpr int kMaxPanelWG = 256;
constexpr int kPanelGroup = 4;  // panels per trailing update of the Cholesky
constexpr int kPGW = kNB * kPanelGroup;  // columns of a panel group
// triangular-inverse levels at least this wide run on the three-part product
// (narrower levels measured faster on the fp32 product, whose 64-tiles skip
// more of the triangular operands' zeros)
constexpr int64_t kTrtriX3 = 2048;
using Blk = float (*)[kLP];
constexpr int kTP = 68;        // row pitch of the 64x64 product buffer
using TBlk = float (*)[kTP];

// v_mfma_f32_16x16x4_f32: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds D[4 (l / 16) + e][l % 16] in element e.
GPTQ_DEV f32x4_t mfma4(float a, float b, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

// acc += sign * A B over one 16-deep slice: A(m, k) = pa[ar + m][ac + k];
// B(k, n) = pb[br + k][bc + n], or pb[br + n][bc + k] when BT.  MFMA step s
// takes k = 4 q + s in lane group q (the same order for A and B), so a lane's
// four A values, and its four B values when BT, are one 16-byte LDS read.
template <bool BT, int PA, int PB>
GPTQ_DEV f32x4_t mma16(const float (*pa)[PA], int ar, int ac, const float (*pb)[PB], int br, int bc,
                       f32x4_t acc, float sign, int lane) {
  const int m = lane & 15, q = lane >> 4;
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&pa[ar + m][ac + 4 * q]);
  f32x4_t b;
  if (BT) {
    b = *reinterpret_cast<const f32x4_t*>(&pb[br + m][bc + 4 * q]);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = pb[br + 4 * q + s][bc + m];
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma4(sign * a[s], b[s], acc);
  return acc;
}

template <int P>
GPTQ_DEV f32x4_t load16(const float (*p)[P], int r, int c, int lane) {
  const int m = lane & 15, q = lane >> 4;
  f32x4_t v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = p[r + 4 * q + e][c + m];
  return v;
}

template <int P>
GPTQ_DEV void store16(float (*p)[P], int r, int c, f32x4_t v, int lane) {
  const int m = lane & 15, q = lane >> 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) p[r + 4 * q + e][c + m] = v[e];
}

// Operand fragments of one 16-deep slice, k = 4 q + s as in mma16:
// rows(p, r, c): lane (m, q) holds p[r + m][c + 4 q .. 4 q + 3] (an A operand,
// or a B operand read transposed); cols(p, r, c): p[r + 4 q + s][c + m] (a B
// operand read as stored).
template <int P>
GPTQ_DEV f32x4_t frag_rows(const float (*p)[P], int r, int c, int lane) {
  return *reinterpret_cast<const f32x4_t*>(&p[r + (lane & 15)][c + 4 * (lane >> 4)]);
}
template <int P>
GPTQ_DEV f32x4_t frag_cols(const float (*p)[P], int r, int c, int lane) {
  f32x4_t v;
#pragma unroll
  for (int s = 0; s < 4; ++s) v[s] = p[r + 4 * (lane >> 4) + s][c + (lane & 15)];
  return v;
}
GPTQ_DEV f32x4_t mma_frag(f32x4_t a, f32x4_t b, f32x4_t acc) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma4(a[s], b[s], acc);
  return acc;
}

// Lower Cholesky of the 64x64 block of L at (base, base), blocked by 16
// columns.  Sub-panel b (columns 16 b .. 16 b + 15 of the block, all its rows)
// is factored by wave 0, lane r holding row base + r's 16 entries in
// registers; the rank-16 update of the lower 16x16 blocks to its right runs on
// MFMA, spread over the four waves.
//
// Sub-panel factor, right-looking: at step j the pivot comes from lane j by
// readlane, every lane scales its column-j entry by 1 / sqrt(pivot) (hardware
// reciprocal square root, about 1 ulp; the pivot chain is the latency-critical
// path), and each later column c of the sub-panel takes -l[lane][j] l[c][j]
// with l[c][j] broadcast from lane c as a scalar operand.  The update of
// column j + 1 comes first, since the next pivot waits for it.  Lanes above
// the pivot only touch their own upper-triangle entries, which are discarded
// (the sub-panel is written back with zeros above the diagonal).  A pivot that
// is not positive (or not finite) leaves a NaN or zero on the diagonal, which
// the caller checks.
template <int base, int b>
GPTQ_DEV void factor_subpanel(Blk L, int lane) {
  constexpr int c0 = 16 * b;
  float v[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) v[c] = L[base + lane][base + c0 + c];
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    const float piv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[jj]), c0 + jj));
    const float l = v[jj] * __builtin_amdgcn_rsqf(piv);
    v[jj] = l;
#pragma unroll
    for (int c = jj + 1; c < 16; ++c) {
      const float lc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l), c0 + c));
      v[c] = fmaf(-l, lc, v[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) L[base + lane][base + c0 + c] = (c0 + c <= lane) ? v[c] : 0.f;
}

// Rank-16 update after sub-panel b: for the lower 16x16 blocks (I, J),
// b < J <= I <= 3, of the 64 block at base: L[I][J] -= P_I P_J^T with
// P_I = L[I][b].  Block t goes to wave t % 4.
template <int base, int b>
GPTQ_DEV void trailing_update(Blk L, int wave, int lane) {
  constexpr int nt = 3 - b;  // trailing blocks per edge
  int t = 0;
#pragma unroll
  for (int i = 0; i < nt; ++i) {
#pragma unroll
    for (int jb = 0; jb <= i; ++jb, ++t) {
      if (t % 4 != wave) continue;
      const int I = base + 16 * (b + 1 + i), J = base + 16 * (b + 1 + jb);
      f32x4_t acc = load16(L, I, J, lane);
      acc = mma16<true>(L, I, base + 16 * b, L, J, base + 16 * b, acc, -1.f, lane);
      store16(L, I, J, acc, lane);
    }
  }
}

template <int base>
GPTQ_DEV void factor64(Blk L, int wave, int lane) {
  if (wave == 0) factor_subpanel<base, 0>(L, lane);
  __syncthreads();
  trailing_update<base, 0>(L, wave, lane);
  __syncthreads();
  if (wave == 0) factor_subpanel<base, 1>(L, lane);
  __syncthreads();
  trailing_update<base, 1>(L, wave, lane);
  __syncthreads();
  if (wave == 0) factor_subpanel<base, 2>(L, lane);
  __syncthreads();
  trailing_update<base, 2>(L, wave, lane);
  __syncthreads();
  if (wave == 0) factor_subpanel<base, 3>(L, lane);
  __syncthreads();
}

// One doubling level of the inverse of a lower factor: for NP pairs of
// neighbouring inverted diagonal blocks (A^-1 at c0, C^-1 at r0 = c0 + 16 H,
// each 16 H wide, pair p at c0 = cb + 32 H p) with the factor block L21 below
// A, M21 = -C^-1 (L21 A^-1), written into M at (r0, c0); T = L21 A^-1 goes
// through the buffer Tb (pair p at column 16 H p).  The 16x16 output blocks of
// a pair are spread over the waves.
template <int H, int NP>
GPTQ_DEV void inverse_level(Blk L, Blk M, TBlk Tb, int cb, int wave, int lane) {
  auto owner = [](int p, int I, int J) { return (p * H * H + I * H + (I + J) % H) % 4; };
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c0 = cb + 32 * H * p, r0 = c0 + 16 * H;
#pragma unroll
    for (int I = 0; I < H; ++I)
#pragma unroll
      for (int J = 0; J < H; ++J) {
        if (owner(p, I, J) != wave) continue;
        f32x4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = J; K < H; ++K)  // A^-1 is lower triangular
          t = mma16<false>(L, r0 + 16 * I, c0 + 16 * K, M, c0 + 16 * K, c0 + 16 * J, t, 1.f, lane);
        store16(Tb, 16 * I, 16 * H * p + 16 * J, t, lane);
      }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c0 = cb + 32 * H * p, r0 = c0 + 16 * H;
#pragma unroll
    for (int I = 0; I < H; ++I)
#pragma unroll
      for (int J = 0; J < H; ++J) {
        if (owner(p, I, J) != wave) continue;
        f32x4_t t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = 0; K <= I; ++K)  // C^-1 is lower triangular
          t = mma16<false>(M, r0 + 16 * I, r0 + 16 * K, Tb, 16 * K, 16 * H * p + 16 * J, t, -1.f, lane);
        store16(M, r0 + 16 * I, c0 + 16 * J, t, lane);
      }
  }
  __syncthreads();
}

// M = inverse of the factored 64x64 block of L at (base, base): the four 16x16
// diagonal blocks by forward substitution (wave 0, lane = 16 block + column,
// one column of the inverse per lane, zeros above the diagonal), then two
// doubling levels.
template <int base>
GPTQ_DEV void inverse64(Blk L, Blk M, TBlk Tb, int wave, int lane) {
  if (wave == 0) {
    const int o = base + 16 * (lane >> 4), c = lane & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int t = 0; t < i; ++t) s = fmaf(-L[o + i][o + t], x[t], s);
      x[i] = s * __builtin_amdgcn_rcpf(L[o + i][o + i]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) M[o + i][o + c] = x[i];
  }
  __syncthreads();
  inverse_level<1, 2>(L, M, Tb, base, wave, lane);
  inverse_level<2, 1>(L, M, Tb, base, wave, lane);
}

// ---- the per-wave MFMA work of the 128 block, K-slices outermost so that a
// wave's output blocks form independent accumulation chains sharing operands;
// the next slice's fragments are read before this slice's products (the
// scheduling barriers keep that order).  Block indices are in 16s; the
// 64-halves start at 0 and 64.

// L21[I][J] = sum_{K <= J} A21[I][K] (L11^-1)[J][K]^T, wave = row I.
template <int I>
GPTQ_DEV void l21_row(Blk L, Blk M, int lane, f32x4_t (&acc)[4]) {
  f32x4_t a, b[4], na, nb[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    acc[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    b[J] = frag_rows(M, 16 * J, 0, lane);
  }
  a = frag_rows(L, 64 + 16 * I, 0, lane);
#pragma unroll
  for (int K = 0; K < 4; ++K) {
    if (K < 3) {
      na = frag_rows(L, 64 + 16 * I, 16 * (K + 1), lane);
#pragma unroll
      for (int J = K + 1; J < 4; ++J) nb[J] = frag_rows(M, 16 * J, 16 * (K + 1), lane);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int J = K; J < 4; ++J) acc[J] = mma_frag(a, b[J], acc[J]);
    __builtin_amdgcn_sched_barrier(0);
    a = na;
#pragma unroll
    for (int J = K + 1; J < 4; ++J) b[J] = nb[J];
  }
}

// A22[I][J] -= sum_K L21[I][K] L21[J][K]^T for J in [J0, J0 + NJ) (J <= I).
template <int I, int J0, int NJ>
GPTQ_DEV void a22_row(Blk L, int lane) {
  f32x4_t acc[NJ], a, b[NJ], na, nb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    acc[j] = load16(L, 64 + 16 * I, 64 + 16 * (J0 + j), lane);
    b[j] = frag_rows(L, 64 + 16 * (J0 + j), 0, lane);
  }
  a = frag_rows(L, 64 + 16 * I, 0, lane);
#pragma unroll
  for (int K = 0; K < 4; ++K) {
    if (K < 3) {
      na = frag_rows(L, 64 + 16 * I, 16 * (K + 1), lane);
#pragma unroll
      for (int j = 0; j < NJ; ++j) nb[j] = frag_rows(L, 64 + 16 * (J0 + j), 16 * (K + 1), lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    const f32x4_t an = -a;
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[j] = mma_frag(an, b[j], acc[j]);
    __builtin_amdgcn_sched_barrier(0);
    a = na;
#pragma unroll
    for (int j = 0; j < NJ; ++j) b[j] = nb[j];
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) store16(L, 64 + 16 * I, 64 + 16 * (J0 + j), acc[j], lane);
}

// T[I][J] = sum_{K >= J} L21[I][K] (L11^-1)[K][J], wave = row I, into Tb.
template <int I>
GPTQ_DEV void t_row(Blk L, Blk M, TBlk Tb, int lane) {
  f32x4_t acc[4], a, b[4], na, nb[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) acc[J] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  a = frag_rows(L, 64 + 16 * I, 0, lane);
  b[0] = frag_cols(M, 0, 0, lane);
#pragma unroll
  for (int K = 0; K < 4; ++K) {
    if (K < 3) {
      na = frag_rows(L, 64 + 16 * I, 16 * (K + 1), lane);
#pragma unroll
      for (int J = 0; J <= K + 1; ++J) nb[J] = frag_cols(M, 16 * (K + 1), 16 * J, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int J = 0; J <= K; ++J) acc[J] = mma_frag(a, b[J], acc[J]);
    __builtin_amdgcn_sched_barrier(0);
    a = na;
#pragma unroll
    for (int J = 0; J <= K + 1 && J < 4; ++J) b[J] = nb[J];
  }
#pragma unroll
  for (int J = 0; J < 4; ++J) store16(Tb, 16 * I, 16 * J, acc[J], lane);
}

// M21[I][J] = -sum_{K <= I} (L22^-1)[I][K] T[K][J], wave = column J, into M.
template <int J>
GPTQ_DEV void m21_col(Blk M, TBlk Tb, int lane) {
  f32x4_t acc[4], b, a[4], nbv, na[4];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    acc[I] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    a[I] = frag_rows(M, 64 + 16 * I, 64, lane);
  }
  b = frag_cols(Tb, 0, 16 * J, lane);
#pragma unroll
  for (int K = 0; K < 4; ++K) {
    if (K < 3) {
      nbv = frag_cols(Tb, 16 * (K + 1), 16 * J, lane);
#pragma unroll
      for (int I = K + 1; I < 4; ++I) na[I] = frag_rows(M, 64 + 16 * I, 64 + 16 * (K + 1), lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    const f32x4_t bn = -b;
#pragma unroll
    for (int I = K; I < 4; ++I) acc[I] = mma_frag(a[I], bn, acc[I]);
    __builtin_amdgcn_sched_barrier(0);
    b = nbv;
#pragma unroll
    for (int I = K + 1; I < 4; ++I) a[I] = na[I];
  }
#pragma unroll
  for (int I = 0; I < 4; ++I) store16(M, 64 + 16 * I, 16 * J, acc[I], lane);
}

// X = P M^T for the 32 staged rows (L rows 0..31): output blocks (I, J) with
// I in {0, 1} and J in {W, 7 - W}; block (I, J) needs slices K <= J.
template <int W>
GPTQ_DEV void solve_rows(Blk L, Blk M, int lane, f32x4_t (&acc)[4]) {
  constexpr int J1 = W, J2 = 7 - W;
  f32x4_t c0, c1, c2, c3, n0, n1, n2, n3;
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  c0 = frag_rows(L, 0, 0, lane);
  c1 = frag_rows(L, 16, 0, lane);
  c2 = frag_rows(M, 16 * J1, 0, lane);
  c3 = frag_rows(M, 16 * J2, 0, lane);
#pragma unroll
  for (int K = 0; K <= J2; ++K) {
    if (K + 1 <= J2) {
      n0 = frag_rows(L, 0, 16 * (K + 1), lane);
      n1 = frag_rows(L, 16, 16 * (K + 1), lane);
      if (K + 1 <= J1) n2 = frag_rows(M, 16 * J1, 16 * (K + 1), lane);
      n3 = frag_rows(M, 16 * J2, 16 * (K + 1), lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (K <= J1) {
      acc[0] = mma_frag(c0, c2, acc[0]);
      acc[1] = mma_frag(c1, c2, acc[1]);
    }
    acc[2] = mma_frag(c0, c3, acc[2]);
    acc[3] = mma_frag(c1, c3, acc[3]);
    __builtin_amdgcn_sched_barrier(0);
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
}

__global__ __launch_bounds__(256, 1) void panel_kernel(float* Hr, int64_t n, int64_t k, int32_t* info,
                                                         float* Dinv, uint16_t* P, int64_t pplane, int64_t kg) {
  __shared__ __attribute__((aligned(16))) float L[kNB][kLP];
  __shared__ __attribute__((aligned(16))) float M[kNB][kLP];
  __shared__ __attribute__((aligned(16))) float Tb[kNB / 2][kTP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = static_cast<int>(std::min<int64_t>(kNB, n - k));
  const int64_t below = (nb == kNB) ? n - k - kNB : 0;
  const int64_t chunks = (below + kChunk - 1) / kChunk;
  // workgroup 0 stores M; the others solve chunks blockIdx - 1, + (grid - 1), ...
  const int64_t ch0 = static_cast<int64_t>(blockIdx.x) - 1, chs = static_cast<int64_t>(gridDim.x) - 1;
  // 16-byte rows: every row of the block and of the panel starts 16-byte aligned
  const bool vec = (n & 3) == 0 && nb == kNB;

  // The diagonal block (lower part; identity past a ragged end) and this
  // workgroup's first 32 panel rows.  Every load reads an in-range address
  // (clamped into the block's lower part or the last row) and the value is
  // selected after, so all loads are in flight at once.
  // pv holds the loaded values as they come and pmask which of them are real
  // rows; the select waits until the rows are staged, so the loads of the
  // next chunk stay in flight during this chunk's products.
  float pv[kChunk * kNB / 256];
  uint32_t pmask = 0;
  const int vr = tid >> 5, vc = 4 * (tid & 31);  // float4 layout: 8 rows x 32 float4 per pass
  const int sr = tid >> 7, sc = tid & 127;       // scalar layout: 2 rows x 128 per pass
  auto load_rows = [&](int64_t ch) {
    const bool live = ch >= 0 && ch < chunks;
    const int64_t r0 = k + kNB + ch * kChunk;
    pmask = 0;
    if (vec) {
#pragma unroll
      for (int i = 0; i < kChunk / 8; ++i) {
        const int64_t row = r0 + 8 * i + vr;
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(Hr + std::min<int64_t>(row, n - 1) * n + k + vc);
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[4 * i + e] = x[e];
        pmask |= (live && row < n) ? (1u << i) : 0u;
      }
    } else {
      const int64_t col = std::min<int64_t>(k + sc, n - 1);
#pragma unroll
      for (int i = 0; i < kChunk / 2; ++i) {
        const int64_t row = r0 + 2 * i + sr;
        pv[i] = Hr[std::min<int64_t>(row, n - 1) * n + col];
        pmask |= (live && row < n) ? (1u << i) : 0u;
      }
    }
  };
  auto stage_rows = [&]() {
    if (vec) {
#pragma unroll
      for (int i = 0; i < kChunk / 8; ++i) {
        const bool ok = (pmask >> i) & 1u;
        *reinterpret_cast<f32x4_t*>(&L[8 * i + vr][vc]) =
            ok ? f32x4_t{pv[4 * i], pv[4 * i + 1], pv[4 * i + 2], pv[4 * i + 3]} : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    } else {
#pragma unroll
      for (int i = 0; i < kChunk / 2; ++i) L[2 * i + sr][sc] = ((pmask >> i) & 1u) ? pv[i] : 0.f;
    }
  };
  if (vec) {
    f32x4_t lv[kNB / 8];
#pragma unroll
    for (int i = 0; i < kNB / 8; ++i) {
      const int r = 8 * i + vr;
      lv[i] = *reinterpret_cast<const f32x4_t*>(Hr + (k + r) * n + k + std::min(vc, r & ~3));
    }
    load_rows(ch0);
#pragma unroll
    for (int i = 0; i < kNB / 8; ++i) {
      const int r = 8 * i + vr;
      f32x4_t x = lv[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (vc + e <= r) ? x[e] : 0.f;
      *reinterpret_cast<f32x4_t*>(&L[r][vc]) = x;
    }
  } else {
    float lv[kNB * kNB / 256];
#pragma unroll
    for (int i = 0; i < kNB * kNB / 256; ++i) {
      const int r = 2 * i + sr;
      const int rr = std::min(r, nb - 1), cc = std::min(sc, rr);
      const float x = Hr[(k + rr) * n + k + cc];
      lv[i] = (r < nb && sc <= r) ? x : ((r == sc) ? 1.f : 0.f);
    }
    load_rows(ch0);
#pragma unroll
    for (int i = 0; i < kNB * kNB / 256; ++i) L[2 * i + sr][sc] = lv[i];
  }
  __syncthreads();

  factor64<0>(L, wave, lane);
  inverse64<0>(L, M, Tb, wave, lane);
  // L21 = A21 L11^-T, in registers until every wave has read A21
  {
    f32x4_t acc[4];
    switch (wave) {
      case 0: l21_row<0>(L, M, lane, acc); break;
      case 1: l21_row<1>(L, M, lane, acc); break;
      case 2: l21_row<2>(L, M, lane, acc); break;
      default: l21_row<3>(L, M, lane, acc); break;
    }
    __syncthreads();
#pragma unroll
    for (int J = 0; J < 4; ++J) store16(L, 64 + 16 * wave, 16 * J, acc[J], lane);
    __syncthreads();
  }
  // A22 -= L21 L21^T on the ten lower 16x16 blocks (3, 3, 2, 2 per wave)
  switch (wave) {
    case 0: a22_row<3, 0, 3>(L, lane); break;
    case 1: a22_row<2, 0, 3>(L, lane); break;
    case 2: a22_row<1, 0, 2>(L, lane); break;
    default: a22_row<0, 0, 1>(L, lane); a22_row<3, 3, 1>(L, lane); break;
  }
  __syncthreads();
  factor64<64>(L, wave, lane);
  // first pivot that was not positive: its diagonal entry is NaN or zero
  if (wave == 0 && blockIdx.x == 0) {
    const uint64_t bad1 = __ballot(lane < nb && !(L[lane][lane] > 0.f));
    const uint64_t bad2 = __ballot(64 + lane < nb && !(L[64 + lane][64 + lane] > 0.f));
    if (lane == 0 && (bad1 | bad2) != 0) {
      const int f = bad1 ? __ffsll(static_cast<long long>(bad1)) - 1 : 64 + __ffsll(static_cast<long long>(bad2)) - 1;
      atomicCAS(info, 0, static_cast<int32_t>(n - (k + f)));
    }
  }
  inverse64<64>(L, M, Tb, wave, lane);
  // M21 = -L22^-1 (L21 L11^-1)
  switch (wave) {
    case 0: t_row<0>(L, M, Tb, lane); break;
    case 1: t_row<1>(L, M, Tb, lane); break;
    case 2: t_row<2>(L, M, Tb, lane); break;
    default: t_row<3>(L, M, Tb, lane); break;
  }
  __syncthreads();
  switch (wave) {
    case 0: m21_col<0>(M, Tb, lane); break;
    case 1: m21_col<1>(M, Tb, lane); break;
    case 2: m21_col<2>(M, Tb, lane); break;
    default: m21_col<3>(M, Tb, lane); break;
  }
  __syncthreads();

  // M = L^-1 (lower, zeros above the diagonal) into block k / 128 of Dinv;
  // past a ragged end the block holds the inverse of the identity padding,
  // which the placement skips
  if (blockIdx.x == 0) {
    float* dst = Dinv + (k / kNB) * (kNB * kNB);
#pragma unroll
    for (int i = 0; i < kNB / 8; ++i) {
      const int r = 8 * i + vr;
      f32x4_t x = *reinterpret_cast<const f32x4_t*>(&M[r][vc]);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (vc + e <= r) ? x[e] : 0.f;
      *reinterpret_cast<f32x4_t*>(dst + r * kNB + vc) = x;
    }
    return;
  }
  // X = P M^T, 32 rows at a time (staged in L's rows 0..31)
  for (int64_t ch = ch0; ch < chunks; ch += chs) {
    stage_rows();
    __syncthreads();
    load_rows(ch + chs);
    f32x4_t acc[4];
    switch (wave) {
      case 0: solve_rows<0>(L, M, lane, acc); break;
      case 1: solve_rows<1>(L, M, lane, acc); break;
      case 2: solve_rows<2>(L, M, lane, acc); break;
      default: solve_rows<3>(L, M, lane, acc); break;
    }
    const int64_t r0 = k + kNB + ch * kChunk;
    const int m = lane & 15, q = lane >> 4;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int J = (t < 2) ? wave : 7 - wave;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = r0 + 16 * (t & 1) + 4 * q + e;
        if (row < n) {
          Hr[row * n + k + 16 * J + m] = acc[t][e];
          // and as three bf16 planes, column (k - kg) + 16 J + m of the
          // group's panel: the operands of the Cholesky updates
          uint16_t hh, mm, ll;
          split3(acc[t][e], hh, mm, ll);
          const int64_t o = x3_offset(row, k - kg + 16 * J + m, kPGW);
          P[o] = hh;
          P[pplane + o] = mm;
          P[2 * pplane + o] = ll;
        }
      }
    }
    __syncthreads();
  }
}

// Hr's diagonal blocks <- the inverted blocks of Dinv (the first level of the
// factor's inverse), rows and columns past a ragged end left alone.
__global__ void place_dinv_kernel(const float* Dinv, int64_t n, float* Hr) {
  const int64_t nblk = (n + kNB - 1) / kNB;
  const int64_t total = nblk * kNB * kNB;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t b = e / (kNB * kNB), r = (e / kNB) % kNB, c = e % kNB;
    const int64_t row = b * kNB + r, col = b * kNB + c;
    if (row < n && col < n) Hr[row * n + col] = Dinv[e];
  }
}

__global__ void reverse_kernel(const float* M, int64_t n, float* U) {
  for (int64_t i = blockIdx.x; i < n; i += gridDim.x)
    for (int64_t j = threadIdx.x; j < n; j += blockDim.x)
      U[i * n + j] = (j >= i) ? M[(n - 1 - i) * n + (n - 1 - j)] : 0.f;
}

// one workgroup per row, at most 8192
int row_grid(int64_t n) { return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(n, 8192))); }

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
  L.off_dinv = off;  // inverted 128x128 diagonal blocks, one per panel
  off += up(static_cast<size_t>((d + kNB - 1) / kNB) * kNB * kNB * sizeof(float));
  L.off_lambda = off;
  off += 256;
  L.off_p = off;  // a panel group's factor columns as three bf16 planes (blocked layout)
  off += up(3 * static_cast<size_t>(x3_plane_elems(d, kPGW)) * sizeof(uint16_t));
  // the triangular inverse's levels on the bf16 matrix cores: both operands
  // of a level's products as three bf16 planes, all of the level's groups
  size_t qa = 0, qb = 0;
  for (int64_t w = kNB; w < d; w *= 2) {
    if (w < kTrtriX3) continue;
    const int64_t full = d / (2 * w), cw = d - (full * 2 * w + w);
    qa = std::max(qa, static_cast<size_t>(full * w * w));  // the full groups' L21, then C^-1
    qb = std::max(qb, static_cast<size_t>(full * w * w));  // A^-1 transposed, then T transposed
    if (cw > 0) {  // the ragged group
      qa = std::max(qa, static_cast<size_t>(std::max(x3_plane_elems(cw, w), x3_plane_elems(cw, cw))));
      qb = std::max(qb, static_cast<size_t>(std::max(x3_plane_elems(w, w), x3_plane_elems(w, cw))));
    }
  }
  L.off_qa = off;
  off += up(3 * qa * sizeof(uint16_t));
  L.off_qb = off;
  off += up(3 * qb * sizeof(uint16_t));
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
  float* Dinv = reinterpret_cast<float*>(w + lay.off_dinv);
  uint16_t* P = reinterpret_cast<uint16_t*>(w + lay.off_p);
  uint16_t* QA = reinterpret_cast<uint16_t*>(w + lay.off_qa);
  uint16_t* QB = reinterpret_cast<uint16_t*>(w + lay.off_qb);
  const int64_t pplane = x3_plane_elems(n, kPGW);

  {
    PhaseScope ph(kPhPrepElem, st);
    finalize_kernel<<<row_grid(n), 256, 0, st>>>(S, n, static_cast<float>(2.0 / static_cast<double>(n_total)), diag);
    GPTQ_TRY(hipGetLastError());
    lambda_kernel<<<1, 1024, 0, st>>>(diag, n, damp, lam, info);
    GPTQ_TRY(hipGetLastError());
    order_kernel<<<static_cast<int>((n + 255) / 256), 256, 0, st>>>(diag, n, desc_act ? 1 : 0, perm);
    GPTQ_TRY(hipGetLastError());
    gather_kernel<<<row_grid(n), 256, 0, st>>>(S, n, perm, lam, Hr);
    GPTQ_TRY(hipGetLastError());
  }

  // blocked right-looking Cholesky of Hr; the panel kernels leave the inverse
  // of every diagonal block in place.  Panels go in groups of kPanelGroup:
  // each later panel's block column is first brought up to date with the
  // group's earlier panels (a tall product, K = 128 per earlier panel), and
  // the trailing matrix past the group takes one update with all of the
  // group's columns (K = 128 kPanelGroup).  The same products as one update
  // per panel, summed in another order; the large lower-triangle update reads
  // and writes the trailing matrix once per group instead of once per panel.
  // Both products run on the bf16 matrix cores (gemm_x3): the panel kernels
  // write their factor rows below the diagonal block also as three bf16
  // planes of the group's panel P, which serves as both operands.
  for (int64_t k = 0; k < n; k += kPGW) {
    for (int h = 0; h < kPanelGroup; ++h) {
      const int64_t kh = k + h * kNB;
      if (kh >= n) break;
      if (h > 0) {
        // the panel's block column takes the group's earlier panels: rows
        // kh .. of their columns, from the group's planes (K = 128 per panel)
        const int64_t wc = std::min<int64_t>(kNB, n - kh);
        const uint16_t* A = P + x3_offset(kh, 0, kPGW);
        PhaseScope ph(kPhCholUpdate, st);
        GPTQ_TRY(gemm_x3(n - kh, wc, kh - k, -1.f, A, pplane, A, pplane, Hr + kh * (n + 1), n, st, kPGW, false));
      }
      const int64_t below = std::max<int64_t>(0, n - kh - kNB);
      const int blocks = 1 + static_cast<int>(std::min<int64_t>((below + kChunk - 1) / kChunk, kMaxPanelWG - 1));
      {
        PhaseScope ph(kPhPanel, st);
        panel_kernel<<<blocks, 256, 0, st>>>(Hr, n, kh, info, Dinv, P, pplane, k);
      }
      GPTQ_TRY(hipGetLastError());
    }
    const int64_t ke = std::min<int64_t>(n, k + kPGW);
    const int64_t below = n - ke;
    if (below > 0) {
      const uint16_t* A = P + x3_offset(ke, 0, kPGW);
      PhaseScope ph(kPhCholUpdate, st);
      GPTQ_TRY(gemm_x3(below, below, ke - k, -1.f, A, pplane, A, pplane, Hr + ke * (n + 1), n, st, kPGW, true));
    }
  }
  // triangular inverse by recursive doubling over the inverted diagonal blocks
  const int64_t nblk = (n + kNB - 1) / kNB;
  PhaseScope ph_trtri(kPhTrtri, st);
  place_dinv_kernel<<<grid_for(nblk * kNB * kNB), 256, 0, st>>>(Dinv, n, Hr);
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
      const int gb = static_cast<int>(groups_full);
      if (w_el >= kTrtriX3) {
        // on the bf16 matrix cores: each operand split into three bf16
        // planes first (A row by row, B transposed); the tiles skip the
        // zero K range of the triangular operand as gemm_f32 does
        const int64_t pe = w_el * w_el;  // elements of one plane (w_el a multiple of 128)
        const int64_t be = 3 * pe;       // one group's three planes
        GPTQ_TRY(split3_rows(L21, n, w_el, w_el, QA, st, gb, gs, be));
        GPTQ_TRY(split3_t(Ainv, n, w_el, w_el, QB, st, gb, gs, be));
        GPTQ_TRY(gemm_x3(w_el, w_el, w_el, 1.f, QA, pe, QB, pe, T, w_el, st, 0, false, 1, true, gb, be, be, pe));
        GPTQ_TRY(split3_rows(Cinv, n, w_el, w_el, QA, st, gb, gs, be));
        GPTQ_TRY(split3_t(T, w_el, w_el, w_el, QB, st, gb, pe, be));
        GPTQ_TRY(gemm_x3(w_el, w_el, w_el, -1.f, QA, pe, QB, pe, Hr + w_el * n, n, st, 0, false, 2, true, gb, be, be,
                         gs));
      } else {
        GPTQ_TRY(gemm_f32(w_el, w_el, w_el, 1.f, L21, n, gs, Ainv, n, gs, false, 0.f, T, w_el, w_el * w_el, gb,
                          false, 1, st));
        GPTQ_TRY(gemm_f32(w_el, w_el, w_el, -1.f, Cinv, n, gs, T, w_el, w_el * w_el, false, 0.f, Hr + w_el * n, n,
                          gs, gb, false, 2, st));
      }
    }
    // ragged last group: A is h blocks wide, C is what remains (< h blocks)
    const int64_t a0 = groups_full * 2 * w_el;
    const int64_t c0 = a0 + w_el;
    if (c0 < n) {
      const int64_t cw = n - c0;
      const float* L21 = Hr + c0 * n + a0;
      const float* Ainv = Hr + a0 * (n + 1);
      const float* Cinv = Hr + c0 * (n + 1);
      if (w_el >= kTrtriX3) {
        GPTQ_TRY(split3_rows(L21, n, cw, w_el, QA, st));
        GPTQ_TRY(split3_t(Ainv, n, w_el, w_el, QB, st));
        GPTQ_TRY(gemm_x3(cw, w_el, w_el, 1.f, QA, x3_plane_elems(cw, w_el), QB, x3_plane_elems(w_el, w_el), T, w_el,
                         st, 0, false, 1, true));
      } else {
        GPTQ_TRY(gemm_f32(cw, w_el, w_el, 1.f, L21, n, 0, Ainv, n, 0, false, 0.f, T, w_el, 0, 1, false, 1, st));
      }
      if (w_el >= kTrtriX3 && cw % 64 == 0) {
        GPTQ_TRY(split3_rows(Cinv, n, cw, cw, QA, st));
        GPTQ_TRY(split3_t(T, w_el, cw, w_el, QB, st));
        GPTQ_TRY(gemm_x3(cw, w_el, cw, -1.f, QA, x3_plane_elems(cw, cw), QB, x3_plane_elems(w_el, cw),
                         Hr + c0 * n + a0, n, st, 0, false, 2, true));
      } else {
        GPTQ_TRY(gemm_f32(cw, w_el, cw, -1.f, Cinv, n, 0, T, w_el, 0, false, 0.f, Hr + c0 * n + a0, n, 0, 1, false,
                          2, st));
      }
    }
  }
  reverse_kernel<<<row_grid(n), 256, 0, st>>>(Hr, n, U);
  return hipGetLastError();  // the triangular inverse's phase closes after the reversal
}

}  // namespace gptq
