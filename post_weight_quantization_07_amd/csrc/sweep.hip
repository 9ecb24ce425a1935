// The GPTQ column sweep over lazy 128-column blocks.
//
// GPTQ 实战 ch.5, section 5.1.8 (the implementation-level pseudocode and the
// OBS closed form): each column is rounded to its group's grid, its error is
// normalised by the factor's diagonal U[i][i] and subtracted, scaled by row i
// of U, from the not-yet-quantized columns of the block; after the block one
// matrix product applies the block's errors to every later column.  Groups
// (skill card, 分组量化; ch.5 section 5.1.10) carry one scale and zero point
// per output row; sym / static_groups follow BaseQuantizeConfig (AutoGPTQ
// examples walkthrough, section 1.4).
//
// Rows are independent given U, so the sweep is parallel over output rows and
// sequential over the block's 128 columns.  Layout: 16 lanes (one DPP row) per
// output row; block column c lives in lane c % 16 of the row, register c / 16
// (interleaved), so from step i = 16 k on no lane needs registers below k and
// the step skips them.  At step i every lane decides its own copy of the
// register holding column i, the owner lane's error is broadcast to its row
// with DPP row_newbcast, and every lane applies the rank-1 update to its live
// registers with row i of the block's U read from LDS.
//
// The LDS copy of U holds each row divided by its diagonal element, so the
// broadcast value is the plain remainder (negated: s q - w) and the update an
// accumulate that reads it through DPP.  Its diagonal is set to zero (the
// diagonal is kept apart for the normalised errors) and it is zero left of
// the diagonal, so the update leaves the column of step i and every earlier
// column unchanged: each register ends the block holding the value its column
// had when it was decided, and codes and errors are taken from it once after
// the sweep with the same arithmetic.  The chain of a step is then the
// decision and one fma.
#include "gptq_common.h"
#include "gptq_internal.h"

#include <algorithm>

namespace gptq {
namespace {

constexpr int kB = 128;         // lazy-batch width
constexpr int kRowsPerWG = 16;  // 256 threads / 16 lanes
constexpr int kUnitsPerGroup = 4;  // pairs of blocks per trailing update

struct SweepParams {
  float* Wp;            // [d_out, d_in] fp32 working copy, sweep order
  const float* U;       // [d_in, d_in]
  const int32_t* perm;  // sweep position -> original column
  uint8_t* codes;       // [d_out, d_in] original order
  float* Q;             // optional [d_out, d_in] original order
  float* scales;        // [n_groups, d_out]
  int32_t* zeros;       // [n_groups, d_out]
  float* row_loss;      // optional [d_out]
  float* Err;           // this block's normalised errors, rows of ld_err floats
  int ld_err;
  const float* Eb;      // bring-up: errors of the previous block of the pair (rows of ld_err floats), or null
  const float* Uo;      // bring-up: U rows of that block, this block's columns (row stride d_in)
  int64_t d_out, d_in;
  int64_t j0;           // first sweep column of the block
  int ncols;            // columns in this block
  int bits;
  float maxq;
  int group;            // group size, or 0 for one group per row
  int sym;
  int preset;           // 1: scales/zeros of every column are already in the outputs
  int identity;         // perm is the identity
  int nblk;             // blocks per launch (group kernel)
  uint16_t* Ea;         // or null: the group's errors as three bf16 planes (blocked panel layout)
  int64_t ea_plane;     // elements per plane
  int ea_col;           // launch per block: the block's first column in the group's panel
};

GPTQ_DEV void group_params(float lo, float hi, const SweepParams& p, float& scale, float& zero) {
  lo = fminf(lo, 0.f);
  hi = fmaxf(hi, 0.f);
  if (p.sym) {
    const float a = fmaxf(-lo, hi);
    lo = -a;
    hi = a;
  }
  if (hi == lo) {
    lo = -1.f;
    hi = 1.f;
  }
  scale = (hi - lo) / p.maxq;
  zero = p.sym ? static_cast<float>(1 << (p.bits - 1)) : rintf(-lo / scale);
}

// The decision on one weight w with scale s (y = 1 / s correctly rounded),
// clamp bounds zl = -z, zh = maxq - z and d = 1 / U[i][i]: the code relative
// to the zero point, qr = q - z, and the normalised error.  w / s is formed
// correctly rounded from y: q0 = w y is within an ulp, the remainder w - s q0
// is exact in one fma, and q0 + (w - s q0) y rounds to the quotient
// (Markstein's correction step).  rint(w / s) clamped to [-z, maxq - z] is
// clamp(rint(w / s) + z, 0, maxq) - z exactly (integers); the dequantized
// weight is s qr and the error w - s qr (one fma).
GPTQ_DEV void decide(float w, float s, float y, float zl, float zh, float d, float& qr, float& err) {
  const float q0 = w * y;
  const float quot = fmaf(fmaf(-s, q0, w), y, q0);
  qr = __builtin_amdgcn_fmed3f(rintf(quot), zl, zh);
  err = fmaf(-s, qr, w) * d;
}

// This lane's values k = R .. 7 of one row of the block's U in LDS (two
// float4 at src): only the live ones are read, each piece at its natural
// alignment, so no read lands in a register that is already dead.
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
template <int R>
GPTQ_DEV void read_urow(const float* src, float (&d)[8]) {
  if constexpr (R == 0) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(src);
    d[0] = a[0]; d[1] = a[1]; d[2] = a[2]; d[3] = a[3];
  } else if constexpr (R == 1 || R == 2) {
    if constexpr (R == 1) d[1] = src[1];
    const f32x2_t a = *reinterpret_cast<const f32x2_t*>(src + 2);
    d[2] = a[0]; d[3] = a[1];
  } else if constexpr (R == 3) {
    d[3] = src[3];
  }
  if constexpr (R <= 4) {
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(src + 4);
    d[4] = b[0]; d[5] = b[1]; d[6] = b[2]; d[7] = b[3];
  } else if constexpr (R == 5 || R == 6) {
    if constexpr (R == 5) d[5] = src[5];
    const f32x2_t b = *reinterpret_cast<const f32x2_t*>(src + 6);
    d[6] = b[0]; d[7] = b[1];
  } else {
    d[7] = src[7];
  }
}

constexpr int kURing = 3;  // rows of U in registers: the current one and two read ahead

// GS > 0: dynamic groups of GS columns start inside the block (GS divides
// 128), so the range code is emitted only at steps I % GS == 0; GS == 0: every
// column's parameters are known before the block.  Keeping the code of the
// 128 unrolled steps small matters: it has to stay in the instruction cache.
// Ut: the block's U in LDS as [row i][lane t][register k] (8 floats a lane).
template <int GS, int I>
GPTQ_DEV void sweep_step(const SweepParams& p, const float* Ut, int t, float (&v)[8],
                         float (&sc)[8], float (&rc)[8], float (&zlo)[8], float (&zhi)[8], int64_t row,
                         float (&un)[kURing][8]) {
  constexpr int r = I >> 4, owner = I & 15;
  // the row of U two steps ahead is read now, so its LDS latency hides behind
  // a whole step; registers below that step's are dead and not read
  if constexpr (I + 2 < kB) {
    constexpr int r2 = (I + 2) >> 4;
    read_urow<r2>(Ut + ((I + 2) * 16 + t) * 8, un[(I + 2) % kURing]);
  }
  const float (&u)[8] = un[I % kURing];
  // dynamic groups that start inside the block: range over the group's
  // current values (registers I / 16 .. (I + GS - 1) / 16, all 16 lanes)
  if constexpr (GS > 0 && (I % GS) == 0) {
    if (I < p.ncols) {
      constexpr int klo = I / 16, khi = (I + GS - 1) / 16 < 8 ? (I + GS - 1) / 16 : 7;
      float lo = 0.f, hi = 0.f;
#pragma unroll
      for (int k = klo; k <= khi; ++k) {
        const int c = t + 16 * k;
        const bool in = (c >= I) && (c < I + GS) && (c < p.ncols);
        lo = in ? fminf(lo, v[k]) : lo;
        hi = in ? fmaxf(hi, v[k]) : hi;
      }
      lo = row_min16(lo);
      hi = row_max16(hi);
      float s, z;
      group_params(lo, hi, p, s, z);
      const float y = 1.0f / s;
#pragma unroll
      for (int k = klo; k <= khi; ++k) {
        const int c = t + 16 * k;
        const bool in = (c >= I) && (c < I + GS);
        sc[k] = in ? s : sc[k];
        rc[k] = in ? y : rc[k];
        zlo[k] = in ? -z : zlo[k];
        zhi[k] = in ? p.maxq - z : zhi[k];
      }
      if (t == owner && row < p.d_out) {
        const int64_t g = p.j0 / GS + I / GS;
        p.scales[g * p.d_out + row] = s;
        p.zeros[g * p.d_out + row] = static_cast<int32_t>(z);
      }
    }
  }
  // the owner's remainder s qr - w (the negated error before normalisation:
  // the rows of U in LDS carry the factor 1 / U[i][i]), broadcast to the row;
  // each update is then an accumulate v += e u[k] that reads the broadcast
  // through DPP
  const float w = v[r];
  const float q0 = w * rc[r];
  const float quot = fmaf(fmaf(-sc[r], q0, w), rc[r], q0);
  const float qr = __builtin_amdgcn_fmed3f(rintf(quot), zlo[r], zhi[r]);
  const float eb = row_bcast<owner>(fmaf(sc[r], qr, -w));
  // the next column first: the next step's decision waits on it
  constexpr int rn = (I + 1) >> 4;
  if constexpr (I + 1 < kB) v[rn] = fmaf(eb, u[rn], v[rn]);
#pragma unroll
  for (int k = r; k < 8; ++k)
    if (k != rn) v[k] = fmaf(eb, u[k], v[k]);
  // keep each step a scheduling region of its own (bounded register pressure)
  __builtin_amdgcn_sched_barrier(0);
}

template <int GS, int... Is>
GPTQ_DEV void sweep_all(const SweepParams& p, const float* Ut, int t, float (&v)[8],
                        float (&sc)[8], float (&rc)[8], float (&zlo)[8], float (&zhi)[8], int64_t row,
                        std::integer_sequence<int, Is...>) {
  float un[kURing][8];
  read_urow<0>(Ut + t * 8, un[0]);
  read_urow<0>(Ut + (16 + t) * 8, un[1]);
  (sweep_step<GS, Is>(p, Ut, t, v, sc, rc, zlo, zhi, row, un), ...);
}

// The block's U (rows and columns jb .. jb + ncols) for the interleaved LDS
// layout: thread tid takes the (row i, lane l) pairs tid + 256 u, u < 8, and
// lane l's columns l + 16 k.  Every address is in range (rows and columns past
// the end are clamped); the values are selected when stored.
GPTQ_DEV void load_ublock(const SweepParams& p, int64_t jb, int ncols, int tid, float (&ul)[64], float (&dg)[8]) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int pi = tid + 256 * u, i = std::min(pi >> 4, ncols - 1), l = pi & 15;
    const float* src = p.U + (jb + i) * p.d_in + jb;
#pragma unroll
    for (int k = 0; k < 8; ++k) ul[8 * u + k] = src[std::min(l + 16 * k, ncols - 1)];
    dg[u] = src[i];
  }
}

// The loaded block of U scaled in registers for its LDS copy: U[i][l + 16 k]
// / U[i][i] (the product with the correctly rounded reciprocal) off the
// diagonal, zero on it and outside the block.
GPTQ_DEV void scale_ublock(float (&ul)[64], const float (&dg)[8], int ncols, int tid) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int pi = tid + 256 * u, i = pi >> 4, l = pi & 15;
    const float d = 1.0f / dg[u];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = l + 16 * k;
      ul[8 * u + k] = (i < ncols && c < ncols && i != c) ? ul[8 * u + k] * d : 0.f;
    }
  }
}

// Ut[i][l][k] from the scaled registers; the diagonal goes to Dg.
GPTQ_DEV void write_ublock(float* Ut, float* Dg, const float (&ul)[64], const float (&dg)[8], int ncols, int tid) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int pi = tid + 256 * u, i = pi >> 4, l = pi & 15;
    if (l == (i & 15) && i < ncols) Dg[i] = dg[u];
    *reinterpret_cast<f32x4_t*>(Ut + 8 * pi) = f32x4_t{ul[8 * u], ul[8 * u + 1], ul[8 * u + 2], ul[8 * u + 3]};
    *reinterpret_cast<f32x4_t*>(Ut + 8 * pi + 4) = f32x4_t{ul[8 * u + 4], ul[8 * u + 5], ul[8 * u + 6], ul[8 * u + 7]};
  }
}

GPTQ_DEV void store_ublock(float* Ut, float* Dg, float (&ul)[64], const float (&dg)[8], int ncols, int tid) {
  scale_ublock(ul, dg, ncols, tid);
  write_ublock(Ut, Dg, ul, dg, ncols, tid);
}

// This lane's weights of the block (columns t + 16 k), in range for any row.
GPTQ_DEV void load_wblock(const SweepParams& p, int64_t jb, int ncols, int64_t row, int t, float (&w)[8]) {
  const float* src = p.Wp + std::min<int64_t>(row, p.d_out - 1) * p.d_in + jb;
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = src[std::min(t + 16 * k, ncols - 1)];
}

// Registers at the start of a block: weights (zero past the block and for
// rows past the end), 1 / U[c][c] of this lane's columns, neutral parameters.
GPTQ_DEV void init_block(const SweepParams& p, const float* Dg, const float (&w)[8], bool row_ok, int t,
                         float (&v)[8], float (&dv)[8], float (&sc)[8], float (&rc)[8], float (&zlo)[8],
                         float (&zhi)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = t + 16 * k;
    dv[k] = (c < p.ncols) ? 1.0f / Dg[c] : 0.f;
    v[k] = (row_ok && c < p.ncols) ? w[k] : 0.f;
    sc[k] = 1.f;
    rc[k] = 1.f;
    zlo[k] = 0.f;
    zhi[k] = p.maxq;
  }
}

// Scales and zero points fixed before the block (static groups, or one group
// per row) of this lane's 8 columns.  Columns and rows past the end read the
// block's last column / last row and are not used; the group indices first,
// then all scale and zero loads, so they are in flight at once.
GPTQ_DEV void load_preset(const SweepParams& p, int64_t row, bool row_ok, int t, float (&sc)[8], float (&rc)[8],
                          float (&zlo)[8], float (&zhi)[8]) {
  const int64_t rr = std::min<int64_t>(row, p.d_out - 1);
  int64_t g[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int64_t j = p.j0 + std::min(t + 16 * k, p.ncols - 1);
    g[k] = 0;
    if (p.group > 0) g[k] = (p.preset && !p.identity) ? p.perm[j] / p.group : j / p.group;
  }
  float sl[8];
  int32_t zl[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sl[k] = p.scales[g[k] * p.d_out + rr];
    zl[k] = p.zeros[g[k] * p.d_out + rr];
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (row_ok && t + 16 * k < p.ncols) {
      sc[k] = sl[k];
      rc[k] = 1.0f / sl[k];
      zlo[k] = -static_cast<float>(zl[k]);
      zhi[k] = p.maxq - static_cast<float>(zl[k]);
    }
  }
}

// After a block's sweep: every register holds the value its column was
// decided on, so the codes and errors are decided again with the same
// arithmetic (bit for bit the chain's); the normalised errors go to `e` (the
// row's block of the error panel, all 128 columns, zero past the block),
// codes q = qr + z and dequantized weights s qr to their original columns.
// Returns this lane's part of the row's loss (sum of squared normalised
// errors); er receives the errors.
// Codes and errors of a swept block, decided again from the values their
// columns were decided on (the same arithmetic as the steps); returns the
// lane's share of the row loss.
GPTQ_DEV float decide_block(const float (&v)[8], const float (&dv)[8], const float (&sc)[8], const float (&rc)[8],
                            const float (&zlo)[8], const float (&zhi)[8], float (&qr)[8], float (&er)[8]) {
  float loss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    decide(v[k], sc[k], rc[k], zlo[k], zhi[k], dv[k], qr[k], er[k]);
    loss = fmaf(er[k], er[k], loss);
  }
  return loss;
}

// codes and dequantized weights of a block, in the original column order
GPTQ_DEV void store_codes(const SweepParams& p, int64_t row, int t, const float (&qr)[8], const float (&sc)[8],
                          const float (&zlo)[8]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int c = t + 16 * k;
    if (c < p.ncols) {
      const int64_t j = p.j0 + c;
      const int64_t oc = p.identity ? j : p.perm[j];
      p.codes[row * p.d_in + oc] = static_cast<uint8_t>(qr[k] - zlo[k]);
      if (p.Q) p.Q[row * p.d_in + oc] = sc[k] * qr[k];
    }
  }
}

GPTQ_DEV float finish_block(const SweepParams& p, int64_t row, bool row_ok, int t, float* e, const float (&v)[8],
                            const float (&dv)[8], const float (&sc)[8], const float (&rc)[8],
                            const float (&zlo)[8], const float (&zhi)[8], float (&er)[8]) {
  float qr[8];
  const float loss = decide_block(v, dv, sc, rc, zlo, zhi, qr, er);
  if (!row_ok) return loss;
  if (e) {
#pragma unroll
    for (int k = 0; k < 8; ++k) e[t + 16 * k] = er[k];
  }
  store_codes(p, row, t, qr, sc, zlo);
  return loss;
}

// One block per launch.  The second block of a pair is first brought up to
// date with the first block's errors (a 128-deep product on MFMA at the start
// of its sweep).
template <int GS>
__global__ __launch_bounds__(256) void sweep_kernel(SweepParams p) {
  __shared__ __attribute__((aligned(16))) float Ut[kB * kB];
  __shared__ __attribute__((aligned(16))) float Stg[kRowsPerWG][kB + 4];  // bring-up result
  __shared__ float Dg[kB];
  const int tid = threadIdx.x;
  const int t = tid & 15, rl = tid >> 4;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerWG + rl;
  const bool row_ok = row < p.d_out;

  // the block's U and this lane's weights, all in flight at once
  float ul[64], dg[8], w[8];
  load_ublock(p, p.j0, p.ncols, tid, ul, dg);
  load_wblock(p, p.j0, p.ncols, row, t, w);
  // Bring-up of the second block of a pair: W[rows, block] -= Eb[rows, :] Uo
  // (16 rows x 128 columns, K = 128, the previous block is full) on MFMA
  // (v_mfma_f32_16x16x4_f32; MFMA step s takes k = 4 q + s in lane group q, so
  // a lane's A values are one float4 of its error row).  Wave w computes the
  // 16-column blocks 2 w and 2 w + 1; Uo goes row-major through the LDS of
  // Ut, the result through Stg.
  const bool bring = p.Eb != nullptr;
  if (bring) {
    float (*Ub)[kB] = reinterpret_cast<float (*)[kB]>(Ut);
    const int lane = tid & 63, wave = tid >> 6, m = lane & 15, q = lane >> 4;
    constexpr int kUL = kB * kB / 4 / 256;
    f32x4_t uo[kUL], ea[kB / 16];
    f32x4_t bup0 = {0.f, 0.f, 0.f, 0.f}, bup1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kUL; ++u) {
      const int e = tid + 256 * u, i = e >> 5, c4 = 4 * (e & 31);
      uo[u] = *reinterpret_cast<const f32x4_t*>(p.Uo + i * p.d_in + std::min(c4, p.ncols - 4));
    }
    const int64_t er = std::min<int64_t>(static_cast<int64_t>(blockIdx.x) * kRowsPerWG + m, p.d_out - 1);
#pragma unroll
    for (int kk = 0; kk < kB / 16; ++kk)
      ea[kk] = *reinterpret_cast<const f32x4_t*>(p.Eb + er * p.ld_err + 16 * kk + 4 * q);
#pragma unroll
    for (int u = 0; u < kUL; ++u) {
      const int e = tid + 256 * u, i = e >> 5, c4 = 4 * (e & 31);
      *reinterpret_cast<f32x4_t*>(&Ub[i][c4]) = (c4 < p.ncols) ? uo[u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kB / 16; ++kk) {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const float b0 = Ub[16 * kk + 4 * q + s4][32 * wave + m];
        const float b1 = Ub[16 * kk + 4 * q + s4][32 * wave + 16 + m];
        bup0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[kk][s4], b0, bup0, 0, 0, 0);
        bup1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[kk][s4], b1, bup1, 0, 0, 0);
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      Stg[4 * q + e][32 * wave + m] = bup0[e];
      Stg[4 * q + e][32 * wave + 16 + m] = bup1[e];
    }
    __syncthreads();  // every wave is done with Uo in Ut
  }
  store_ublock(Ut, Dg, ul, dg, p.ncols, tid);
  if (bring) {
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] -= Stg[rl][t + 16 * k];
  }
  __syncthreads();

  float v[8], sc[8], rc[8], zlo[8], zhi[8], dv[8];
  init_block(p, Dg, w, row_ok, t, v, dv, sc, rc, zlo, zhi);
  // parameters fixed before this block: static groups, one group per row, or a
  // dynamic group wider than the block that started in an earlier block
  const bool wide_group_running = !p.preset && p.group > kB && (p.j0 % p.group) != 0;
  if (p.preset || wide_group_running) load_preset(p, row, row_ok, t, sc, rc, zlo, zhi);
  // a dynamic group wider than the block starts here: range over W[row, j0 : j0+group)
  if (!p.preset && p.group > kB && (p.j0 % p.group) == 0) {
    float lo = 0.f, hi = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      lo = fminf(lo, v[k]);
      hi = fmaxf(hi, v[k]);
    }
    if (row_ok) {
      const int64_t end = std::min<int64_t>(p.j0 + p.group, p.d_in);
      for (int64_t c = p.j0 + kB + t; c < end; c += 16) {
        const float x = p.Wp[row * p.d_in + c];
        lo = fminf(lo, x);
        hi = fmaxf(hi, x);
      }
    }
    lo = row_min16(lo);
    hi = row_max16(hi);
    float s, z;
    group_params(lo, hi, p, s, z);
    const float y = 1.0f / s;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sc[k] = s;
      rc[k] = y;
      zlo[k] = -z;
      zhi[k] = p.maxq - z;
    }
    if (t == 0 && row_ok) {
      const int64_t g = p.j0 / p.group;
      p.scales[g * p.d_out + row] = s;
      p.zeros[g * p.d_out + row] = static_cast<int32_t>(z);
    }
  }

  sweep_all<GS>(p, Ut, t, v, sc, rc, zlo, zhi, row, std::make_integer_sequence<int, kB>{});
  float er[8];
  const float loss = row_sum16(finish_block(p, row, row_ok, t, p.Err + std::min<int64_t>(row, p.d_out - 1) * p.ld_err,
                                            v, dv, sc, rc, zlo, zhi, er));
  if (!row_ok) return;
  if (p.Ea) {
    // and as three bf16 planes, for the product past the group
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint16_t hh, mm, ll;
      split3(er[k], hh, mm, ll);
      const int64_t o = x3_offset(row, p.ea_col + t + 16 * k, 2 * kB * kUnitsPerGroup);
      p.Ea[o] = hh;
      p.Ea[p.ea_plane + o] = mm;
      p.Ea[2 * p.ea_plane + o] = ll;
    }
  }
  if (p.row_loss && t == 0) p.row_loss[row] = (p.j0 == 0 ? 0.f : p.row_loss[row]) + loss;
}

// One launch sweeps a whole group of kGW columns (up to 8 blocks) for 16 rows
// per workgroup, for layers whose rows fit one workgroup per CU.  The group's
// normalised errors of the workgroup's rows stay in LDS (El), and each block is
// brought up to date with the errors of the blocks before it in the group
// inside the kernel: W[rows, block] -= E[rows, j0 : jb] U[j0 : jb, block] on
// MFMA (v_mfma_f32_16x16x4_f32, A = errors from El, B = rows of U straight
// from memory).  This replaces the per-block launches and the products inside
// a group; the product past the group stays one GEMM per group.  The sum is
// the lazy-batch sweep's, taken in another order.  Only groups that fit inside
// a block (or parameters fixed before the sweep) are handled here.
//
// 512 threads: waves 0-3 sweep (the chain of a block is bound by the latency
// of its dependent operations, with one chain wave per SIMD), waves 4-7
// produce.  While the chain waves sweep block b, the producer waves bring
// block b + 1 up to date with the errors of blocks 0 .. b - 1 on the same
// SIMDs' matrix cores and load its U and weights; once block b is swept they
// add its own errors (K = 128), stage the weights and the block's U in LDS,
// and the chain waves go on.  Two workgroup barriers a block, in the same
// order on both sides: A(b) (block b staged) and B(b) (block b swept).
constexpr int kGW = 2 * kB * kUnitsPerGroup;  // columns per group
constexpr int kELd = kGW + 4;                 // El row stride in floats
constexpr int kWnLd = kB + 4;                 // staged weights: row stride in floats
// error of (row r, group column k): four consecutive MFMA k-steps of lane
// group q = k & 3 are one float4
GPTQ_DEV int el_index(int r, int k) { return r * kELd + (k & 3) * (kGW / 4) + (k >> 2); }

// Producer side of the bring-up of block jb from the group errors of columns
// [k0, k0 + 128 n) (El, k relative to the group start g0): acc[h] += E U for
// the wave's two 16-column tiles h.  MFMA k-step s takes k = 4 s + q in lane
// group q: A = El (row m, k), B = U[g0 + k][jb + column m of the tile].  Rows
// of U go through a ring of kRing register sets, four k-steps each.
GPTQ_DEV void bring_up(const SweepParams& p, const float* El, int64_t g0, int64_t jb, int ncols, int k0, int n,
                       int pw, int m, int q, f32x4_t& acc0, f32x4_t& acc1) {
  const int ca = std::min(32 * pw + m, ncols - 1), cb = std::min(32 * pw + 16 + m, ncols - 1);
  const float* ua = p.U + (g0 + k0 + q) * p.d_in + jb + ca;
  const float* ub = p.U + (g0 + k0 + q) * p.d_in + jb + cb;
  const int64_t kstep = 4 * p.d_in;  // one MFMA k-step down U
  const int nit = 8 * n;             // iterations of four k-steps, a multiple of kRing
  constexpr int kRing = 4;
  float ra[kRing][4], rb[kRing][4];
  auto fetch = [&](int it, float (&da)[4], float (&db)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t off = (4 * static_cast<int64_t>(it) + e) * kstep;
      da[e] = ua[off];
      db[e] = ub[off];
    }
  };
#pragma unroll
  for (int d = 0; d < kRing - 1; ++d) fetch(d, ra[d], rb[d]);
  const float* ea = El + m * kELd + q * (kGW / 4) + k0 / 4;
  f32x4_t an = *reinterpret_cast<const f32x4_t*>(ea);
  for (int it0 = 0; it0 < nit; it0 += kRing) {
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
      const int it = it0 + d;
      // past the end the ring refetches the last rows (unused): no branch, so
      // the loads stay in flight across the loop's back edge; the errors of
      // the next step are read one step early as well
      fetch(std::min(it + kRing - 1, nit - 1), ra[(d + kRing - 1) % kRing], rb[(d + kRing - 1) % kRing]);
      const f32x4_t a = an;
      an = *reinterpret_cast<const f32x4_t*>(ea + 4 * std::min(it + 1, nit - 1));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], ra[d][e], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], rb[d][e], acc1, 0, 0, 0);
      }
      // keep the ring in program order: this step's loads stay behind the
      // earlier steps' products, so each set lands kRing - 1 steps early
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The last 128 k of a bring-up (the block just swept), split: its rows of U
// are read before that block's sweep ends (tail_fetch), the products run once
// its errors are in El (tail_mfma).
GPTQ_DEV void tail_fetch(const SweepParams& p, int64_t g0, int64_t jb, int ncols, int k0, int pw, int m, int q,
                         float (&tb)[32][2]) {
  const int ca = std::min(32 * pw + m, ncols - 1), cb = std::min(32 * pw + 16 + m, ncols - 1);
  const float* src = p.U + (g0 + k0 + q) * p.d_in + jb;
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    tb[s][0] = src[4 * s * p.d_in + ca];
    tb[s][1] = src[4 * s * p.d_in + cb];
  }
}

GPTQ_DEV void tail_mfma(const float* El, int k0, int m, int q, const float (&tb)[32][2], f32x4_t& acc0,
                        f32x4_t& acc1) {
  const float* ea = El + m * kELd + q * (kGW / 4) + k0 / 4;
  f32x4_t a[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = *reinterpret_cast<const f32x4_t*>(ea + 4 * j);
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s >> 2][s & 3], tb[s][0], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s >> 2][s & 3], tb[s][1], acc1, 0, 0, 0);
  }
}

template <int GS>
__global__ __launch_bounds__(512) void sweep_group_kernel(SweepParams p) {
  __shared__ __attribute__((aligned(16))) float Ut[kB * kB];
  __shared__ __attribute__((aligned(16))) float El[kRowsPerWG * kELd];
  __shared__ __attribute__((aligned(16))) float Wn[kRowsPerWG * kWnLd];
  __shared__ float Dg[kB];
  const int64_t g0 = p.j0;
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kRowsPerWG;
  auto block_cols = [&](int b) { return static_cast<int>(std::min<int64_t>(kB, p.d_in - g0 - int64_t{kB} * b)); };

  if (threadIdx.x >= 256) {
    // ------------------------------------------------------------ producers
    const int pt = threadIdx.x - 256;
    const int pw = pt >> 6, lane = pt & 63, m = lane & 15, q = lane >> 4;
    // weights in the MFMA output layout: tile h, element e = row 4 q + e,
    // column 32 pw + 16 h + m of the block
    auto load_w = [&](int64_t jb, int ncols, float (&wv)[2][4]) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t r = std::min<int64_t>(row0 + 4 * q + e, p.d_out - 1);
          wv[h][e] = p.Wp[r * p.d_in + jb + std::min(32 * pw + 16 * h + m, ncols - 1)];
        }
    };
    auto stage_w = [&](const float (&wv)[2][4], const f32x4_t& acc0, const f32x4_t& acc1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Wn[(4 * q + e) * kWnLd + 32 * pw + m] = wv[0][e] - acc0[e];
        Wn[(4 * q + e) * kWnLd + 32 * pw + 16 + m] = wv[1][e] - acc1[e];
      }
    };
    {
      float ul[64], dg[8], wv[2][4];
      const int nc = block_cols(0);
      load_ublock(p, g0, nc, pt, ul, dg);
      load_w(g0, nc, wv);
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      stage_w(wv, z, z);
      store_ublock(Ut, Dg, ul, dg, nc, pt);
    }
    for (int b = 0; b < p.nblk; ++b) {
      __syncthreads();  // A(b): block b staged
      const bool next = b + 1 < p.nblk;
      const int64_t jn = g0 + int64_t{kB} * (b + 1);
      const int nc = next ? block_cols(b + 1) : kB;
      float ul[64], dg[8], wv[2][4], tb[32][2];
      f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
      if (next) {
        load_ublock(p, jn, nc, pt, ul, dg);
        load_w(jn, nc, wv);
        tail_fetch(p, g0, jn, nc, kB * b, pw, m, q, tb);
        if (b > 0) bring_up(p, El, g0, jn, nc, 0, b, pw, m, q, acc0, acc1);  // blocks 0 .. b - 1
        scale_ublock(ul, dg, nc, pt);
      }
      __syncthreads();  // B(b): block b swept, its errors in El, Ut free
      if (next) {
        tail_mfma(El, kB * b, m, q, tb, acc0, acc1);  // block b
        stage_w(wv, acc0, acc1);
        write_ublock(Ut, Dg, ul, dg, nc, pt);
      }
    }
    return;
  }

  // ---------------------------------------------------------------- chain
  const int tid = threadIdx.x;
  const int t = tid & 15, rl = tid >> 4;
  const int64_t row = row0 + rl;
  const bool row_ok = row < p.d_out;
  float loss = 0.f;
  for (int b = 0; b < p.nblk; ++b) {
    SweepParams pb = p;
    pb.j0 = g0 + int64_t{kB} * b;
    pb.ncols = block_cols(b);
    __syncthreads();  // A(b)
    float w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = Wn[rl * kWnLd + t + 16 * k];
    float v[8], sc[8], rc[8], zlo[8], zhi[8], dv[8];
    init_block(pb, Dg, w, row_ok, t, v, dv, sc, rc, zlo, zhi);
    if (p.preset) load_preset(pb, row, row_ok, t, sc, rc, zlo, zhi);

    sweep_all<GS>(pb, Ut, t, v, sc, rc, zlo, zhi, row, std::make_integer_sequence<int, kB>{});

    // errors to El (for the next blocks' bring-up; rows past the end keep
    // finite zeros); the stores to memory wait until after the barrier,
    // beside the producers' part of the next block's bring-up
    const int kb = kB * b;
    float er[8], qr[8];
    loss += decide_block(v, dv, sc, rc, zlo, zhi, qr, er);
#pragma unroll
    for (int k = 0; k < 8; ++k) El[el_index(rl, kb + t + 16 * k)] = er[k];
    __syncthreads();  // B(b)
    if (row_ok) {
      store_codes(pb, row, t, qr, sc, zlo);
      // the errors as three bf16 planes of the group's panel, for the
      // product past the group
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        uint16_t hh, mm, ll;
        split3(er[k], hh, mm, ll);
        const int64_t o = x3_offset(row, kb + t + 16 * k, kGW);
        p.Ea[o] = hh;
        p.Ea[p.ea_plane + o] = mm;
        p.Ea[2 * p.ea_plane + o] = ll;
      }
    }
  }
  loss = row_sum16(loss);
  if (row_ok && p.row_loss && t == 0) p.row_loss[row] = (g0 == 0 ? 0.f : p.row_loss[row]) + loss;
}

// Wp[r][i] = W[r][perm[i]] in fp32.
// Without act-order the working copy is W converted to fp32: eight values a
// thread, 16-byte loads and stores (W 16-byte aligned).
__global__ void convert_w_kernel(const void* W, int w_bf16, int64_t total, float* Wp) {
  const int64_t n8 = total / 8;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t t0 = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  for (int64_t v = t0; v < n8; v += stride) {
    f32x4_t a, b;
    if (w_bf16) {
      const u32x4_t q = reinterpret_cast<const u32x4_t*>(W)[v];
      a = f32x4_t{__uint_as_float(q[0] << 16), __uint_as_float(q[0] & 0xFFFF0000u), __uint_as_float(q[1] << 16),
                  __uint_as_float(q[1] & 0xFFFF0000u)};
      b = f32x4_t{__uint_as_float(q[2] << 16), __uint_as_float(q[2] & 0xFFFF0000u), __uint_as_float(q[3] << 16),
                  __uint_as_float(q[3] & 0xFFFF0000u)};
    } else {
      a = reinterpret_cast<const f32x4_t*>(W)[2 * v];
      b = reinterpret_cast<const f32x4_t*>(W)[2 * v + 1];
    }
    reinterpret_cast<f32x4_t*>(Wp)[2 * v] = a;
    reinterpret_cast<f32x4_t*>(Wp)[2 * v + 1] = b;
  }
  for (int64_t e = 8 * n8 + t0; e < total; e += stride)
    Wp[e] = w_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(W)[e]) : static_cast<const float*>(W)[e];
}

__global__ void gather_w_kernel(const void* W, int w_bf16, int64_t d_out, int64_t d_in, const int32_t* perm,
                                int identity, float* Wp) {
  const int64_t total = d_out * d_in;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t r = e / d_in, i = e - r * d_in;
    const int64_t c = identity ? i : perm[i];
    const int64_t src = r * d_in + c;
    Wp[e] = w_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(W)[src]) : static_cast<const float*>(W)[src];
  }
}

// Group parameters from the original weights: static groups (original column
// groups) or one group per row.  One wave per (group, row).
__global__ __launch_bounds__(256) void static_params_kernel(const void* W, int w_bf16, int64_t d_out,
                                                            int64_t d_in, int group, int n_groups, int bits,
                                                            int sym, float* scales, int32_t* zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x) >> 6;
  const int64_t nwaves = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 6;
  const int64_t pairs = static_cast<int64_t>(n_groups) * d_out;
  for (int64_t pr = wave; pr < pairs; pr += nwaves) {
    const int64_t g = pr / d_out, row = pr - g * d_out;
    const int64_t c_begin = (group > 0) ? g * group : 0;
    const int64_t c_end = (group > 0) ? std::min<int64_t>(d_in, c_begin + group) : d_in;
    float lo = 0.f, hi = 0.f;
    for (int64_t c = c_begin + lane; c < c_end; c += 64) {
      const int64_t src = row * d_in + c;
      const float x = w_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(W)[src]) : static_cast<const float*>(W)[src];
      lo = fminf(lo, x);
      hi = fmaxf(hi, x);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, off));
      hi = fmaxf(hi, __shfl_xor(hi, off));
    }
    if (lane == 0) {
      SweepParams p{};
      p.sym = sym;
      p.bits = bits;
      p.maxq = static_cast<float>((1 << bits) - 1);
      float s, z;
      group_params(lo, hi, p, s, z);
      scales[g * d_out + row] = s;
      zeros[g * d_out + row] = static_cast<int32_t>(z);
    }
  }
}

__global__ void g_idx_kernel(int64_t d_in, int group, int by_position, const int32_t* perm, int32_t* g_idx) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < d_in;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    if (group <= 0)
      g_idx[i] = 0;
    else if (by_position)
      g_idx[perm[i]] = static_cast<int32_t>(i / group);  // dynamic groups follow the sweep order
    else
      g_idx[i] = static_cast<int32_t>(i / group);
  }
}

int grid_for(int64_t total) {
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 8192)));
}

}  // namespace

bool quant_planes(int group_size, bool static_groups) {
  const int group = group_size > 0 ? group_size : 0;
  const bool preset = static_groups || group == 0;
  const bool pair = preset || group <= kB || group % (2 * kB) == 0;
  return pair && (preset || group <= 2 * kB || group % (2 * kB * kUnitsPerGroup) == 0);
}

bool group_launch(int group_size, bool static_groups) {
  const int group = group_size > 0 ? group_size : 0;
  const bool preset = static_groups || group == 0;
  return preset || group <= kB;
}

QuantLayout quant_layout(int64_t d_out, int64_t d_in, bool planes) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  QuantLayout L{};
  L.off_wp = 0;
  L.off_err = up(static_cast<size_t>(d_out) * d_in * sizeof(float));
  L.ws_bytes = L.off_err + up(static_cast<size_t>(d_out) * 2 * kB * kUnitsPerGroup * sizeof(float));
  if (planes) {
    // the group's errors and the transposed rows of U past the group, three
    // bf16 planes each, for the product on the bf16 matrix cores
    L.off_ea = L.ws_bytes;
    L.ws_bytes += up(3 * static_cast<size_t>(x3_plane_elems(d_out, kGW)) * sizeof(uint16_t));
    L.off_bt = L.ws_bytes;
    L.ws_bytes += up(3 * static_cast<size_t>(x3_plane_elems(d_in, kGW)) * sizeof(uint16_t));
  }
  return L;
}

hipError_t quantize_launch(const void* W, bool w_bf16, int64_t d_out, int64_t d_in, const float* U,
                           const int32_t* perm, int bits, int group_size, bool sym, bool static_groups,
                           uint8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx, float* Q,
                           float* row_loss, void* ws, hipStream_t st, bool identity) {
  const bool by_group = group_launch(group_size, static_groups);
  const QuantLayout lay = quant_layout(d_out, d_in, quant_planes(group_size, static_groups));
  float* Wp = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.off_wp);
  float* Err = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.off_err);
  const int group = group_size > 0 ? group_size : 0;
  const int n_groups = group > 0 ? static_cast<int>((d_in + group - 1) / group) : 1;
  const bool preset = static_groups || group == 0;

  hipError_t e;
  {
    PhaseScope ph(kPhQuantElem, st);
    if (identity && reinterpret_cast<uintptr_t>(W) % 16 == 0)
      convert_w_kernel<<<grid_for((d_out * d_in + 7) / 8), 256, 0, st>>>(W, w_bf16 ? 1 : 0, d_out * d_in, Wp);
    else
      gather_w_kernel<<<grid_for(d_out * d_in), 256, 0, st>>>(W, w_bf16 ? 1 : 0, d_out, d_in, perm,
                                                              identity ? 1 : 0, Wp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (preset) {
      const int64_t pairs = static_cast<int64_t>(n_groups) * d_out;
      const int blocks = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>((pairs + 3) / 4, 16384)));
      static_params_kernel<<<blocks, 256, 0, st>>>(W, w_bf16 ? 1 : 0, d_out, d_in, group, n_groups, bits,
                                                   sym ? 1 : 0, scales, zeros);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    g_idx_kernel<<<grid_for(d_in), 256, 0, st>>>(d_in, group, (!preset && !identity) ? 1 : 0, perm, g_idx);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }

  SweepParams p{};
  p.Wp = Wp;
  p.U = U;
  p.perm = perm;
  p.codes = codes;
  p.Q = Q;
  p.scales = scales;
  p.zeros = zeros;
  p.row_loss = row_loss;
  p.Err = Err;
  p.d_out = d_out;
  p.d_in = d_in;
  p.bits = bits;
  p.maxq = static_cast<float>((1 << bits) - 1);
  p.group = group;
  p.sym = sym ? 1 : 0;
  p.preset = preset ? 1 : 0;
  p.identity = identity ? 1 : 0;
  const int blocks = static_cast<int>((d_out + kRowsPerWG - 1) / kRowsPerWG);
  // Blocks are swept in units of two (pairs): the second block of a pair is
  // first brought up to date with the first block's errors (a 128-deep
  // product at the start of its sweep kernel).  Two pairs form a group: the
  // second pair's columns are first brought up to date with the first pair's
  // errors (one d_out x 256 product, K = 256), and the trailing update of the
  // columns past the group runs once per group (K = 512), so it reads and
  // writes the rest of W once per 512 columns.  The result is the lazy-batch
  // sweep's (the same products, summed in another order).  A dynamic group
  // wider than a block reads columns past the block at its start, so units and
  // groups are used only when such groups start on their boundaries: pairs for
  // groups of 256 columns or a multiple, groups of pairs for groups up to 256
  // or a multiple of 512.
  // Groups inside a block or fixed before the sweep: one launch per group of
  // 1024 columns, the products inside the group on MFMA in the kernel (the
  // sweep is latency-bound, so launches cost as much as the sweep; measured
  // faster than the per-block launches below from 4096 to 22016 rows).
  const int gs = (!preset && group <= kB) ? group : 0;
  if (by_group) {
    p.ld_err = kGW;
    p.Eb = nullptr;
    p.Uo = nullptr;
    p.Err = Err;
    p.Ea = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + lay.off_ea);
    p.ea_plane = x3_plane_elems(d_out, kGW);
    uint16_t* Bt = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + lay.off_bt);
    for (int64_t g0 = 0; g0 < d_in; g0 += kGW) {
      p.j0 = g0;
      p.nblk = static_cast<int>(std::min<int64_t>(kGW / kB, (d_in - g0 + kB - 1) / kB));
      p.ncols = static_cast<int>(std::min<int64_t>(kB, d_in - g0));
      {
        PhaseScope ph(kPhSweep, st);
        switch (gs) {
          case 0: sweep_group_kernel<0><<<blocks, 512, 0, st>>>(p); break;
          case 1: sweep_group_kernel<1><<<blocks, 512, 0, st>>>(p); break;
          case 2: sweep_group_kernel<2><<<blocks, 512, 0, st>>>(p); break;
          case 4: sweep_group_kernel<4><<<blocks, 512, 0, st>>>(p); break;
          case 8: sweep_group_kernel<8><<<blocks, 512, 0, st>>>(p); break;
          case 16: sweep_group_kernel<16><<<blocks, 512, 0, st>>>(p); break;
          case 32: sweep_group_kernel<32><<<blocks, 512, 0, st>>>(p); break;
          case 64: sweep_group_kernel<64><<<blocks, 512, 0, st>>>(p); break;
          case 128: sweep_group_kernel<128><<<blocks, 512, 0, st>>>(p); break;
          default: return hipErrorInvalidValue;  // the ABI admits only groups dividing 128 here
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      // the columns past the group: W[:, c0:] -= E U[g0 : g0 + kGW, c0:] on the
      // bf16 matrix cores (three-part split of both operands)
      const int64_t rest = d_in - g0 - kGW;
      if (rest > 0) {
        PhaseScope ph(kPhUpdate, st);
        const int64_t c0 = g0 + kGW;
        if ((e = split3_t(U + g0 * d_in + c0, d_in, kGW, rest, Bt, st)) != hipSuccess) return e;
        e = gemm_x3(d_out, rest, kGW, -1.f, p.Ea, p.ea_plane, Bt, x3_plane_elems(rest, kGW), Wp + c0, d_in, st);
        if (e != hipSuccess) return e;
      }
    }
    return hipSuccess;
  }

  const bool pair = preset || group <= kB || group % (2 * kB) == 0;
  const int SB = pair ? 2 * kB : kB;
  const bool grouped = pair && (preset || group <= 2 * kB || group % (2 * kB * kUnitsPerGroup) == 0);
  const int NU = grouped ? kUnitsPerGroup : 1;  // units per trailing update
  const int64_t GW = static_cast<int64_t>(NU) * SB;
  p.ld_err = static_cast<int>(GW);
  p.nblk = 1;
  // groups of kGW columns: the product past each group on the bf16 matrix
  // cores (the sweep kernels also write the errors as planes)
  const bool planes = GW == kGW;
  uint16_t* Bt = planes ? reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + lay.off_bt) : nullptr;
  p.Ea = planes ? reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + lay.off_ea) : nullptr;
  p.ea_plane = x3_plane_elems(d_out, kGW);
  for (int64_t g0 = 0; g0 < d_in; g0 += GW) {
    for (int u = 0; u < NU; ++u) {
      const int64_t j0 = g0 + static_cast<int64_t>(u) * SB;
      if (j0 >= d_in) break;
      if (u > 0) {
        // the unit's columns take the group's earlier units' errors
        const int64_t w = std::min<int64_t>(SB, d_in - j0);
        PhaseScope ph(kPhUpdate, st);
        e = gemm_f32(d_out, w, j0 - g0, -1.f, Err, GW, 0, U + g0 * d_in + j0, d_in, 0, false, 1.f, Wp + j0, d_in, 0, 1,
                     false, 0, st);
        if (e != hipSuccess) return e;
      }
      for (int h = 0; h < SB / kB; ++h) {
        const int64_t jb = j0 + static_cast<int64_t>(h) * kB;
        if (jb >= d_in) break;
        const int ncols = static_cast<int>(std::min<int64_t>(kB, d_in - jb));
        // the second block of a pair is brought up to date inside its sweep
        p.Eb = (h > 0) ? Err + u * SB : nullptr;
        p.Uo = (h > 0) ? U + j0 * d_in + jb : nullptr;
        p.j0 = jb;
        p.ncols = ncols;
        p.Err = Err + u * SB + h * kB;
        p.ea_col = u * SB + h * kB;
        PhaseScope ph(kPhSweep, st);
        switch (gs) {
          case 0: sweep_kernel<0><<<blocks, 256, 0, st>>>(p); break;
          case 1: sweep_kernel<1><<<blocks, 256, 0, st>>>(p); break;
          case 2: sweep_kernel<2><<<blocks, 256, 0, st>>>(p); break;
          case 4: sweep_kernel<4><<<blocks, 256, 0, st>>>(p); break;
          case 8: sweep_kernel<8><<<blocks, 256, 0, st>>>(p); break;
          case 16: sweep_kernel<16><<<blocks, 256, 0, st>>>(p); break;
          case 32: sweep_kernel<32><<<blocks, 256, 0, st>>>(p); break;
          case 64: sweep_kernel<64><<<blocks, 256, 0, st>>>(p); break;
          case 128: sweep_kernel<128><<<blocks, 256, 0, st>>>(p); break;
          default: return hipErrorInvalidValue;  // the ABI admits only groups dividing 128 here
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
    }
    const int64_t rest = d_in - g0 - GW;
    if (rest > 0) {
      PhaseScope ph(kPhUpdate, st);
      const int64_t c0 = g0 + GW;
      if (planes) {
        if ((e = split3_t(U + g0 * d_in + c0, d_in, kGW, rest, Bt, st)) != hipSuccess) return e;
        e = gemm_x3(d_out, rest, kGW, -1.f, p.Ea, p.ea_plane, Bt, x3_plane_elems(rest, kGW), Wp + c0, d_in, st);
      } else {
        e = gemm_f32(d_out, rest, GW, -1.f, Err, GW, 0, U + g0 * d_in + c0, d_in, 0, false, 1.f, Wp + c0, d_in, 0, 1,
                     false, 0, st);
      }
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace gptq
