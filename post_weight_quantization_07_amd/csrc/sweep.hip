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
// output row, lane t owning block columns 8t .. 8t+7 in registers.  At step i
// every lane quantizes its own copy of register i%8, the owner lane's error is
// broadcast to its row with DPP row_newbcast, and every lane applies the
// rank-1 update to its 8 columns with U[i][8t .. 8t+7] read from LDS (zeros
// left of the diagonal make the update uniform).  Group ranges reduce over the
// 16-lane row with DPP mirrors.
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

// GS > 0: dynamic groups of GS columns start inside the block (GS divides
// 128), so the range code is emitted only at steps I % GS == 0; GS == 0: every
// column's parameters are known before the block.  Keeping the code of the
// 128 unrolled steps small matters: it has to stay in the instruction cache.
template <int GS, int I>
GPTQ_DEV void sweep_step(const SweepParams& p, const float (*Ub)[kB], const float (&dv)[8], int t,
                         float (&v)[8], float (&sc)[8], float (&rc)[8], float (&zlo)[8], float (&zhi)[8],
                         float (&qc)[8], float (&er)[8], int64_t row, f32x4_t (&ua)[2],
                         f32x4_t (&ub)[2]) {
  constexpr int r = I & 7, owner = I >> 3;
  // the next step's row of U is read now (two register sets), so its LDS
  // latency hides behind this whole step
  if constexpr (I + 1 < kB) {
    ua[(I + 1) & 1] = *reinterpret_cast<const f32x4_t*>(&Ub[I + 1][8 * t]);
    ub[(I + 1) & 1] = *reinterpret_cast<const f32x4_t*>(&Ub[I + 1][8 * t + 4]);
  }
  const f32x4_t u0 = ua[I & 1], u1 = ub[I & 1];
  // dynamic groups that start inside the block: range over the group's current values
  if constexpr (GS > 0 && (I % GS) == 0) {
    if (I < p.ncols) {
      float lo = 0.f, hi = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = 8 * t + k;
        const bool in = (c >= I) && (c < I + GS) && (c < p.ncols);
        lo = in ? fminf(lo, v[k]) : lo;
        hi = in ? fmaxf(hi, v[k]) : hi;
      }
      if constexpr (GS > 8) {  // the group spans several lanes of the row
        lo = row_min16(lo);
        hi = row_max16(hi);
      }
      float s, z;
      group_params(lo, hi, p, s, z);
      const float y = 1.0f / s;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = 8 * t + k;
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
  const float w = v[r];
  const float s = sc[r];
  // w / s correctly rounded from the correctly rounded reciprocal y = 1 / s:
  // q0 = w y is within an ulp, the remainder w - s q0 is exact in one fma, and
  // q0 + (w - s q0) y rounds to the quotient (Markstein's correction step).
  // Three dependent operations instead of the division sequence.
  const float y = rc[r];
  const float q0 = w * y;
  const float quot = fmaf(fmaf(-s, q0, w), y, q0);
  // the code relative to the zero point, qr = q - z: rint(w / s) clamped to
  // [-z, maxq - z] is clamp(rint(w / s) + z, 0, maxq) - z exactly (integers);
  // the dequantized weight is s qr and the error w - s qr (one fma)
  const float qr = __builtin_amdgcn_fmed3f(rintf(quot), zlo[r], zhi[r]);
  const float err = fmaf(-s, qr, w) * dv[r];
  const float eb = row_bcast<owner>(err);
  qc[r] = (t == owner) ? qr : qc[r];
  er[r] = (t == owner) ? eb : er[r];
  // materialise the selects here: left alone, the compiler sinks them to the
  // end of the block and keeps every step's code alive until then
  asm volatile("" : "+v"(qc[r]), "+v"(er[r]));
  // the next column first: the next step's decision waits on it
  constexpr int rn = (I + 1) & 7;
  v[rn] = fmaf(-eb, rn < 4 ? u0[rn & 3] : u1[rn & 3], v[rn]);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (k != rn) v[k] = fmaf(-eb, u0[k], v[k]);
    if (k + 4 != rn) v[k + 4] = fmaf(-eb, u1[k], v[k + 4]);
  }
  // keep each step a scheduling region of its own (bounded register pressure)
  __builtin_amdgcn_sched_barrier(0);
}

template <int GS, int... Is>
GPTQ_DEV void sweep_all(const SweepParams& p, const float (*Ub)[kB], const float (&dv)[8], int t, float (&v)[8],
                        float (&sc)[8], float (&rc)[8], float (&zlo)[8], float (&zhi)[8], float (&qc)[8],
                        float (&er)[8], int64_t row, std::integer_sequence<int, Is...>) {
  f32x4_t ua[2], ub[2];
  ua[0] = *reinterpret_cast<const f32x4_t*>(&Ub[0][8 * t]);
  ub[0] = *reinterpret_cast<const f32x4_t*>(&Ub[0][8 * t + 4]);
  (sweep_step<GS, Is>(p, Ub, dv, t, v, sc, rc, zlo, zhi, qc, er, row, ua, ub), ...);
}

template <int GS>
__global__ __launch_bounds__(256) void sweep_kernel(SweepParams p) {
  __shared__ __attribute__((aligned(16))) float Ub[kB][kB];
  __shared__ __attribute__((aligned(16))) float Stg[kRowsPerWG][kB + 4];  // bring-up result
  const int tid = threadIdx.x;
  const int t = tid & 15;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerWG + (tid >> 4);
  const bool row_ok = row < p.d_out;

  // The diagonal block of U (zeros outside the block's columns) and this
  // lane's 8 weights.  Every load reads an in-range address (the block width
  // is a multiple of 4; rows and columns past the end are clamped) and the
  // value is selected after, so all of them are in flight at once.
  constexpr int kUL = kB * kB / 4 / 256;  // float4 of the U block per thread
  const int c0 = 8 * t;
  f32x4_t ul[kUL], wa, wb;
#pragma unroll
  for (int u = 0; u < kUL; ++u) {
    const int e = tid + 256 * u, i = e >> 5, c4 = 4 * (e & 31);
    const int ic = std::min(i, p.ncols - 1), cc = std::min(c4, p.ncols - 4);
    ul[u] = *reinterpret_cast<const f32x4_t*>(p.U + (p.j0 + ic) * p.d_in + p.j0 + cc);
  }
  {
    const float* src = p.Wp + std::min<int64_t>(row, p.d_out - 1) * p.d_in + p.j0;
    wa = *reinterpret_cast<const f32x4_t*>(src + std::min(c0, p.ncols - 4));
    wb = *reinterpret_cast<const f32x4_t*>(src + std::min(c0 + 4, p.ncols - 4));
  }
  // Bring-up of the second block of a pair: W[rows, block] -= Eb[rows, :] Uo
  // (16 rows x 128 columns, K = 128, the previous block is full) on MFMA
  // (v_mfma_f32_16x16x4_f32; MFMA step s takes k = 4 q + s in lane group q, so
  // a lane's A values are one float4 of its error row).  Wave w computes the
  // 16-column blocks 2 w and 2 w + 1; Uo goes through Ub, the result through
  // Stg into the lanes' column layout.
  const bool bring = p.Eb != nullptr;
  f32x4_t bup0 = {0.f, 0.f, 0.f, 0.f}, bup1 = {0.f, 0.f, 0.f, 0.f};
  if (bring) {
    const int lane = tid & 63, wave = tid >> 6, m = lane & 15, q = lane >> 4;
    f32x4_t uo[kUL], ea[kB / 16];
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
    __syncthreads();  // every wave is done with Uo in Ub
  }
#pragma unroll
  for (int u = 0; u < kUL; ++u) {
    const int e = tid + 256 * u, i = e >> 5, c4 = 4 * (e & 31);
    *reinterpret_cast<f32x4_t*>(&Ub[i][c4]) = (i < p.ncols && c4 < p.ncols) ? ul[u] : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  if (bring) {
    const f32x4_t d0 = *reinterpret_cast<const f32x4_t*>(&Stg[tid >> 4][c0]);
    const f32x4_t d1 = *reinterpret_cast<const f32x4_t*>(&Stg[tid >> 4][c0 + 4]);
    wa -= d0;
    wb -= d1;
  }
  __syncthreads();

  // zlo, zhi: the clamp bounds -z and maxq - z of each column's relative code
  float v[8], sc[8], rc[8], zlo[8], zhi[8], qc[8], er[8], dv[8];
  // 1 / U[i][i] of this lane's own columns (only the owner of a column uses it)
#pragma unroll
  for (int k = 0; k < 8; ++k) dv[k] = (c0 + k < p.ncols) ? 1.0f / Ub[c0 + k][c0 + k] : 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[k] = (row_ok && c0 < p.ncols) ? wa[k] : 0.f;
    v[k + 4] = (row_ok && c0 + 4 < p.ncols) ? wb[k] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    sc[k] = 1.f;
    rc[k] = 1.f;
    zlo[k] = 0.f;
    zhi[k] = p.maxq;
    qc[k] = 0.f;
    er[k] = 0.f;
  }
  // parameters fixed before this block: static groups, one group per row, or a
  // dynamic group wider than the block that started in an earlier block
  const bool wide_group_running = !p.preset && p.group > kB && (p.j0 % p.group) != 0;
  if (p.preset || wide_group_running) {
    // columns and rows past the end read the block's last column / last row
    // and are not used; the group indices first, then all scale and zero loads
    const int64_t rr = std::min<int64_t>(row, p.d_out - 1);
    int64_t g[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t j = p.j0 + std::min(c0 + k, p.ncols - 1);
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
      if (row_ok && c0 + k < p.ncols) {
        sc[k] = sl[k];
        rc[k] = 1.0f / sl[k];
        zlo[k] = -static_cast<float>(zl[k]);
        zhi[k] = p.maxq - static_cast<float>(zl[k]);
      }
    }
  }
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
  __syncthreads();

  sweep_all<GS>(p, Ub, dv, t, v, sc, rc, zlo, zhi, qc, er, row, std::make_integer_sequence<int, kB>{});
  // codes q = qr + z, dequantized weights s qr, and the row's loss (sum of the
  // squared normalised errors over the row's 16 lanes)
  float qv[8], loss = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    qv[k] = sc[k] * qc[k];
    qc[k] -= zlo[k];
    loss = fmaf(er[k], er[k], loss);
  }
  loss = row_sum16(loss);

  if (!row_ok) return;
  // normalised errors of the block, for the trailing update
  float* e = p.Err + row * p.ld_err + c0;
  *reinterpret_cast<f32x4_t*>(e) = f32x4_t{er[0], er[1], er[2], er[3]};
  *reinterpret_cast<f32x4_t*>(e + 4) = f32x4_t{er[4], er[5], er[6], er[7]};
  // codes and dequantized weights, written in original column order
  if (p.identity && c0 + 8 <= p.ncols) {
    const int64_t base = row * p.d_in + p.j0 + c0;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo |= static_cast<uint32_t>(qc[k]) << (8 * k);
      hi |= static_cast<uint32_t>(qc[k + 4]) << (8 * k);
    }
    *reinterpret_cast<uint2*>(p.codes + base) = make_uint2(lo, hi);
    if (p.Q) {
      *reinterpret_cast<f32x4_t*>(p.Q + base) = f32x4_t{qv[0], qv[1], qv[2], qv[3]};
      *reinterpret_cast<f32x4_t*>(p.Q + base + 4) = f32x4_t{qv[4], qv[5], qv[6], qv[7]};
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (c0 + k < p.ncols) {
        const int64_t j = p.j0 + c0 + k;
        const int64_t oc = p.identity ? j : p.perm[j];
        p.codes[row * p.d_in + oc] = static_cast<uint8_t>(qc[k]);
        if (p.Q) p.Q[row * p.d_in + oc] = qv[k];
      }
    }
  }
  if (p.row_loss && t == 0) p.row_loss[row] = (p.j0 == 0 ? 0.f : p.row_loss[row]) + loss;
}

// Wp[r][i] = W[r][perm[i]] in fp32.
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

QuantLayout quant_layout(int64_t d_out, int64_t d_in) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  QuantLayout L{};
  L.off_wp = 0;
  L.off_err = up(static_cast<size_t>(d_out) * d_in * sizeof(float));
  L.ws_bytes = L.off_err + up(static_cast<size_t>(d_out) * 2 * kB * kUnitsPerGroup * sizeof(float));
  return L;
}

hipError_t quantize_launch(const void* W, bool w_bf16, int64_t d_out, int64_t d_in, const float* U,
                           const int32_t* perm, int bits, int group_size, bool sym, bool static_groups,
                           uint8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx, float* Q,
                           float* row_loss, void* ws, hipStream_t st, bool identity) {
  const QuantLayout lay = quant_layout(d_out, d_in);
  float* Wp = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.off_wp);
  float* Err = reinterpret_cast<float*>(static_cast<char*>(ws) + lay.off_err);
  const int group = group_size > 0 ? group_size : 0;
  const int n_groups = group > 0 ? static_cast<int>((d_in + group - 1) / group) : 1;
  const bool preset = static_groups || group == 0;

  hipError_t e;
  {
    PhaseScope ph(kPhQuantElem, st);
    gather_w_kernel<<<grid_for(d_out * d_in), 256, 0, st>>>(W, w_bf16 ? 1 : 0, d_out, d_in, perm, identity ? 1 : 0,
                                                            Wp);
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
  const bool pair = preset || group <= kB || group % (2 * kB) == 0;
  const int SB = pair ? 2 * kB : kB;
  const bool grouped = pair && (preset || group <= 2 * kB || group % (2 * kB * kUnitsPerGroup) == 0);
  const int NU = grouped ? kUnitsPerGroup : 1;  // units per trailing update
  const int64_t GW = static_cast<int64_t>(NU) * SB;
  const int gs = (!preset && group <= kB) ? group : 0;
  p.ld_err = static_cast<int>(GW);
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
      e = gemm_f32(d_out, rest, GW, -1.f, Err, GW, 0, U + g0 * d_in + g0 + GW, d_in, 0, false, 1.f, Wp + g0 + GW,
                   d_in, 0, 1, false, 0, st);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace gptq
