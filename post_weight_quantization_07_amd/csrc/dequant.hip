// Weight-only quantized matrix product on gfx950: y = x W^T with W dequantized
// on the fly from the solve's outputs (qweight, scales, zeros, g_idx).
//
// GPTQ 实战 ch.5 (group quantization, section 5.1.10): a weight is
// s_g (q - z_g) with its group's scale and zero point; the inference kernels
// the pages list (ExLlama, Marlin, Triton) read the packed codes and
// dequantize inside the product.  At decode batch sizes the product is bound
// by reading the packed weights (bits / 8 bytes per weight), so this is a
// bandwidth kernel, not a tile GEMM:
//
//   Lanes map to output columns (64 per workgroup), so a packed word load is
//   64 consecutive int32 of one qweight row.  K is walked in chunks of 32
//   codes (bits words per column); code j of a chunk sits at bit bits * j of
//   the chunk's words (a funnel shift where a 3-bit code straddles two words),
//   all offsets compile-time.  x (up to MT tokens per pass) is staged in LDS as
//   fp32 and read as wave-uniform broadcasts.  When a chunk's 32 columns share
//   one group (every case but act-order with dynamic groups), its scale and
//   zero point are read once per chunk and y += s * sum_k x_k (q_k - z);
//   otherwise each code reads its own group's s and z.  The four waves of a
//   workgroup take interleaved chunks of the workgroup's K range and are summed
//   through LDS in wave order; K is further split over KS workgroups whose
//   partial products a second kernel adds in slice order, so the result does
//   not depend on scheduling.
#include "gptq_common.h"
#include "gptq_internal.h"

#include <algorithm>

namespace gptq {
namespace {

constexpr int kCols = 64;          // output columns per workgroup
constexpr int kChunk = 32;         // codes per chunk
constexpr int kMaxChunksPerWG = 16;

struct DqParams {
  const void* x;
  int xbf16;
  int64_t ldx;
  int64_t m0, m;       // token rows of this pass: [m0, m0 + m)
  int64_t d_in, d_out;
  const int32_t* qweight;  // [d_in * bits / 32, d_out]
  const float* scales;     // [n_groups, d_out]
  const int32_t* zeros;    // [n_groups, d_out]
  const int32_t* g_idx;    // [d_in]
  int n_groups;
  int chunks;          // d_in / 32
  int cpw;             // chunks per workgroup
  int ks;              // K slices
  float* out;          // ks == 1: y rows m0.. (ld_out); else partial [ks][MT][d_out]
  int64_t ld_out;
};

// code j (0..31) of a chunk held in BITS words
template <int BITS, int J>
GPTQ_DEV uint32_t chunk_code(const uint32_t (&w)[BITS]) {
  constexpr int bit = BITS * J, wi = bit >> 5, sh = bit & 31;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  if constexpr (sh + BITS <= 32) {
    return (w[wi] >> sh) & mask;
  } else {
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & mask;
  }
}

template <int BITS, int MT, int... Js>
GPTQ_DEV void chunk_uniform(const uint32_t (&w)[BITS], const float (*xs)[MT], float z, float (&acc)[MT],
                            std::integer_sequence<int, Js...>) {
  (
      [&] {
        const float qz = static_cast<float>(chunk_code<BITS, Js>(w)) - z;
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[t] = fmaf(xs[Js][t], qz, acc[t]);
      }(),
      ...);
}

template <int BITS, int MT, int... Js>
GPTQ_DEV void chunk_grouped(const uint32_t (&w)[BITS], const float (*xs)[MT], const int32_t* gl, const DqParams& p,
                            int64_t n, float (&y)[MT], std::integer_sequence<int, Js...>) {
  (
      [&] {
        const int64_t g = gl[Js];
        const float s = p.scales[g * p.d_out + n];
        const float z = static_cast<float>(p.zeros[g * p.d_out + n]);
        const float wv = s * (static_cast<float>(chunk_code<BITS, Js>(w)) - z);
#pragma unroll
        for (int t = 0; t < MT; ++t) y[t] = fmaf(xs[Js][t], wv, y[t]);
      }(),
      ...);
}

template <int BITS, int MT>
__global__ __launch_bounds__(256) void dequant_matmul_kernel(DqParams p) {
  __shared__ __attribute__((aligned(16))) float xs[kMaxChunksPerWG][kChunk][MT];
  __shared__ int32_t gl[kMaxChunksPerWG][kChunk];
  __shared__ int uni[kMaxChunksPerWG];
  __shared__ float ys[4][MT][kCols];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblocks = static_cast<int>((p.d_out + kCols - 1) / kCols);
  const int nb = blockIdx.x % nblocks, ks = blockIdx.x / nblocks;
  const int c0 = ks * p.cpw, c1 = min(p.chunks, c0 + p.cpw), nc = max(0, c1 - c0);

  // stage x[m0 + t][32 c0 ..] (fp32, zero rows past m) and the chunks' groups
  for (int e = tid; e < nc * kChunk * MT; e += 256) {
    const int t = e % MT, kk = e / MT;  // kk: column within the workgroup's range
    const int64_t k = static_cast<int64_t>(c0) * kChunk + kk;
    float v = 0.f;
    if (t < p.m) {
      const int64_t off = (p.m0 + t) * p.ldx + k;
      v = p.xbf16 ? bf16_to_f32(static_cast<const uint16_t*>(p.x)[off]) : static_cast<const float*>(p.x)[off];
    }
    xs[kk / kChunk][kk % kChunk][t] = v;
  }
  for (int e = tid; e < nc * kChunk; e += 256) gl[e / kChunk][e % kChunk] = p.g_idx[static_cast<int64_t>(c0) * kChunk + e];
  __syncthreads();
  if (tid < nc) {
    int same = 1;
    for (int j = 1; j < kChunk; ++j) same &= (gl[tid][j] == gl[tid][0]);
    uni[tid] = same;
  }
  __syncthreads();

  const int64_t n = static_cast<int64_t>(nb) * kCols + lane;
  const int64_t nl = min(n, p.d_out - 1);  // loads of columns past the end read the last one
  float y[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) y[t] = 0.f;
  for (int cl = wave; cl < nc; cl += 4) {
    const int64_t c = c0 + cl;
    uint32_t w[BITS];
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = static_cast<uint32_t>(p.qweight[(c * BITS + i) * p.d_out + nl]);
    if (uni[cl]) {
      const int64_t g = gl[cl][0];
      const float s = p.scales[g * p.d_out + nl];
      const float z = static_cast<float>(p.zeros[g * p.d_out + nl]);
      float acc[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = 0.f;
      chunk_uniform<BITS, MT>(w, xs[cl], z, acc, std::make_integer_sequence<int, kChunk>{});
#pragma unroll
      for (int t = 0; t < MT; ++t) y[t] = fmaf(s, acc[t], y[t]);
    } else {
      chunk_grouped<BITS, MT>(w, xs[cl], gl[cl], p, nl, y, std::make_integer_sequence<int, kChunk>{});
    }
  }
  // the four waves' partial sums, added in wave order
#pragma unroll
  for (int t = 0; t < MT; ++t) ys[wave][t][lane] = y[t];
  __syncthreads();
  for (int e = tid; e < MT * kCols; e += 256) {
    const int t = e / kCols, col = e % kCols;
    const int64_t nn = static_cast<int64_t>(nb) * kCols + col;
    if (nn >= p.d_out || t >= p.m) continue;
    const float v = ((ys[0][t][col] + ys[1][t][col]) + ys[2][t][col]) + ys[3][t][col];
    if (p.ks == 1) p.out[(p.m0 + t) * p.ld_out + nn] = v;
    else p.out[(static_cast<int64_t>(ks) * MT + t) * p.d_out + nn] = v;
  }
}

// y[m0 + t][n] = sum over the K slices, in slice order
template <int MT>
__global__ void dequant_reduce_kernel(const float* part, int ks, int64_t m0, int64_t m, int64_t d_out, float* y,
                                      int64_t ld_y) {
  const int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (e >= m * d_out) return;
  const int64_t t = e / d_out, n = e - t * d_out;
  float v = 0.f;
  for (int s = 0; s < ks; ++s) v += part[(static_cast<int64_t>(s) * MT + t) * d_out + n];
  y[(m0 + t) * ld_y + n] = v;
}

struct DqPlan {
  int chunks, cpw, ks, nblocks;
};

DqPlan dq_plan(int64_t d_in, int64_t d_out) {
  DqPlan pl{};
  pl.chunks = static_cast<int>(d_in / kChunk);
  pl.nblocks = static_cast<int>((d_out + kCols - 1) / kCols);
  // about 2048 workgroups, at least 4 chunks (one per wave) per workgroup
  int ks = std::max(1, (2048 + pl.nblocks - 1) / pl.nblocks);
  ks = std::min(ks, std::max(1, pl.chunks / 4));
  pl.cpw = std::min(kMaxChunksPerWG, (pl.chunks + ks - 1) / ks);
  pl.ks = (pl.chunks + pl.cpw - 1) / pl.cpw;
  return pl;
}

constexpr int kMaxMT = 16;

template <int BITS, int MT>
hipError_t dq_pass(DqParams p, const DqPlan& pl, float* y, float* part, hipStream_t st) {
  p.out = (pl.ks == 1) ? y : part;
  dequant_matmul_kernel<BITS, MT><<<pl.nblocks * pl.ks, 256, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.ks == 1) return e;
  const int64_t total = p.m * p.d_out;
  dequant_reduce_kernel<MT><<<static_cast<unsigned>((total + 255) / 256), 256, 0, st>>>(part, pl.ks, p.m0, p.m,
                                                                                      p.d_out, y, p.ld_out);
  return hipGetLastError();
}

template <int BITS>
hipError_t dq_bits(DqParams p, const DqPlan& pl, float* y, float* part, hipStream_t st) {
  const int64_t mr = p.m;
  if (mr <= 1) return dq_pass<BITS, 1>(p, pl, y, part, st);
  if (mr <= 2) return dq_pass<BITS, 2>(p, pl, y, part, st);
  if (mr <= 4) return dq_pass<BITS, 4>(p, pl, y, part, st);
  if (mr <= 8) return dq_pass<BITS, 8>(p, pl, y, part, st);
  return dq_pass<BITS, 16>(p, pl, y, part, st);
}

}  // namespace

size_t dequant_workspace_bytes(int64_t m, int64_t d_in, int64_t d_out) {
  (void)m;
  const DqPlan pl = dq_plan(d_in, d_out);
  if (pl.ks == 1) return 256;
  return (static_cast<size_t>(pl.ks) * kMaxMT * d_out * sizeof(float) + 255) & ~static_cast<size_t>(255);
}

hipError_t dequant_matmul_launch(const void* x, bool x_bf16, int64_t m, int64_t d_in, const int32_t* qweight,
                                 const float* scales, const int32_t* zeros, const int32_t* g_idx, int bits,
                                 int64_t d_out, int n_groups, float* y, void* ws, hipStream_t st) {
  const DqPlan pl = dq_plan(d_in, d_out);
  DqParams p{};
  p.x = x;
  p.xbf16 = x_bf16 ? 1 : 0;
  p.ldx = d_in;
  p.d_in = d_in;
  p.d_out = d_out;
  p.qweight = qweight;
  p.scales = scales;
  p.zeros = zeros;
  p.g_idx = g_idx;
  p.n_groups = n_groups;
  p.chunks = pl.chunks;
  p.cpw = pl.cpw;
  p.ks = pl.ks;
  p.ld_out = d_out;
  float* part = static_cast<float*>(ws);
  for (int64_t m0 = 0; m0 < m; m0 += kMaxMT) {
    p.m0 = m0;
    p.m = std::min<int64_t>(kMaxMT, m - m0);
    hipError_t e;
    switch (bits) {
      case 2: e = dq_bits<2>(p, pl, y, part, st); break;
      case 3: e = dq_bits<3>(p, pl, y, part, st); break;
      case 4: e = dq_bits<4>(p, pl, y, part, st); break;
      case 8: e = dq_bits<8>(p, pl, y, part, st); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gptq
