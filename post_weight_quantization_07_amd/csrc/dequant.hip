// Weight-only quantized matrix product on gfx950: y = x W^T with W dequantized
// on the fly from the solve's outputs (qweight, scales, zeros, g_idx).
//
// GPTQ 实战 ch.5 (group quantization, section 5.1.10): a weight is
// s_g (q - z_g) with its group's scale and zero point; the inference kernels
// the pages list (ExLlama, Marlin, Triton) read the packed codes and
// dequantize inside the product.  At decode batch sizes the product is bound
// by reading the packed weights (bits / 8 bytes per weight).
//
// K is walked in chunks of 32 codes (bits words per column), x staged in LDS
// per 16 chunks.  Whether a chunk's 32 channels share one group is read from
// g_idx by a ballot (lanes 0-31 hold one chunk's entries, 32-63 the next).  A
// one-group chunk (every case but act-order with dynamic groups) reads its
// scale and zero point once; otherwise each code reads its own group's s and
// z.  Partial sums are added in a fixed order, so the result does not depend
// on scheduling.  An act-order layer can be put in group order once (the
// order_* kernels at the end: channels stably sorted by group, codes
// repacked, x gathered in that order per call), which makes its chunks
// one-group again.
//
// MFMA path (bf16 x, 3 tokens or more; v_mfma_f32_16x16x32_bf16): a wave
// computes 16 tokens x 16 columns of one chunk.  Inside a chunk, codes 8 g ..
// 8 g + 7 go to lane group g (lanes 16 g .. 16 g + 15), in both operands
// alike, so lane group g of column n needs one packed word at 4 bits, two at
// 8, half a word at 2, a 24-bit funnel-shifted field at 3.  For a one-group
// chunk the B operand is the codes themselves (integers <= 255, exact in
// bf16), a second MFMA adds x times -z, and the column's scale multiplies the
// chunk's sum in fp32, so the products are exact.  At 4 bits the operands
// are 16 + q and -(16 + z), built from the packed word with integer
// operations only (interleave_halves), which widens the rounding bound by 32
// per term.  A chunk spread over several groups uses B = s (q - z) split into
// bf16 high and low parts (two MFMAs).  A workgroup of 4 waves owns 64
// output columns (16 per wave) and walks its K range in stages of 16 chunks;
// K is split over workgroups, with fewer slices than the VALU path.
//
// VALU path (fp32 x, or 1-2 tokens): lanes map to output columns (64 per
// workgroup, so a packed word load is 64 consecutive int32 of one qweight
// row); a lane converts its chunk's 32 codes with compile-time offsets and
// accumulates MT tokens.  A one-group chunk adds s (sum_k x_k q_k - z sum_k
// x_k), the chunk's sum of x formed once per workgroup while x is staged,
// which takes the subtraction of z out of the per-code work (two operations
// per code at 2, 4 and 8 bits: a byte-to-float conversion and an FMA; with
// bf16 x at 4 bits one v_dot2_f32_bf16 per two codes on the MFMA path's
// 16 + q operands); its rounding error is bounded by the sum of
// |x_k| s (q_k + z) instead of |x_k| s |q_k - z|.  The four waves take
// interleaved chunks of the workgroup's K range and are summed through LDS in
// wave order; K is split over workgroups whose partial products a second
// kernel adds in slice order.
#include "gptq_common.h"
#include "gptq_internal.h"

#include <algorithm>
#include <atomic>
#include <mutex>

namespace gptq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kValuCols = 64;  // output columns per workgroup
constexpr int kChunk = 32;     // codes per chunk
constexpr int kStage = 16;     // chunks per LDS stage
constexpr int kMaxMT = 16;     // tokens per pass

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
  const int32_t* xorder;   // VALU path: x channel of sorted position j is xorder[j] (null: j)
  uint32_t qbytes;         // bytes of qweight, < 2^31
  uint32_t gbytes;         // bytes of scales (and of zeros), < 2^31
  int chunks;              // d_in / 32
  int cpw;                 // chunks per workgroup
  int ks;                  // K slices
  float* y;                // [m_total, d_out]
  float* part;             // ks > 1: partial sums [ks][MT][d_out] (MT = 16 on the MFMA path)
};

// qweight, scales and zeros are read through buffer descriptors: a lane's
// column offset is its 32-bit VGPR offset, and the part common to the wave
// (chunk row, group row) goes into the scalar offset, so a load costs no
// vector address arithmetic.  Every offset stays inside the tensor.
GPTQ_DEV __amdgpu_buffer_rsrc_t buffer_of(const void* ptr, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(ptr), 0, static_cast<int>(bytes), 0x00020000);
}

GPTQ_DEV uint32_t bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

GPTQ_DEV int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// At 4 bits the operands of a lane group hold its 8 k in the order 0 4 1 5 2
// 6 3 7 (dword j = k j and k j + 4): nibbles j and j + 4 of a code word are
// 16 bits apart, so one shift and one mask-or turn them into a bf16 pair.
// interleave_halves puts 8 bf16 of x into that order; operand_code gives the
// k of half h of dword j.
GPTQ_DEV u32x4_t interleave_halves(const u32x4_t& v) {
  u32x4_t r;
  r[0] = (v[0] & 0xffffu) | (v[2] << 16);
  r[1] = (v[0] >> 16) | (v[2] & 0xffff0000u);
  r[2] = (v[1] & 0xffffu) | (v[3] << 16);
  r[3] = (v[1] >> 16) | (v[3] & 0xffff0000u);
  return r;
}

// x[m0 + t][32 c0 ..] for the stage's chunks in 16-byte pieces (4 fp32 or 8
// bf16): piece e is token e / row_pieces, piece e % row_pieces of that row.
// load_x issues a thread's pieces (a clamped, in-range piece past the stage's
// live chunks or tokens); store_x writes them to LDS after the code words'
// loads are in flight: xs[chunk][t][j] as fp32 (0 for t >= m) and, for the dot
// form, xi[chunk][t] as the interleaved bf16 pairs.
template <int MT>
struct XPieces {
  static constexpr int kN = (MT * kStage * kChunk / 4 + 255) / 256;  // fp32 x; bf16 uses half
  u32x4_t v[kN];
};

template <int MT>
GPTQ_DEV void load_x(const DqParams& p, int64_t c0, int nc, int tid, XPieces<MT>& xp) {
  const int per = p.xbf16 ? 8 : 4;               // elements per piece
  const int row_pieces = kStage * kChunk / per;  // pieces per token row of the stage
  const int live = std::max(1, nc * kChunk / per);
#pragma unroll
  for (int i = 0; i < XPieces<MT>::kN; ++i) {
    const int e = tid + 256 * i;
    if (e < MT * row_pieces) {
      const int t = e / row_pieces, k = std::min(e % row_pieces, live - 1);
      const int64_t row = p.m0 + std::min<int64_t>(t, p.m - 1);
      const int64_t col = c0 * kChunk + static_cast<int64_t>(k) * per;
      if (p.xorder) {  // group order: gather the piece's channels
        if (p.xbf16) {
          const uint16_t* xr = static_cast<const uint16_t*>(p.x) + row * p.ldx;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            xp.v[i][q] = static_cast<uint32_t>(xr[p.xorder[col + 2 * q]]) |
                         (static_cast<uint32_t>(xr[p.xorder[col + 2 * q + 1]]) << 16);
        } else {
          const uint32_t* xr = static_cast<const uint32_t*>(p.x) + row * p.ldx;
#pragma unroll
          for (int q = 0; q < 4; ++q) xp.v[i][q] = xr[p.xorder[col + q]];
        }
      } else {
        xp.v[i] = p.xbf16 ? *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p.x) + row * p.ldx + col)
                          : *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(p.x) + row * p.ldx + col);
      }
    }
  }
}

// v moved between lanes by a DPP control (quad permutation or row shift;
// lanes with no source read 0)
template <int CTRL>
GPTQ_DEV float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}

// Also the chunk's sum of x per token into xsum[chunk][t]: a thread adds its
// piece's elements in order, then the pieces of a chunk (4 consecutive lanes
// for bf16, 8 for fp32, aligned) are added across lanes by DPP moves (quad
// xor 1, xor 2, then for fp32 the neighbouring quad by a row shift of 4), and
// the lane of the chunk's last piece writes the sum.  Every lane takes part
// in the moves; lanes without a live piece carry zeros.
template <int MT>
GPTQ_DEV void store_x(const DqParams& p, int nc, int tid, const XPieces<MT>& xp, float (*xs)[MT][kChunk + 4],
                      uint32_t (*xi)[MT][kChunk / 2 + 4], float (*xsum)[MT]) {
  const int per = p.xbf16 ? 8 : 4;
  const int row_pieces = kStage * kChunk / per;
  const int live = nc * kChunk / per;
#pragma unroll
  for (int i = 0; i < XPieces<MT>::kN; ++i) {
    const int e = tid + 256 * i;
    const int t = e / row_pieces, k = e % row_pieces;
    const bool here = t < MT && k < live;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    const u32x4_t v = (here && t < p.m) ? xp.v[i] : z;
    float f[8];
    int nf = 4;
    if (p.xbf16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(v[q] << 16);
        f[2 * q + 1] = __uint_as_float(v[q] & 0xffff0000u);
      }
      nf = 8;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = __uint_as_float(v[q]);
    }
    float sum = f[0];
#pragma unroll
    for (int q = 1; q < 8; ++q)
      if (q < nf) sum += f[q];
    sum += dpp_move<0xb1>(sum);  // quad lanes xor 1
    sum += dpp_move<0x4e>(sum);  // quad lanes xor 2
    if (!p.xbf16) sum += dpp_move<0x114>(sum);  // row shift right by 4: the chunk's first quad
    if (!here) continue;
    const int kk = k * per, cl = kk / kChunk, j = kk % kChunk;
    if (p.xbf16) {
#pragma unroll
      for (int q = 0; q < 8; ++q) xs[cl][t][j + q] = f[q];
      // the 8 bf16 as interleaved pairs (k, k + 4), the 4-bit operand order
      if (xi) *reinterpret_cast<u32x4_t*>(&xi[cl][t][j / 2]) = interleave_halves(v);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) xs[cl][t][j + q] = f[q];
    }
    if (j + per == kChunk) xsum[cl][t] = sum;
  }
}

// ---------------------------------------------------------------- VALU path

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

// x & M with the mask hidden from the optimizer: with the mask visible it
// turns each later byte extraction back into a bit-field extract of the
// original word, one more operation per code
template <uint32_t M>
GPTQ_DEV uint32_t opaque_and(uint32_t x) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "i"(M), "v"(x));
  return r;
}

// code j of a chunk as a float.  Widths that divide 8 spread the word's codes
// over bytes first (one shift and one mask per byte lane set, shared by the
// codes of a word) so that each code then converts in one byte-to-float step.
template <int BITS, int J>
GPTQ_DEV float chunk_code_f(const uint32_t (&w)[BITS]) {
  if constexpr (BITS == 8) {
    return static_cast<float>((w[J >> 2] >> (8 * (J & 3))) & 0xffu);
  } else if constexpr (BITS == 4) {
    constexpr int i = J & 7;  // nibble i: byte i / 2 of the even or odd nibbles
    const uint32_t v = opaque_and<0x0f0f0f0fu>((i & 1) ? (w[J >> 3] >> 4) : w[J >> 3]);
    return static_cast<float>((v >> (8 * (i >> 1))) & 0xffu);
  } else if constexpr (BITS == 2) {
    constexpr int i = J & 15;  // 2-bit field i: byte i / 4 after a shift by 2 (i % 4)
    const uint32_t v = opaque_and<0x03030303u>(w[J >> 4] >> (2 * (i & 3)));
    return static_cast<float>((v >> (8 * (i >> 2))) & 0xffu);
  } else {
    return static_cast<float>(chunk_code<BITS, J>(w));
  }
}

// acc[t] += sum_j x[t][j] q_j over the chunk; the zero point is applied once
// per chunk by the caller, as z times the chunk's sum of x
template <int BITS, int MT, int... J4s>
GPTQ_DEV void valu_uniform(const uint32_t (&w)[BITS], const float (*xs)[kChunk + 4], float (&acc)[MT],
                           std::integer_sequence<int, J4s...>) {
  (
      [&] {
        // codes 4 J4 .. 4 J4 + 3 against one 16-byte read of x per token
        const float q0 = chunk_code_f<BITS, 4 * J4s>(w), q1 = chunk_code_f<BITS, 4 * J4s + 1>(w);
        const float q2 = chunk_code_f<BITS, 4 * J4s + 2>(w), q3 = chunk_code_f<BITS, 4 * J4s + 3>(w);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const f32x4_t xv = *reinterpret_cast<const f32x4_t*>(&xs[t][4 * J4s]);
          acc[t] = fmaf(xv[0], q0, acc[t]);
          acc[t] = fmaf(xv[1], q1, acc[t]);
          acc[t] = fmaf(xv[2], q2, acc[t]);
          acc[t] = fmaf(xv[3], q3, acc[t]);
        }
      }(),
      ...);
}

// 4-bit codes against bf16 x: acc[t] += sum_k x[t][k] (16 + q_k) over the
// chunk by v_dot2_f32_bf16, two codes per instruction.  Nibbles j and j + 4
// of a code word sit 16 bits apart, so one shift and one mask-or give the
// bf16 pair (16 + q_j, 16 + q_{j+4}) (0x4180 | q << 3); xi holds x as the
// matching pairs (k, k + 4) of each 8 k.  The caller subtracts (16 + z) sum x.
template <int MT>
GPTQ_DEV void valu_uniform_dot4(const uint32_t (&w)[4], const uint32_t (*xi)[kChunk / 2 + 4], float (&acc)[MT]) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  // the bf16 pair (16, 16) held in a vector register: with both constants
  // literal the mask and the or do not fuse into one v_and_or_b32 (a 3-operand
  // instruction takes one scalar operand and no literal here)
  const uint32_t magic = opaque_and<0xffffffffu>(0x41804180u);
#pragma unroll
  for (int wi = 0; wi < 4; ++wi) {
    const uint32_t f = w[wi];
    uint32_t b[4];
    b[0] = ((f << 3) & 0x00780078u) | magic;
#pragma unroll
    for (int j = 1; j < 4; ++j) b[j] = ((f >> (4 * j - 3)) & 0x00780078u) | magic;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(&xi[t][4 * wi]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // copied out first: __builtin_bit_cast of a vector-element lvalue
        // (xv[j]) reads element 0 whatever j is
        const uint32_t xj = xv[j];
        acc[t] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, xj), __builtin_bit_cast(bf16x2_t, b[j]),
                                                 acc[t], false);
      }
    }
  }
}

// codes J0 .. J0 + 7 of a chunk spread over groups: gv holds the chunk's
// g_idx in lanes base .. base + 31.  The eight codes' scale and zero-point
// loads are issued together, then used: one wait per eight codes.
template <int BITS, int MT, int J0, int... Us>
GPTQ_DEV void valu_grouped8(const uint32_t (&w)[BITS], const float (*xs)[kChunk + 4], int32_t gv, int base,
                            __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rz, uint32_t rowb, uint32_t vo,
                            float (&y)[MT], std::integer_sequence<int, Us...>) {
  uint32_t sb[sizeof...(Us)], zb[sizeof...(Us)];
  (
      [&] {
        const uint32_t so = static_cast<uint32_t>(__builtin_amdgcn_readlane(gv, base + J0 + Us)) * rowb;
        sb[Us] = bload(rs, vo, so);
        zb[Us] = bload(rz, vo, so);
      }(),
      ...);
  (
      [&] {
        const float z = static_cast<float>(static_cast<int32_t>(zb[Us]));
        const float wv = __builtin_bit_cast(float, sb[Us]) * (static_cast<float>(chunk_code<BITS, J0 + Us>(w)) - z);
#pragma unroll
        for (int t = 0; t < MT; ++t) y[t] = fmaf(xs[t][J0 + Us], wv, y[t]);
      }(),
      ...);
}

template <int BITS, int MT, int... J8s>
GPTQ_DEV void valu_grouped(const uint32_t (&w)[BITS], const float (*xs)[kChunk + 4], int32_t gv, int base,
                           __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rz, uint32_t rowb, uint32_t vo,
                           float (&y)[MT], std::integer_sequence<int, J8s...>) {
  (valu_grouped8<BITS, MT, 8 * J8s>(w, xs, gv, base, rs, rz, rowb, vo, y, std::make_integer_sequence<int, 8>{}), ...);
}

// gix is g_idx again, as its own restrict argument, so that its reads
// (wave-uniform addresses: a chunk's entries) become scalar loads.
// DOT: 4-bit codes with bf16 x, one-group chunks on v_dot2_f32_bf16.
// A workgroup's x pieces are loaded first (they hit L2: every workgroup of
// the K slice reads them), then each wave's chunks' g_idx (lanes 0-31 one
// chunk, 32-63 the next), code words, scales and zero points; a ballot over
// the g_idx lanes tells which chunks lie in one group, one barrier makes the
// staged x visible, and each wave forms its chunks' sums of x itself.
template <int BITS, int MT, bool DOT>
__global__ __launch_bounds__(256) void dequant_valu_kernel(DqParams p, const int32_t* __restrict__ gix) {
  static_assert(!DOT || BITS == 4, "the dot form is for 4-bit codes");
  __shared__ __attribute__((aligned(16))) float xs[kStage][MT][kChunk + 4];
  __shared__ __attribute__((aligned(16))) uint32_t xi[DOT ? kStage : 1][MT][kChunk / 2 + 4];
  __shared__ float xsum[kStage][MT];
  __shared__ float ys[4][MT][kValuCols];
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_uniform(tid >> 6);
  const int nblocks = static_cast<int>((p.d_out + kValuCols - 1) / kValuCols);
  const int nb = blockIdx.x % nblocks, ks = blockIdx.x / nblocks;
  const int64_t c0 = static_cast<int64_t>(ks) * p.cpw;
  const int nc = static_cast<int>(std::max<int64_t>(0, std::min<int64_t>(p.chunks, c0 + p.cpw) - c0));
  const int64_t n = static_cast<int64_t>(nb) * kValuCols + lane;
  const int64_t nl = std::min(n, p.d_out - 1);  // columns past the end read the last one
  XPieces<MT> xp;
  load_x<MT>(p, c0, nc, tid, xp);
  // the wave's chunks wave, wave + 4, ...: code words and first group's scale
  // and zero point at in-range chunk indices, and whether the chunk is one group
  const __amdgpu_buffer_rsrc_t rq = buffer_of(p.qweight, p.qbytes), rs = buffer_of(p.scales, p.gbytes),
                               rz = buffer_of(p.zeros, p.gbytes);
  const uint32_t rowb = static_cast<uint32_t>(p.d_out) * 4u, vo = static_cast<uint32_t>(nl) * 4u;
  constexpr int kPerWave = kStage / 4;
  auto chunk_of = [&](int i) {  // the wave's i-th chunk, clamped in range
    return std::min<int64_t>(c0 + std::min(wave + 4 * i, std::max(nc, 1) - 1), p.chunks - 1);
  };
  int32_t gv[kPerWave / 2];
#pragma unroll
  for (int h = 0; h < kPerWave / 2; ++h) gv[h] = p.g_idx[chunk_of(2 * h + (lane >> 5)) * kChunk + (lane & 31)];
  uint32_t wq[kPerWave][BITS];
  float sc[kPerWave];
  int32_t zc[kPerWave], g0[kPerWave];
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int64_t c = chunk_of(i);
#pragma unroll
    for (int b = 0; b < BITS; ++b) wq[i][b] = bload(rq, vo, static_cast<uint32_t>(c * BITS + b) * rowb);
    g0[i] = gix[c * kChunk];
    const uint32_t so = static_cast<uint32_t>(g0[i]) * rowb;
    sc[i] = __builtin_bit_cast(float, bload(rs, vo, so));
    zc[i] = static_cast<int32_t>(bload(rz, vo, so));
  }
  bool one[kPerWave];
#pragma unroll
  for (int h = 0; h < kPerWave / 2; ++h) {
    // each half against its chunk's first entry (a wave-uniform value)
    one[2 * h] = static_cast<uint32_t>(__ballot(gv[h] != g0[2 * h])) == 0u;
    one[2 * h + 1] = (__ballot(gv[h] != g0[2 * h + 1]) >> 32) == 0u;
  }
  store_x<MT>(p, nc, tid, xp, xs, DOT ? xi : nullptr, xsum);
  __syncthreads();
  float y[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) y[t] = 0.f;
#pragma unroll
  for (int i = 0; i < kPerWave; ++i) {
    const int cl = wave + 4 * i;
    if (cl >= nc) continue;
    const uint32_t(&w)[BITS] = wq[i];
    if (one[i]) {
      const float s = sc[i];
      const float z = static_cast<float>(zc[i]);
      float acc[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = 0.f;
      if constexpr (DOT) {
        valu_uniform_dot4<MT>(w, xi[cl], acc);
#pragma unroll
        for (int t = 0; t < MT; ++t) y[t] = fmaf(s, fmaf(-(16.f + z), xsum[cl][t], acc[t]), y[t]);
      } else {
        valu_uniform<BITS, MT>(w, xs[cl], acc, std::make_integer_sequence<int, kChunk / 4>{});
#pragma unroll
        for (int t = 0; t < MT; ++t) y[t] = fmaf(s, fmaf(-z, xsum[cl][t], acc[t]), y[t]);
      }
    } else {
      valu_grouped<BITS, MT>(w, xs[cl], gv[i / 2], 32 * (i & 1), rs, rz, rowb, vo, y,
                             std::make_integer_sequence<int, kChunk / 8>{});
    }
  }
  // the four waves' partial sums, added in wave order
#pragma unroll
  for (int t = 0; t < MT; ++t) ys[wave][t][lane] = y[t];
  __syncthreads();
  for (int e = tid; e < MT * kValuCols; e += 256) {
    const int t = e / kValuCols, col = e % kValuCols;
    const int64_t nn = static_cast<int64_t>(nb) * kValuCols + col;
    if (nn >= p.d_out || t >= p.m) continue;
    const float v = ((ys[0][t][col] + ys[1][t][col]) + ys[2][t][col]) + ys[3][t][col];
    if (p.ks == 1) p.y[(p.m0 + t) * p.d_out + nn] = v;
    else p.part[(static_cast<int64_t>(ks) * MT + t) * p.d_out + nn] = v;
  }
}

// y[m0 + t][n] = sum over the K slices, in slice order
template <int MT>
__global__ void dequant_reduce_kernel(const float* part, int ks, int64_t m0, int64_t m, int64_t d_out, float* y) {
  const int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (e >= m * d_out) return;
  const int64_t t = e / d_out, n = e - t * d_out;
  const float* q = part + t * d_out + n;
  const int64_t step = static_cast<int64_t>(MT) * d_out;
  float v = 0.f;
  int s = 0;
  for (; s + 16 <= ks; s += 16) {
    float l[16];  // sixteen slices' loads in flight, added in slice order
#pragma unroll
    for (int i = 0; i < 16; ++i) l[i] = q[(s + i) * step];
#pragma unroll
    for (int i = 0; i < 16; ++i) v += l[i];
  }
  for (; s + 4 <= ks; s += 4) {
    float l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) l[i] = q[(s + i) * step];
#pragma unroll
    for (int i = 0; i < 4; ++i) v += l[i];
  }
  for (; s < ks; ++s) v += q[s * step];
  y[(m0 + t) * d_out + n] = v;
}

// ---------------------------------------------------------------- MFMA path

// Lane group g's 8 codes of a chunk in column n (codes 8 g .. 8 g + 7 of the
// chunk) sit at bits 8 g BITS .. 8 g BITS + 8 BITS - 1 of the chunk's BITS
// words, so a lane group loads only the word or two that hold them: word g
// at 4 bits, word g / 2 (half g % 2) at 2, words 2 g and 2 g + 1 at 8, and at
// 3 bits the words holding bit 24 g and 24 g + 23: (0, 1), (0, 1), (1, 2),
// (2, 2).  LaneWords holds their byte offsets within the chunk's rows.
template <int BITS>
constexpr int kLaneWords = (BITS == 8 || BITS == 3) ? 2 : 1;

template <int BITS>
struct LaneWords {
  uint32_t off[kLaneWords<BITS>];
  GPTQ_DEV LaneWords() {}
  GPTQ_DEV LaneWords(int g, int64_t d_out, int64_t n) {
    const uint32_t rowb = static_cast<uint32_t>(d_out) * 4u, nb = static_cast<uint32_t>(n) * 4u;
    if constexpr (BITS == 8) {
      off[0] = (2 * g) * rowb + nb;
      off[1] = (2 * g + 1) * rowb + nb;
    } else if constexpr (BITS == 3) {
      const int lo = (24 * g) >> 5;
      off[0] = lo * rowb + nb;
      off[1] = std::min(lo + 1, 2) * rowb + nb;
    } else if constexpr (BITS == 4) {
      off[0] = g * rowb + nb;
    } else {
      off[0] = (g >> 1) * rowb + nb;
    }
  }
};

// the words of chunk c: soff is the chunk's first row, c BITS d_out 4 bytes
template <int BITS>
GPTQ_DEV void lane_words(__amdgpu_buffer_rsrc_t rq, const LaneWords<BITS>& lw, uint32_t soff, int g,
                         uint32_t (&w)[kLaneWords<BITS>]) {
#pragma unroll
  for (int i = 0; i < kLaneWords<BITS>; ++i) w[i] = bload(rq, lw.off[i], soff);
  if constexpr (BITS == 2) w[0] >>= 16 * (g & 1);
}

// those 8 codes as floats (exact integers)
template <int BITS>
GPTQ_DEV void lane_codes(const uint32_t (&w)[kLaneWords<BITS>], int g, float (&q)[8]) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[i] = static_cast<float>((w[0] >> (8 * i)) & 0xffu);
      q[4 + i] = static_cast<float>((w[1] >> (8 * i)) & 0xffu);
    }
  } else if constexpr (BITS == 4) {
    const uint32_t ev = opaque_and<0x0f0f0f0fu>(w[0]), od = opaque_and<0x0f0f0f0fu>(w[0] >> 4);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      q[2 * b] = static_cast<float>((ev >> (8 * b)) & 0xffu);
      q[2 * b + 1] = static_cast<float>((od >> (8 * b)) & 0xffu);
    }
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t v = opaque_and<0x03030303u>(w[0] >> (2 * k));  // codes k and 4 + k in bytes 0 and 1
      q[k] = static_cast<float>(v & 0xffu);
      q[4 + k] = static_cast<float>((v >> 8) & 0xffu);
    }
  } else {
    const uint32_t f = __builtin_amdgcn_alignbit(w[1], w[0], static_cast<uint32_t>((24 * g) & 31));
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = static_cast<float>((f >> (3 * i)) & 7u);
  }
}

// two floats that are bf16 values (here integers of at most 8 significant
// bits) as a bf16 pair, a in the low half: the low 16 bits of each are zero
GPTQ_DEV uint32_t pack_exact_bf16(float a, float b) {
  return (__builtin_bit_cast(uint32_t, b) & 0xffff0000u) | (__builtin_bit_cast(uint32_t, a) >> 16);
}

GPTQ_DEV uint32_t bf16_bits_of(float v) {
  // round to nearest even; inputs are finite
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

GPTQ_DEV float bf16_value(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

template <int BITS>
constexpr int operand_code(int j, int h) {
  return BITS == 4 ? j + 4 * h : 2 * j + h;
}

GPTQ_DEV f32x4_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// T column tiles of 16 per wave (64 T columns per workgroup: x staged once
// serves them all) and SC chunks per LDS stage
template <int BITS, int T, int SC, int NW>
__global__ __launch_bounds__(64 * NW) void dequant_mfma_kernel(DqParams p, const int32_t* __restrict__ gix) {
  static_assert(SC % 2 == 0, "chunks go to the g_idx lanes in pairs");
  constexpr int kThreads = 64 * NW;
  __shared__ __attribute__((aligned(16))) uint16_t xb[SC][16][kChunk + 8];  // bf16 x, [chunk][token][k]
  __shared__ int32_t gl[SC][kChunk];  // g_idx of the stage's chunks
  __shared__ int uni[SC];             // whether each chunk lies in one group
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_uniform(tid >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  constexpr int kCols = 16 * T * NW;
  constexpr int kPairsPerWave = (SC / 2 + NW - 1) / NW;  // chunk pairs whose g_idx a wave checks
  const int nblocks = static_cast<int>((p.d_out + kCols - 1) / kCols);
  const int nb = blockIdx.x % nblocks, ks = blockIdx.x / nblocks;
  const int64_t cb = static_cast<int64_t>(ks) * p.cpw;
  const int64_t ce = std::min<int64_t>(p.chunks, cb + p.cpw);
  const uint16_t* xh = static_cast<const uint16_t*>(p.x);
  const __amdgpu_buffer_rsrc_t rq = buffer_of(p.qweight, p.qbytes), rs = buffer_of(p.scales, p.gbytes),
                               rz = buffer_of(p.zeros, p.gbytes);
  const uint32_t rowb = static_cast<uint32_t>(p.d_out) * 4u;
  // wave w: columns 16 T w .. 16 T w + 16 T - 1 of the workgroup, tile t the
  // 16 from 16 T w + 16 t
  int64_t n[T];
  uint32_t vo[T];
  LaneWords<BITS> lwo[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    n[t] = static_cast<int64_t>(nb) * kCols + 16 * T * wave + 16 * t + c16;
    const int64_t nl = std::min(n[t], p.d_out - 1);
    vo[t] = static_cast<uint32_t>(nl) * 4u;
    lwo[t] = LaneWords<BITS>(g, p.d_out, nl);
  }
  f32x4_t y[T];  // tokens 4 g + e, column n[t]
#pragma unroll
  for (int t = 0; t < T; ++t) y[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the workgroup's K range in stages of up to SC chunks
  for (int64_t c0 = cb; c0 < ce; c0 += SC) {
    const int nc = static_cast<int>(std::min<int64_t>(SC, ce - c0));  // >= 1
    if (c0 != cb) __syncthreads();  // the previous stage's LDS reads are done
    // 16 tokens x nc chunks of bf16 x as 16-byte pieces, issued first (L2
    // hits: every workgroup of the K slice reads them); every load at an
    // in-range address (rows past m repeat the last row, pieces past the
    // range the last piece), selected after
    constexpr int kRowPieces = SC * kChunk / 8;
    constexpr int kPieces = 16 * kRowPieces;
    static_assert(kPieces % kThreads == 0, "whole passes over the stage's pieces");
    const int live = nc * kChunk / 8;
    u32x4_t v[kPieces / kThreads];
#pragma unroll
    for (int i = 0; i < kPieces / kThreads; ++i) {
      const int e = tid + kThreads * i, t = e / kRowPieces, k8 = std::min(e % kRowPieces, live - 1);
      const int64_t row = p.m0 + std::min<int64_t>(t, p.m - 1);
      v[i] = *reinterpret_cast<const u32x4_t*>(xh + row * p.ldx + c0 * kChunk + 8 * k8);
    }
    // g_idx of chunk pairs wave, wave + NW, ..: lanes 0-31 hold chunk 2 h,
    // lanes 32-63 chunk 2 h + 1 (in-range chunk indices)
    int32_t gv[kPairsPerWave];
#pragma unroll
    for (int u = 0; u < kPairsPerWave; ++u) {
      const int h = std::min(wave + NW * u, SC / 2 - 1);
      gv[u] = p.g_idx[(c0 + std::min(2 * h + (lane >> 5), nc - 1)) * kChunk + (lane & 31)];
    }
    // the stage's code words, scales and zero points (the chunk's first
    // group's), loaded at in-range chunk indices (chunks past nc repeat the
    // last)
    uint32_t wq[SC][T][kLaneWords<BITS>];
    float sc[SC][T];
    int32_t zc[SC][T];
#pragma unroll
    for (int cl = 0; cl < SC; ++cl) {
      const int64_t c = c0 + std::min(cl, nc - 1);
      const uint32_t so = static_cast<uint32_t>(gix[c * kChunk]) * rowb;
#pragma unroll
      for (int t = 0; t < T; ++t) {
        lane_words<BITS>(rq, lwo[t], static_cast<uint32_t>(c * BITS) * rowb, g, wq[cl][t]);
        sc[cl][t] = __builtin_bit_cast(float, bload(rs, vo[t], so));
        zc[cl][t] = static_cast<int32_t>(bload(rz, vo[t], so));
      }
    }
#pragma unroll
    for (int i = 0; i < kPieces / kThreads; ++i) {
      const int e = tid + kThreads * i, t = e / kRowPieces, k8 = e % kRowPieces;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      u32x4_t w = (t < p.m) ? v[i] : z;
      if constexpr (BITS == 4) w = interleave_halves(w);
      if (k8 < live) *reinterpret_cast<u32x4_t*>(&xb[k8 / 4][t][8 * (k8 % 4)]) = w;
    }
    // the checked pairs' g_idx to LDS, and whether each chunk lies in one
    // group: a ballot of the lanes that differ from the chunk's first entry
#pragma unroll
    for (int u = 0; u < kPairsPerWave; ++u) {
      const int h = wave + NW * u;
      if (h >= SC / 2) continue;
      gl[2 * h + (lane >> 5)][lane & 31] = gv[u];
      const int32_t f0 = __builtin_amdgcn_readlane(gv[u], 0), f1 = __builtin_amdgcn_readlane(gv[u], 32);
      const uint64_t d0 = __ballot(gv[u] != f0), d1 = __ballot(gv[u] != f1);
      if (lane == 0) {
        uni[2 * h] = static_cast<uint32_t>(d0) == 0u;
        uni[2 * h + 1] = (d1 >> 32) == 0u;
      }
    }
    __syncthreads();
#pragma unroll
    for (int cl = 0; cl < SC; ++cl) {
      if (cl >= nc) continue;
      // A: x[token c16][8 g .. 8 g + 7], shared by the wave's tiles; B: codes
      // 8 g .. 8 g + 7 of column n[t]
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&xb[cl][c16][8 * g]);
      const int one_group = uni[cl];
#pragma unroll
      for (int t = 0; t < T; ++t) {
        // one group: B0 = the codes, B1 = -z, scaled by the column's s after,
        // giving s (sum_k x_k q_k - z sum_k x_k); several groups: B0 + B1 =
        // s (q - z) per code in bf16 high and low parts, scale 1.  At 4 bits
        // both operands are in the order of interleave_halves and the
        // one-group operands are built from the word directly: B0 = 16 + q,
        // B1 = -(16 + z)
        u32x4_t b0, b1;
        float s;
        if (BITS == 4 && one_group) {
          s = sc[cl][t];
          const uint32_t f = wq[cl][t][0];
          b0[0] = ((f << 3) & 0x00780078u) | 0x41804180u;
#pragma unroll
          for (int j = 1; j < 4; ++j) b0[j] = ((f >> (4 * j - 3)) & 0x00780078u) | 0x41804180u;
          const uint32_t hz = 0xc180u | (static_cast<uint32_t>(zc[cl][t]) << 3);
          const uint32_t bz = hz | (hz << 16);
#pragma unroll
          for (int j = 0; j < 4; ++j) b1[j] = bz;
        } else if (one_group) {
          float q[8];
          lane_codes<BITS>(wq[cl][t], g, q);
          s = sc[cl][t];
          const float z = static_cast<float>(zc[cl][t]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            b0[j] = pack_exact_bf16(q[2 * j], q[2 * j + 1]);
            b1[j] = pack_exact_bf16(-z, -z);
          }
        } else {
          float q[8];
          lane_codes<BITS>(wq[cl][t], g, q);
          s = 1.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t hw[2], lw[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int i = operand_code<BITS>(j, h);  // the code in half h of dword j
              const uint32_t o = static_cast<uint32_t>(gl[cl][8 * g + i]) * rowb + vo[t];
              const float sg = __builtin_bit_cast(float, bload(rs, o, 0u));
              const float z = static_cast<float>(static_cast<int32_t>(bload(rz, o, 0u)));
              const float v = sg * (q[i] - z);
              hw[h] = bf16_bits_of(v);
              lw[h] = bf16_bits_of(v - bf16_value(hw[h]));
            }
            b0[j] = hw[0] | (hw[1] << 16);
            b1[j] = lw[0] | (lw[1] << 16);
          }
        }
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma32(a, b0, acc);
        acc = mfma32(a, b1, acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) y[t][e] = fmaf(s, acc[e], y[t][e]);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (n[t] >= p.d_out) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tok = 4 * g + e;
      if (tok >= p.m) continue;
      if (p.ks == 1) p.y[(p.m0 + tok) * p.d_out + n[t]] = y[t][e];
      else p.part[(static_cast<int64_t>(ks) * kMaxMT + tok) * p.d_out + n[t]] = y[t][e];
    }
  }
}

struct ValuPlan {
  int chunks, cpw, ks, nblocks;
};

ValuPlan valu_plan(int64_t d_in, int64_t d_out) {
  ValuPlan pl{};
  pl.chunks = static_cast<int>(d_in / kChunk);
  pl.nblocks = static_cast<int>((d_out + kValuCols - 1) / kValuCols);
  // about 1024 workgroups, at least 4 chunks (one per wave) per workgroup
  int ks = std::max(1, (1024 + pl.nblocks - 1) / pl.nblocks);
  ks = std::min(ks, std::max(1, pl.chunks / 4));
  pl.cpw = std::min(kStage, (pl.chunks + ks - 1) / ks);
  pl.ks = (pl.chunks + pl.cpw - 1) / pl.cpw;
  return pl;
}

template <int BITS, int MT>
hipError_t valu_pass(DqParams p, hipStream_t st) {
  const ValuPlan pl = valu_plan(p.d_in, p.d_out);
  p.cpw = pl.cpw;
  p.ks = pl.ks;
  if (BITS == 4 && p.xbf16) dequant_valu_kernel<BITS, MT, BITS == 4><<<pl.nblocks * pl.ks, 256, 0, st>>>(p, p.g_idx);
  else dequant_valu_kernel<BITS, MT, false><<<pl.nblocks * pl.ks, 256, 0, st>>>(p, p.g_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.ks == 1) return e;
  const int64_t total = p.m * p.d_out;
  dequant_reduce_kernel<MT><<<static_cast<unsigned>((total + 255) / 256), 256, 0, st>>>(p.part, pl.ks, p.m0, p.m,
                                                                                      p.d_out, p.y);
  return hipGetLastError();
}

// MFMA path: 16 T NW columns per workgroup, its K range in stages of SC
// chunks.  One staged x serves all NW waves: 8 waves stage half the x bytes
// per column that 4 do, but measured slower on one-group chunks (55.5 against
// 53 us at 16 tokens, 28672 x 8192 4-bit) and on 4-bit act-order; faster only
// on 3-bit act-order at 8192 x 8192 (45 against 60 us).  One tile per wave
// measured best (more tiles raise the register count and lower occupancy).  Fewer K slices than the VALU plan, so that the partial sums
// (written and read back, 8 m d_out bytes per slice) stay a small part of the
// packed weights' bytes, while keeping 512 workgroups or more; never more
// slices than the VALU plan, whose partial buffer is the workspace.
constexpr int kMfmaTiles = 1;
constexpr int kMfmaStage = 16;
constexpr int kMfmaWaves = 4;

ValuPlan mfma_plan(int64_t d_in, int64_t d_out, int bits) {
  const ValuPlan vp = valu_plan(d_in, d_out);
  ValuPlan pl = vp;
  constexpr int kCols = 16 * kMfmaTiles * kMfmaWaves;
  pl.nblocks = static_cast<int>((d_out + kCols - 1) / kCols);
  const int64_t cap = std::max<int64_t>(d_in * bits / (512 * kMaxMT), (512 + pl.nblocks - 1) / pl.nblocks);
  const int ks = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(vp.ks, cap)));
  pl.cpw = (pl.chunks + ks - 1) / ks;
  pl.ks = (pl.chunks + pl.cpw - 1) / pl.cpw;
  return pl;
}

template <int BITS>
hipError_t mfma_pass(DqParams p, hipStream_t st) {
  const ValuPlan pl = mfma_plan(p.d_in, p.d_out, BITS);
  p.cpw = pl.cpw;
  p.ks = pl.ks;
  dequant_mfma_kernel<BITS, kMfmaTiles, kMfmaStage, kMfmaWaves>
      <<<pl.nblocks * pl.ks, 64 * kMfmaWaves, 0, st>>>(p, p.g_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.ks == 1) return e;
  const int64_t total = p.m * p.d_out;
  dequant_reduce_kernel<kMaxMT><<<static_cast<unsigned>((total + 255) / 256), 256, 0, st>>>(p.part, pl.ks, p.m0,
                                                                                          p.m, p.d_out, p.y);
  return hipGetLastError();
}

template <int BITS>
hipError_t dq_bits(const DqParams& p, hipStream_t st) {
  if (p.xbf16 && p.m >= 3) return mfma_pass<BITS>(p, st);
  if (p.m <= 1) return valu_pass<BITS, 1>(p, st);
  if (p.m <= 2) return valu_pass<BITS, 2>(p, st);
  if (p.m <= 4) return valu_pass<BITS, 4>(p, st);
  if (p.m <= 8) return valu_pass<BITS, 8>(p, st);
  return valu_pass<BITS, 16>(p, st);
}

// ------------------------------------------------- act-order channel order

// The stable rank of channel k by group: the number of channels of a smaller
// group plus those of its own group before it.  Every thread compares its key
// with all d_in keys, staged through LDS 256 at a time (a one-time step;
// d_in^2 comparisons).
__global__ __launch_bounds__(256) void order_rank_kernel(const int32_t* g_idx, int64_t d_in, int32_t* order,
                                                         int32_t* g_out) {
  __shared__ int32_t tile[256];
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int32_t key = g_idx[std::min(k, d_in - 1)];
  int64_t rank = 0;
  for (int64_t t0 = 0; t0 < d_in; t0 += 256) {
    __syncthreads();
    if (t0 + threadIdx.x < d_in) tile[threadIdx.x] = g_idx[t0 + threadIdx.x];
    __syncthreads();
    const int n = static_cast<int>(std::min<int64_t>(256, d_in - t0));
    for (int j = 0; j < n; ++j) {
      const int32_t g2 = tile[j];
      rank += (g2 < key || (g2 == key && t0 + j < k)) ? 1 : 0;
    }
  }
  if (k < d_in) {
    order[rank] = static_cast<int32_t>(k);
    g_out[rank] = key;
  }
}

// chunk c of the reordered layer (words c bits .. c bits + bits - 1 of column
// n): the codes of channels order[32 c + j], j < 32, taken from the original
// packed stream (code k at bits k bits .. k bits + bits - 1 of the column) and
// packed in the same stream order
template <int BITS>
__global__ __launch_bounds__(256) void order_pack_kernel(const int32_t* qweight, const int32_t* order, int64_t d_in,
                                                         int64_t d_out, int32_t* qout) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t chunks = d_in / kChunk;
  if (e >= chunks * d_out) return;
  const int64_t c = e / d_out, n = e - c * d_out;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  uint32_t words[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) words[i] = 0u;
#pragma unroll
  for (int j = 0; j < kChunk; ++j) {
    const int64_t k = order[c * kChunk + j];
    const int64_t b = k * BITS;
    const int64_t w = b >> 5;
    const int sh = static_cast<int>(b & 31);
    uint32_t v = static_cast<uint32_t>(qweight[w * d_out + n]) >> sh;
    if (sh + BITS > 32) v |= static_cast<uint32_t>(qweight[(w + 1) * d_out + n]) << (32 - sh);
    v &= mask;
    const int ob = j * BITS, ow = ob >> 5, os = ob & 31;
    words[ow] |= v << os;
    if (os + BITS > 32) words[ow + 1] |= v >> (32 - os);
  }
#pragma unroll
  for (int i = 0; i < BITS; ++i) qout[(c * BITS + i) * d_out + n] = static_cast<int32_t>(words[i]);
}

// xo[t][j] = x[t][order[j]] (2- or 4-byte elements)
template <typename E>
__global__ __launch_bounds__(256) void order_gather_kernel(const E* x, int64_t m, int64_t d_in, const int32_t* order,
                                                           E* xo) {
  const int64_t total = m * d_in;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = e / d_in, j = e - t * d_in;
    xo[e] = x[t * d_in + order[j]];
  }
}

}  // namespace

size_t dequant_workspace_bytes(int64_t m, int64_t d_in, int64_t d_out) {
  (void)m;
  const ValuPlan pl = valu_plan(d_in, d_out);
  if (pl.ks == 1) return 0;
  return (static_cast<size_t>(pl.ks) * kMaxMT * d_out * sizeof(float) + 255) & ~static_cast<size_t>(255);
}

namespace {
hipError_t dequant_passes(const void* x, bool x_bf16, int64_t m, int64_t d_in, const int32_t* qweight,
                          const float* scales, const int32_t* zeros, const int32_t* g_idx, const int32_t* xorder,
                          int bits, int64_t d_out, int n_groups, float* y, void* ws, hipStream_t st);
}  // namespace

hipError_t dequant_matmul_launch(const void* x, bool x_bf16, int64_t m, int64_t d_in, const int32_t* qweight,
                                 const float* scales, const int32_t* zeros, const int32_t* g_idx, int bits,
                                 int64_t d_out, int n_groups, float* y, void* ws, hipStream_t st) {
  return dequant_passes(x, x_bf16, m, d_in, qweight, scales, zeros, g_idx, nullptr, bits, d_out, n_groups, y, ws, st);
}

namespace {
hipError_t dequant_passes(const void* x, bool x_bf16, int64_t m, int64_t d_in, const int32_t* qweight,
                          const float* scales, const int32_t* zeros, const int32_t* g_idx, const int32_t* xorder,
                          int bits, int64_t d_out, int n_groups, float* y, void* ws, hipStream_t st) {
  const int64_t qbytes = d_in / kChunk * bits * d_out * 4, gbytes = static_cast<int64_t>(n_groups) * d_out * 4;
  if (qbytes >= (int64_t{1} << 31) || gbytes >= (int64_t{1} << 31)) return hipErrorInvalidValue;
  DqParams p{};
  p.qbytes = static_cast<uint32_t>(qbytes);
  p.gbytes = static_cast<uint32_t>(gbytes);
  p.x = x;
  p.xbf16 = x_bf16 ? 1 : 0;
  p.ldx = d_in;
  p.d_in = d_in;
  p.d_out = d_out;
  p.qweight = qweight;
  p.scales = scales;
  p.zeros = zeros;
  p.g_idx = g_idx;
  p.xorder = xorder;
  p.chunks = static_cast<int>(d_in / kChunk);
  p.y = y;
  p.part = static_cast<float*>(ws);
  for (int64_t m0 = 0; m0 < m; m0 += kMaxMT) {
    p.m0 = m0;
    p.m = std::min<int64_t>(kMaxMT, m - m0);
    hipError_t e;
    switch (bits) {
      case 2: e = dq_bits<2>(p, st); break;
      case 3: e = dq_bits<3>(p, st); break;
      case 4: e = dq_bits<4>(p, st); break;
      case 8: e = dq_bits<8>(p, st); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
}  // namespace

hipError_t dequant_order_launch(const int32_t* qweight, const int32_t* g_idx, int bits, int64_t d_in, int64_t d_out,
                                int32_t* qweight_out, int32_t* g_idx_out, int32_t* order, hipStream_t st) {
  order_rank_kernel<<<static_cast<unsigned>((d_in + 255) / 256), 256, 0, st>>>(g_idx, d_in, order, g_idx_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = d_in / kChunk * d_out;
  const unsigned grid = static_cast<unsigned>((total + 255) / 256);
  switch (bits) {
    case 2: order_pack_kernel<2><<<grid, 256, 0, st>>>(qweight, order, d_in, d_out, qweight_out); break;
    case 3: order_pack_kernel<3><<<grid, 256, 0, st>>>(qweight, order, d_in, d_out, qweight_out); break;
    case 4: order_pack_kernel<4><<<grid, 256, 0, st>>>(qweight, order, d_in, d_out, qweight_out); break;
    case 8: order_pack_kernel<8><<<grid, 256, 0, st>>>(qweight, order, d_in, d_out, qweight_out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t dequant_partial_bytes(int64_t m, int64_t d_in, int64_t d_out, bool x_bf16, int bits) {
  // what the passes of one call write: [ks][MT][d_out] floats for a VALU pass
  // of up to MT tokens, [ks][16][d_out] for an MFMA pass; the first pass and
  // a shorter last pass are the only distinct shapes
  size_t need = 0;
  const int64_t lens[2] = {std::min<int64_t>(kMaxMT, m), m % kMaxMT};
  for (int64_t len : lens) {
    if (len <= 0) continue;
    size_t b = 0;
    if (x_bf16 && len >= 3) {
      const ValuPlan pl = mfma_plan(d_in, d_out, bits);
      if (pl.ks > 1) b = static_cast<size_t>(pl.ks) * kMaxMT * d_out * sizeof(float);
    } else {
      const ValuPlan pl = valu_plan(d_in, d_out);
      const int64_t mt = len <= 1 ? 1 : len <= 2 ? 2 : len <= 4 ? 4 : len <= 8 ? 8 : 16;
      if (pl.ks > 1) b = static_cast<size_t>(pl.ks) * mt * d_out * sizeof(float);
    }
    need = std::max(need, b);
  }
  return need;
}

size_t dequant_ordered_workspace_bytes(int64_t m, int64_t d_in, int64_t d_out) {
  const size_t xb = (static_cast<size_t>(m) * d_in * sizeof(float) + 255) & ~static_cast<size_t>(255);
  return xb + dequant_workspace_bytes(m, d_in, d_out);
}

// ---------------------------------------------------- fixed scratch buffer
// The partial sums of the K slices in a buffer the library owns, for callers
// that cannot allocate.  One copy per GPU, at its own device address, kept
// until the process ends; every call on that GPU shares it.
static __device__ __align__(256) float scratch[kDequantScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t dequant_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      // the address of this device's copy (the current device); the host-side
      // name of the array is not a device address
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!ptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return hipSuccess;
}

hipError_t dequant_matmul_ordered_launch(const void* x, bool x_bf16, int64_t m, int64_t d_in, const int32_t* qweight,
                                         const float* scales, const int32_t* zeros, const int32_t* g_idx,
                                         const int32_t* order, int bits, int64_t d_out, int n_groups, float* y,
                                         void* ws, hipStream_t st) {
  const size_t xb = (static_cast<size_t>(m) * d_in * sizeof(float) + 255) & ~static_cast<size_t>(255);
  // the VALU passes (fp32 x, or bf16 with 1-2 tokens) gather x's channels as
  // they stage it; the MFMA passes read a gathered copy
  if (!x_bf16 || m <= 2)
    return dequant_passes(x, x_bf16, m, d_in, qweight, scales, zeros, g_idx, order, bits, d_out, n_groups, y,
                          static_cast<char*>(ws) + xb, st);
  const int64_t total = m * d_in;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>((total + 255) / 256, 4096));
  if (x_bf16)
    order_gather_kernel<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), m, d_in, order,
                                                        static_cast<uint16_t*>(ws));
  else
    order_gather_kernel<float><<<grid, 256, 0, st>>>(static_cast<const float*>(x), m, d_in, order,
                                                     static_cast<float*>(ws));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return dequant_matmul_launch(ws, x_bf16, m, d_in, qweight, scales, zeros, g_idx, bits, d_out, n_groups, y,
                               static_cast<char*>(ws) + xb, st);
}

}  // namespace gptq
