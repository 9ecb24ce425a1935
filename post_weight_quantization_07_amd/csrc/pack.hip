// Bit-packing of the codes into int32 words.
//
// The AutoGPTQ examples walkthrough names the packed tensor qweight; the
// practitioner blog, section 3.3, fixes the density (128 4-bit codes fill 64
// bytes).  Layout: qweight[w][n] holds bits [32w, 32w+32) of output row n's
// code stream, code (n, j) occupying stream bits [bits*j, bits*j + bits).
//
// One thread per (output row n, run of 32 codes): 32 codes make exactly
// `bits` words for every bit width, so a thread never shares a word.  Threads
// of a wave take consecutive rows, so each word store is coalesced across the
// wave; each thread reads its 32 codes as two 16-byte loads when aligned.
#include "gptq_common.h"
#include "gptq_internal.h"

#include <algorithm>

namespace gptq {
namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, int64_t d_out,
                                                   int64_t d_in, int bits, int32_t* __restrict__ qweight) {
  const int64_t n = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  const int64_t run = blockIdx.y;  // codes [32 run, 32 run + 32)
  if (n >= d_out) return;
  const int64_t j0 = 32 * run;
  const uint8_t* src = codes + n * d_in + j0;
  uint32_t c[32];
  if (j0 + 32 <= d_in && (d_in & 15) == 0) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(src);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(src + 16);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c[4 * q + k] = (a[q] >> (8 * k)) & 0xFFu;
        c[16 + 4 * q + k] = (b[q] >> (8 * k)) & 0xFFu;
      }
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) c[k] = (j0 + k < d_in) ? src[k] : 0u;
  }
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const uint32_t v = c[k] & mask;
    const int bit = bits * k;
    const int wi = bit >> 5, off = bit & 31;
    w[wi] |= v << off;
    if (off + bits > 32) w[wi + 1] |= v >> (32 - off);
  }
  const int64_t n_words = (d_in * bits + 31) / 32;
  const int64_t w0 = run * bits;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < bits && w0 + k < n_words) qweight[(w0 + k) * d_out + n] = static_cast<int32_t>(w[k]);
}

}  // namespace

hipError_t pack_launch(const uint8_t* codes, int64_t d_out, int64_t d_in, int bits, int32_t* qweight,
                       hipStream_t stream) {
  if (d_out <= 0 || d_in <= 0) return hipSuccess;
  const int64_t runs = (d_in + 31) / 32;
  dim3 grid(static_cast<unsigned>((d_out + 255) / 256), static_cast<unsigned>(runs));
  PhaseScope ph(kPhPack, stream);
  pack_kernel<<<grid, 256, 0, stream>>>(codes, d_out, d_in, bits, qweight);
  return hipGetLastError();
}

}  // namespace gptq
