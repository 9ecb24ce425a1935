// Shared device helpers of the gfx950 GPTQ kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define GPTQ_DEV __device__ __forceinline__

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

namespace gptq {

constexpr int kWave = 64;

GPTQ_DEV int lane_id() { return static_cast<int>(threadIdx.x) & (kWave - 1); }

// bf16 bit pattern -> fp32 (exact)
GPTQ_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (finite values)
GPTQ_DEV uint16_t f32_to_bf16_rn(float x) {
  const uint32_t u = __float_as_uint(x);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// The exact split x = hi + mid + lo into bf16 parts: hi = bf16(x), the
// remainder x - hi is exact (Sterbenz), mid = bf16 of it, and the rest has at
// most 6 significant bits, so lo is exact (finite x above the fp32 normal
// range's bottom by 2^23).
GPTQ_DEV void split3(float x, uint16_t& h, uint16_t& m, uint16_t& l) {
  h = f32_to_bf16_rn(x);
  const float r1 = x - bf16_to_f32(h);
  m = f32_to_bf16_rn(r1);
  const float r2 = r1 - bf16_to_f32(m);
  l = f32_to_bf16_rn(r2);
}

// Broadcast the value of lane `src` of every 16-lane DPP row to the whole row.
// Every lane has a valid source, so no old value is needed (plain mov_dpp).
template <int src>
GPTQ_DEV float row_bcast(float v) {
  static_assert(src >= 0 && src < 16, "row lane");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + src, 0xf, 0xf, false));
}

// Reductions over one 16-lane row with DPP (quad_perm, row_half_mirror, row_mirror).
GPTQ_DEV float row_max16(float v) {
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xf, 0xf, false));  // quad_perm [1,0,3,2]
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xf, 0xf, false));  // quad_perm [2,3,0,1]
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xf, 0xf, false)); // row_half_mirror
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xf, 0xf, false)); // row_mirror
  return v;
}
GPTQ_DEV float row_sum16(float v) {
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xf, 0xf, false);
  return v;
}
GPTQ_DEV float row_min16(float v) {
  v = fminf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0xB1, 0xf, 0xf, false));
  v = fminf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x4E, 0xf, 0xf, false));
  v = fminf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x141, 0xf, 0xf, false));
  v = fminf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x140, 0xf, 0xf, false));
  return v;
}

}  // namespace gptq
