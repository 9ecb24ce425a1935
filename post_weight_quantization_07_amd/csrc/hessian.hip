// S += X^T X on gfx950 matrix cores.
//
// GPTQ 实战 ch.5, section 5.1.7: the layer Hessian is X X^T (up to a constant)
// estimated from calibration activations.  X arrives token-major
// ([tokens, d_in]), so the contraction runs over the strided token axis.
//
// Work split: the d_in x d_in output is cut into tiles of the upper triangle
// (diagonal tiles computed whole); the token axis is cut into n_split equal
// slices so a launch has enough workgroups for 256 CUs.  Each workgroup owns
// one (tile, slice) pair and stores its fp32 partial tile.  A second, wide
// kernel sums the partials of every tile in slice order and adds the result
// to S and to its mirror.  The sum order is fixed, so the result does not
// depend on scheduling.
//
// bf16 path: 256x256 tile, 4 waves of 128x128, v_mfma_f32_32x32x16_bf16.
//   X moves to LDS with buffer_load ... lds (no VGPRs, no register
//   transposition) through a ring of eight 16-token stages, and the MFMA
//   operands come out of the token-major LDS tile through ds_read_b64_tr_b16.
// fp32 path: 128x128 tile, 4 waves of 64x64, v_mfma_f32_16x16x4_f32, LDS
//   holds [token][channel] rows padded to 144 floats.
// fp32 path on the bf16 matrix cores (large calls): X is split exactly into
//   three bf16 planes, the bf16 kernel runs the tiles of the part products
//   above 2^-24, and a reduction combines them (see the plane kernels below).
#include "gptq_common.h"
#include "gptq_internal.h"

#include <algorithm>

namespace gptq {
namespace {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 256;

struct HessParams {
  const void* X;
  int64_t ldx;
  int64_t n_tokens;
  int32_t d_in;
  int32_t nt;
  int32_t n_tiles;
  int32_t n_split;
  int64_t split_len;
  float* partial;
  int32_t planes;  // 1: the tiles of the three-plane list below (fp32 X split into bf16 parts)
};

// Tiles of the upper triangle in "super-tile" order: 4x4 blocks of tiles
// row-major over the block-upper triangle, tiles row-major inside a block.
// Consecutive tiles then share few row and column blocks of X.
GPTQ_DEV void tile_coords(int pos, int nt, int& I, int& J) {
  const int ns = (nt + 3) >> 2;
  for (int si = 0; si < ns; ++si) {
    const int ri = min(4, nt - 4 * si);
    for (int sj = si; sj < ns; ++sj) {
      const int cj = min(4, nt - 4 * sj);
      const int cnt = (si == sj) ? ri * (ri + 1) / 2 : ri * cj;
      if (pos >= cnt) {
        pos -= cnt;
        continue;
      }
      if (si == sj) {
        int i = 0;
        while (pos >= ri - i) {
          pos -= ri - i;
          ++i;
        }
        I = 4 * si + i;
        J = 4 * si + i + pos;
      } else {
        I = 4 * si + pos / cj;
        J = 4 * sj + pos % cj;
      }
      return;
    }
  }
  I = J = 0;
}

// Row-major upper triangle of an nt x nt tile grid: u -> (i, j), i <= j.
GPTQ_DEV void tri_coords(int u, int nt, int& i, int& j) {
  i = 0;
  while (u >= nt - i) {
    u -= nt - i;
    ++i;
  }
  j = i + u;
}

// fp32 X enters as three bf16 planes X = Xh + Xm + Xl (exact split), stored
// side by side, each nt tiles wide.  X^T X is the sum of the part products
// above 2^-24 of the total: Xh^T Xh + Xm^T Xm + (Xh^T Xm + Xh^T Xl) + their
// transposes.  The tile list (I, J index 256-column blocks of the planes):
//   [0, T)             Xh^T Xh, upper triangle (T = nt (nt + 1) / 2)
//   [T, T + nt^2)       Xh^T Xm, every tile
//   [T + nt^2, ...)     Xh^T Xl, every tile
//   [T + 2 nt^2, ...)   Xm^T Xm, upper triangle
GPTQ_DEV void plane_tile_coords(int t, int nt, int& I, int& J) {
  const int T = nt * (nt + 1) / 2, Q = nt * nt;
  if (t < T) {
    tri_coords(t, nt, I, J);
  } else if (t < T + 2 * Q) {
    const int u = t - T, pl = u / Q, v = u % Q;
    I = v / nt;
    J = (1 + pl) * nt + v % nt;
  } else {
    tri_coords(t - T - 2 * Q, nt, I, J);
    I += nt;
    J += nt;
  }
}

// Work item of workgroup b.  Workgroups are dispatched round-robin over the
// 8 XCDs (b % 8), each with its own L2.  The item list (tile groups in
// super-tile order, every group swept over all token slices, slice-major
// inside the group) is cut into 8 contiguous pieces, one per XCD, so the ~32
// workgroups resident on one XCD work on a compact group of tiles and the
// same token slice, and share X through that XCD's L2.
GPTQ_DEV void work_item(int b, int n_tiles, int n_split, int& tile_pos, int& split) {
  constexpr int kXcd = 8;
  const int B = n_tiles * n_split;
  const int x = b % kXcd, l = b / kXcd;
  const int base = B / kXcd, rem = B % kXcd;
  const int q = x * base + min(x, rem) + l;
  int g = 0;
  while (g + 1 < kXcd && q >= n_split * (((g + 1) * n_tiles) / kXcd)) ++g;
  const int g0 = (g * n_tiles) / kXcd, g1 = ((g + 1) * n_tiles) / kXcd;
  const int local = q - n_split * g0;
  const int gsize = g1 - g0;
  split = local / gsize;
  tile_pos = g0 + local % gsize;
}

// Partial tiles are stored in register order: fragment f of wave w, lane l
// holds 4 floats at ((w * NF + f) * 64 + l) * 4 of the (tile, slice) block.
GPTQ_DEV float* partial_tile(const HessParams& p, int t, int split, int64_t elems) {
  return p.partial + (static_cast<int64_t>(t) * p.n_split + split) * elems;
}

// ============================================================ bf16 path ====
constexpr int kBTile = 256;

#define GPTQ_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

// Buffer resource over one stage of X: `rows` token rows starting at Xs.  Reads
// past the end (tokens beyond the slice) return zeros in hardware.
GPTQ_DEV __amdgpu_buffer_rsrc_t stage_rsrc(const uint16_t* Xs, int rows, int ldx) {
  // every field is workgroup-uniform; say so, or the compiler builds a waterfall loop
  const uint64_t a = reinterpret_cast<uint64_t>(Xs);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane(rows * ldx * 2);
  void* base = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0), n, 0x00020000);
}

// X moves to LDS by buffer_load ... lds in 16-token stages through a ring of
// eight (7 in flight), and each stage's MFMA operands are read from LDS while
// the previous stage's MFMAs run: every v_mfma is paired with one
// ds_read_b64_tr_b16 of the next stage, so the matrix pipe never waits for an
// operand at a stage boundary.  One barrier per stage: it publishes the next
// stage's DMA to all waves and frees the slot read two stages ago.
//
// LDS: token rows of 512 bytes (256 channels).  The 16-byte chunk c of row r
// sits at physical chunk c ^ 2 (r & 3) ^ 8 bit1(c): for one transposed read,
// the 32 lanes of each half-wave then cover all 64 banks exactly once.
constexpr int kPStage = 16;               // tokens per stage
constexpr int kPSlots = 8;                // ring depth
constexpr int kPOpBytes = kPStage * 512;  // one operand stage: 8 KB

// logical chunk held by physical chunk p of token row `row` (inverse swizzle)
GPTQ_DEV int pipe_logical_chunk(int p, int row) {
  const int j = row & 3;
  const int c1 = ((p >> 1) & 1) ^ (j & 1);
  const int c2 = ((p >> 2) & 1) ^ (j >> 1);
  const int c3 = ((p >> 3) & 1) ^ c1;
  return (p & 0x11) | (c1 << 1) | (c2 << 2) | (c3 << 3);
}

// One operand stage (16 rows x 512 bytes = eight 1 KB pieces); wave w moves
// pieces 2w and 2w + 1.  Lane l of a piece writes bytes [16 l, 16 l + 16).
GPTQ_DEV void pipe_dma(__amdgpu_buffer_rsrc_t rs, uint8_t* slot, int ldx, int col0, int d_in, int wave_u,
                       int lane) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = 2 * wave_u + u;
    const int row = 2 * q + (lane >> 5);
    const int col = col0 + 8 * pipe_logical_chunk(lane & 31, row);
    const uint32_t voff = (col < d_in) ? static_cast<uint32_t>((row * ldx + col) * 2) : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(slot + q * 1024), 16, voff, 0, 0, 0);
  }
}

// Byte offsets of a lane's low transposed read for the four 32-channel MFMA
// tiles of wave block wb; the high read (tokens +4) is 2048 bytes further.
struct PipeLane {
  uint32_t off[4];
};
GPTQ_DEV PipeLane pipe_lane(int lane, int wb) {
  const int g = lane >> 4, s = lane & 15;
  const int row = 8 * (g >> 1) + (s >> 2);
  const int j = s >> 2;
  const int c1 = g & 1, c0 = (s >> 1) & 1;
  PipeLane t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 16 * wb + 4 * i + 2 * c1 + c0;
    const int pc = c ^ (2 * j) ^ (c1 << 3);
    t.off[i] = static_cast<uint32_t>(row * 512 + pc * 16 + (s & 1) * 8);
  }
  return t;
}

GPTQ_DEV bf16x8_t pipe_operand(const uint8_t* slot, uint32_t off) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
  uint8_t* b = const_cast<uint8_t*>(slot) + off;
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)b);
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(b + 2048));
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8_t;
  const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// operands of one stage, in the order the MFMAs below consume them
GPTQ_DEV void pipe_read(const uint8_t* A, const uint8_t* B, const PipeLane& la, const PipeLane& lb,
                        bf16x8_t (&a)[4], bf16x8_t (&b)[4]) {
  a[0] = pipe_operand(A, la.off[0]);
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = pipe_operand(B, lb.off[j]);
#pragma unroll
  for (int i = 1; i < 4; ++i) a[i] = pipe_operand(A, la.off[i]);
}

GPTQ_DEV void pipe_mfma(const bf16x8_t (&a)[4], const bf16x8_t (&b)[4], f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// MFMAs of the current stage with the reads of the next one interleaved 1:1,
// and the stage's four DMA loads (issued just before) spread one per four
// MFMAs: issued back to back they held the wave at the address unit instead
// of letting it issue MFMAs (measured 5% faster on the whole call)
GPTQ_DEV void pipe_step(const bf16x8_t (&a)[4], const bf16x8_t (&b)[4], const uint8_t* nA, const uint8_t* nB,
                        const PipeLane& la, const PipeLane& lb, bf16x8_t (&na)[4], bf16x8_t (&nb)[4],
                        f32x16_t (&acc)[4][4]) {
  pipe_read(nA, nB, la, lb, na, nb);
  pipe_mfma(a, b, acc);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                    // one LDS read
    if ((k & 3) == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one DMA load
  }
}

__global__ __launch_bounds__(kThreads, 1) void hessian_bf16_pipe_kernel(HessParams p) {
  // one array per slot: the compiler's wait insertion then sees that reads of
  // one slot do not alias DMA writes in flight into another
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[kPOpBytes], sA1[kPOpBytes], sA2[kPOpBytes],
      sA3[kPOpBytes], sA4[kPOpBytes], sA5[kPOpBytes], sA6[kPOpBytes], sA7[kPOpBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[kPOpBytes], sB1[kPOpBytes], sB2[kPOpBytes],
      sB3[kPOpBytes], sB4[kPOpBytes], sB5[kPOpBytes], sB6[kPOpBytes], sB7[kPOpBytes];
  int t, split, I, J;
  work_item(blockIdx.x, p.n_tiles, p.n_split, t, split);
  if (p.planes)
    plane_tile_coords(t, p.nt, I, J);
  else
    tile_coords(t, p.nt, I, J);
  const int64_t k0 = static_cast<int64_t>(split) * p.split_len;
  const int64_t k1 = min(p.n_tokens, k0 + p.split_len);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int colA = I * kBTile, colB = J * kBTile;
  const int ldx = static_cast<int>(p.ldx);
  const uint16_t* X = static_cast<const uint16_t*>(p.X);
  const PipeLane la = pipe_lane(lane, wm), lb = pipe_lane(lane, wn);

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // stages run in blocks of eight; stages past the slice end read zeros
  const int nstage = (k1 > k0) ? static_cast<int>((k1 - k0 + kPStage - 1) / kPStage) : 0;
  const int nblk = (nstage + kPSlots - 1) / kPSlots;
  auto slotA = [&](int u) -> uint8_t* {
    switch (u & 7) {
      case 0: return sA0; case 1: return sA1; case 2: return sA2; case 3: return sA3;
      case 4: return sA4; case 5: return sA5; case 6: return sA6; default: return sA7;
    }
  };
  auto slotB = [&](int u) -> uint8_t* {
    switch (u & 7) {
      case 0: return sB0; case 1: return sB1; case 2: return sB2; case 3: return sB3;
      case 4: return sB4; case 5: return sB5; case 6: return sB6; default: return sB7;
    }
  };
  auto issue = [&](int s, int slot) {
    const int64_t t0 = k0 + static_cast<int64_t>(s) * kPStage;
    const int64_t rem = k1 - t0;
    const int left = rem <= 0 ? 0 : (rem >= kPStage ? kPStage : static_cast<int>(rem));
    const __amdgpu_buffer_rsrc_t rs = stage_rsrc(X + t0 * p.ldx, left, ldx);
    pipe_dma(rs, slotA(slot), ldx, colA, p.d_in, wave, lane);
    pipe_dma(rs, slotB(slot), ldx, colB, p.d_in, wave, lane);
  };
  bf16x8_t a0[4], b0[4], a1[4], b1[4];
  // on a diagonal tile the lower-left quadrant is the mirror of the upper-right
  // one: its wave only moves its share of the operands (the reduction mirrors)
  const bool idle = (I == J) && wm == 1 && wn == 0;
  if (idle && nblk >= 2) {
    for (int x = 0; x < 7; ++x) issue(x, x);
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(24));
    __builtin_amdgcn_s_barrier();
    for (int blk = 0; blk + 1 < nblk; ++blk) {
      const int s = blk * kPSlots;
#pragma unroll
      for (int u = 0; u < 8; u += 2) {
        __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(20));
        __builtin_amdgcn_s_barrier();
        issue(s + u + 7, u + 7);
        __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(20));
        __builtin_amdgcn_s_barrier();
        issue(s + u + 8, u + 8);
      }
    }
    const int L = (nblk - 1) * kPSlots;
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(20));
    __builtin_amdgcn_s_barrier();
    issue(L + 7, 7);
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(20));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(16));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(12));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(8));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(4));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(0));
    __builtin_amdgcn_s_barrier();
  } else if (idle) {
#pragma unroll
    for (int x = 0; x < 8; ++x) issue(x, x);
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(0));
    __builtin_amdgcn_s_barrier();
  } else if (nblk >= 2) {
    // Stage s lives in slot s % 8 and its operands in register set s % 2.
    // Before stage s: wait for the DMA of stage s + 1 (stages s + 2 .. s + 6
    // stay in flight: 4 loads each per wave), barrier, refill the slot of
    // stage s - 1 (read during stage s - 2, consumed by everyone's MFMAs of
    // stage s - 1, which precede the barrier) with stage s + 7.
    for (int x = 0; x < 7; ++x) issue(x, x);
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(24));
    __builtin_amdgcn_s_barrier();
    pipe_read(slotA(0), slotB(0), la, lb, a0, b0);
    for (int blk = 0; blk + 1 < nblk; ++blk) {
      const int s = blk * kPSlots;
#pragma unroll
      for (int u = 0; u < 8; u += 2) {
        __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(20));
        __builtin_amdgcn_s_barrier();
        issue(s + u + 7, u + 7);
        pipe_step(a0, b0, slotA(u + 1), slotB(u + 1), la, lb, a1, b1, acc);
        __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(20));
        __builtin_amdgcn_s_barrier();
        issue(s + u + 8, u + 8);
        pipe_step(a1, b1, slotA(u + 2), slotB(u + 2), la, lb, a0, b0, acc);
      }
    }
    // last block: its first stage issues the final stage, then the waits drain
    const int L = (nblk - 1) * kPSlots;
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(20));
    __builtin_amdgcn_s_barrier();
    issue(L + 7, 7);
    pipe_step(a0, b0, slotA(1), slotB(1), la, lb, a1, b1, acc);
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(20));
    __builtin_amdgcn_s_barrier();
    pipe_step(a1, b1, slotA(2), slotB(2), la, lb, a0, b0, acc);
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(16));
    __builtin_amdgcn_s_barrier();
    pipe_step(a0, b0, slotA(3), slotB(3), la, lb, a1, b1, acc);
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(12));
    __builtin_amdgcn_s_barrier();
    pipe_step(a1, b1, slotA(4), slotB(4), la, lb, a0, b0, acc);
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(8));
    __builtin_amdgcn_s_barrier();
    pipe_step(a0, b0, slotA(5), slotB(5), la, lb, a1, b1, acc);
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(4));
    __builtin_amdgcn_s_barrier();
    pipe_step(a1, b1, slotA(6), slotB(6), la, lb, a0, b0, acc);
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(0));
    __builtin_amdgcn_s_barrier();
    pipe_step(a0, b0, slotA(7), slotB(7), la, lb, a1, b1, acc);
    pipe_mfma(a1, b1, acc);
  } else if (nblk == 1) {
    // at most eight stages: load them all, then compute
#pragma unroll
    for (int x = 0; x < 8; ++x) issue(x, x);
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(0));
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      pipe_read(slotA(u), slotB(u), la, lb, a0, b0);
      pipe_mfma(a0, b0, acc);
    }
  }
  // 32x32 accumulator layout: element r of lane l is tile row 8 (r / 4) +
  // 4 (l / 32) + r % 4, column l % 32.  Stored as fragments of 4 rows; the
  // accumulators only leave through stores, which read AGPRs directly
  float* mine = partial_tile(p, t, split, static_cast<int64_t>(kBTile) * kBTile);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<f32x4_t*>(mine + (((wave * 64 + (i * 4 + j) * 4 + e) * 64 + lane) << 2)) =
            f32x4_t{acc[i][j][4 * e], acc[i][j][4 * e + 1], acc[i][j][4 * e + 2], acc[i][j][4 * e + 3]};
}

// ============================================================ fp32 path ====
constexpr int kFTile = 128;
constexpr int kFStage = 32;    // tokens per stage
constexpr int kFPitch = 144;   // floats per LDS row (128 + 16 pad)

// d_in is a multiple of 4, so a 4-channel group is either wholly inside or outside.
GPTQ_DEV void load_stage_f32(const float* __restrict__ X, int64_t ldx, int64_t row0, int64_t row_end,
                             int col0, int d_in, int tid, f32x4_t (&r)[4]) {
  const int c = col0 + 4 * (tid & 31);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t row = row0 + (tid >> 5) + 8 * u;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (c < d_in && row < row_end) v = *reinterpret_cast<const f32x4_t*>(X + row * ldx + c);
    r[u] = v;
  }
}

GPTQ_DEV void store_stage_f32(float* lds, int tid, const f32x4_t (&r)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
    *reinterpret_cast<f32x4_t*>(lds + ((tid >> 5) + 8 * u) * kFPitch + 4 * (tid & 31)) = r[u];
}

__global__ __launch_bounds__(kThreads, 2) void hessian_f32_kernel(HessParams p) {
  __shared__ __attribute__((aligned(16))) float lds[2][2][kFStage * kFPitch];
  int t, split, I, J;
  work_item(blockIdx.x, p.n_tiles, p.n_split, t, split);
  tile_coords(t, p.nt, I, J);
  const bool diag = (I == J);
  const int64_t k0 = static_cast<int64_t>(split) * p.split_len;
  const int64_t k1 = min(p.n_tokens, k0 + p.split_len);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const float* X = static_cast<const float*>(p.X);

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nstage = (k1 > k0) ? static_cast<int>((k1 - k0 + kFStage - 1) / kFStage) : 0;
  f32x4_t ra[4], rb[4];
  if (nstage > 0) {
    load_stage_f32(X, p.ldx, k0, k1, I * kFTile, p.d_in, tid, ra);
    if (!diag) load_stage_f32(X, p.ldx, k0, k1, J * kFTile, p.d_in, tid, rb);
    store_stage_f32(lds[0][0], tid, ra);
    if (!diag) store_stage_f32(lds[0][1], tid, rb);
  }
  __syncthreads();
  for (int s = 0; s < nstage; ++s) {
    const int cur = s & 1;
    const bool more = (s + 1) < nstage;
    if (more) {
      const int64_t row0 = k0 + static_cast<int64_t>(s + 1) * kFStage;
      load_stage_f32(X, p.ldx, row0, k1, I * kFTile, p.d_in, tid, ra);
      if (!diag) load_stage_f32(X, p.ldx, row0, k1, J * kFTile, p.d_in, tid, rb);
    }
    const float* A = lds[cur][0];
    const float* B = diag ? lds[cur][0] : lds[cur][1];
#pragma unroll
    for (int k4 = 0; k4 < kFStage / 4; ++k4) {
      const int kr = 4 * k4 + (lane >> 4);
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = A[kr * kFPitch + wm * 64 + 16 * i + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = B[kr * kFPitch + wn * 64 + 16 * j + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_stage_f32(lds[cur ^ 1][0], tid, ra);
      if (!diag) store_stage_f32(lds[cur ^ 1][1], tid, rb);
    }
    __syncthreads();
  }
  float* mine = partial_tile(p, t, split, static_cast<int64_t>(kFTile) * kFTile);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<f32x4_t*>(mine + (((wave * 16 + i * 4 + j) * 64 + lane) << 2)) = acc[i][j];
}

// ========================================================= slice reduce ====
// One workgroup per (tile, wave w, MFMA tile i, j): a BS x BS block made of
// NE fragments x 64 lanes x 4 rows.  Sums the n_split partials of the block
// in slice order, stages the sum in LDS and adds it to S row by row, then to
// the mirror block (tile (J, I)) column by column, so both updates are
// coalesced.  On a diagonal tile of the bf16 kernel the lower-left quadrant
// was not computed (its wave idles): the upper-right quadrant's blocks write
// it as their mirror.  Every element of S is updated by exactly one thread.
//   bf16 (TILE 256, BS 32, NE 4): fragment e, lane l -> rows 8 e + 4 (l / 32) + r, col l % 32
//   fp32 (TILE 128, BS 16, NE 1): lane l -> rows 4 (l / 16) + r, col l % 16
template <int TILE, int BS, int NE>
__global__ __launch_bounds__(NE * 64) void hessian_reduce_kernel(const float* __restrict__ partial, int n_split,
                                                                 int nt, int d, float* __restrict__ S) {
  __shared__ float blk[BS][BS + 1];
  const int t = blockIdx.x >> 6, b = blockIdx.x & 63;
  int I, J;
  tile_coords(t, nt, I, J);
  const int w = b >> 4, i = (b >> 2) & 3, j = b & 3;
  if (I == J && w == 2 && NE == 4) return;  // filled by the mirror of quadrant 1
  const bool mirror = (I != J) || (w == 1 && NE == 4);
  const int tid = threadIdx.x, e = tid >> 6, lane = tid & 63;
  constexpr int64_t kElems = static_cast<int64_t>(TILE) * TILE;
  const int64_t off = static_cast<int64_t>((w * 16 * NE + (i * 4 + j) * NE + e) * 64 + lane) << 2;
  const float* src = partial + static_cast<int64_t>(t) * n_split * kElems + off;
  // sixteen slices' loads in flight at a time (a plain loop waits for each
  // load before the next), added in slice order
  f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < n_split; k += 16) {
    f32x4_t v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      v[u] = (k + u < n_split) ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src + (k + u) * kElems))
                               : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (k + u < n_split) sum += v[u];
  }
  const int r0 = (NE == 4) ? 8 * e + 4 * (lane >> 5) : 4 * (lane >> 4);
  const int c = lane & (BS - 1);
#pragma unroll
  for (int r = 0; r < 4; ++r) blk[r0 + r][c] = sum[r];
  __syncthreads();
  const int row0 = I * TILE + (w >> 1) * (TILE / 2) + BS * i;
  const int col0 = J * TILE + (w & 1) * (TILE / 2) + BS * j;
  // all reads of S first, then the writes (each element of S is read and
  // written by one thread only)
  constexpr int NI = BS * BS / (NE * 64);
  float vd[NI], vm[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int idx = tid + u * NE * 64, rr = idx / BS, cc = idx % BS;
    vd[u] = (row0 + rr < d && col0 + cc < d) ? S[static_cast<int64_t>(row0 + rr) * d + col0 + cc] : 0.f;
    vm[u] = (mirror && col0 + rr < d && row0 + cc < d) ? S[static_cast<int64_t>(col0 + rr) * d + row0 + cc] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int idx = tid + u * NE * 64, rr = idx / BS, cc = idx % BS;
    if (row0 + rr < d && col0 + cc < d) S[static_cast<int64_t>(row0 + rr) * d + col0 + cc] = vd[u] + blk[rr][cc];
    if (mirror && col0 + rr < d && row0 + cc < d) S[static_cast<int64_t>(col0 + rr) * d + row0 + cc] = vm[u] + blk[cc][rr];
  }
}

// ======================================================== fp32 X planes ====
// X (fp32, [n, ldx]) -> X3 (bf16, [n, 3 dp]): part q of channel c at q dp + c
// (hi, mid, lo of the exact split), zeros for d <= c < dp.  d is a multiple
// of 4 and rows of X are 16-byte aligned.
__global__ __launch_bounds__(256) void plane_split_kernel(const float* __restrict__ X, int64_t ldx, int64_t n, int d,
                                                         int dp, uint16_t* __restrict__ X3) {
  const int64_t q = dp / 4;
  const int64_t total = n * q;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < total; idx += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = idx / q;
    const int c = static_cast<int>(idx % q) * 4;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (c < d) v = *reinterpret_cast<const f32x4_t*>(X + t * ldx + c);
    uint16_t h[4], m[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split3(v[e], h[e], m[e], l[e]);
    uint16_t* row = X3 + t * 3 * static_cast<int64_t>(dp) + c;
    typedef __attribute__((__vector_size__(4 * sizeof(uint16_t)))) uint16_t u16x4_t;
    *reinterpret_cast<u16x4_t*>(row) = u16x4_t{h[0], h[1], h[2], h[3]};
    *reinterpret_cast<u16x4_t*>(row + dp) = u16x4_t{m[0], m[1], m[2], m[3]};
    *reinterpret_cast<u16x4_t*>(row + 2 * dp) = u16x4_t{l[0], l[1], l[2], l[3]};
  }
}

// S += Xh^T Xh + Xm^T Xm + Xh^T Xm + (Xh^T Xm)^T + Xh^T Xl + (Xh^T Xl)^T from
// the partial tiles of the plane list.  One workgroup per 32x32 block (rb, cb)
// of an upper-triangle output tile (I, J) of S: the blocks at (rb, cb) of the
// tiles Xh^T Xh (I, J), Xh^T Xm (I, J), Xh^T Xl (I, J), Xm^T Xm (I, J), plus
// the transposes of the blocks at (cb, rb) of Xh^T Xm (J, I) and Xh^T Xl
// (J, I), each summed over the slices in slice order.  On a diagonal tile
// only blocks with rb <= cb run, and the mirror of every block above the
// diagonal is written too, so every element of S is updated by one thread.
__global__ __launch_bounds__(256) void plane_reduce_kernel(const float* __restrict__ partial, int n_split, int nt,
                                                          int d, float* __restrict__ S) {
  __shared__ float D[32][33], Tr[32][33];
  const int t = blockIdx.x >> 6, b = blockIdx.x & 63;
  int I, J;
  tri_coords(t, nt, I, J);
  const int rb = b >> 3, cb = b & 7;
  if (I == J && rb > cb) return;
  const int T = nt * (nt + 1) / 2, Q = nt * nt;
  constexpr int64_t kElems = static_cast<int64_t>(kBTile) * kBTile;
  const int tid = threadIdx.x, e = tid >> 6, lane = tid & 63;
  // this thread's 4 floats of block (r, c) of a tile in register order
  auto off = [&](int r, int c) -> int64_t {
    const int w = 2 * (r >> 2) + (c >> 2), i = r & 3, j = c & 3;
    return static_cast<int64_t>(((w * 64 + (i * 4 + j) * 4 + e) * 64 + lane) << 2);
  };
  const int64_t od = off(rb, cb), ot = off(cb, rb);
  const float* src[6] = {partial + static_cast<int64_t>(t) * n_split * kElems + od,                      // hh (I, J)
                         partial + static_cast<int64_t>(T + I * nt + J) * n_split * kElems + od,         // hm (I, J)
                         partial + static_cast<int64_t>(T + Q + I * nt + J) * n_split * kElems + od,     // hl (I, J)
                         partial + static_cast<int64_t>(T + 2 * Q + t) * n_split * kElems + od,          // mm (I, J)
                         partial + static_cast<int64_t>(T + J * nt + I) * n_split * kElems + ot,         // hm (J, I)
                         partial + static_cast<int64_t>(T + Q + J * nt + I) * n_split * kElems + ot};    // hl (J, I)
  f32x4_t sum[6];
#pragma unroll
  for (int x = 0; x < 6; ++x) sum[x] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < n_split; k += 4) {
    f32x4_t v[4][6];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int x = 0; x < 6; ++x)
        v[u][x] = (k + u < n_split)
                      ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src[x] + (k + u) * kElems))
                      : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int x = 0; x < 6; ++x)
        if (k + u < n_split) sum[x] += v[u][x];
  }
  // the small parts first
  const f32x4_t dsum = sum[0] + (sum[1] + (sum[2] + sum[3]));
  const f32x4_t tsum = sum[4] + sum[5];
  const int r0 = 8 * e + 4 * (lane >> 5), c = lane & 31;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    D[r0 + r][c] = dsum[r];
    Tr[r0 + r][c] = tsum[r];
  }
  __syncthreads();
  // a block on the diagonal of S takes its upper triangle and that
  // triangle's mirror, so S stays exactly symmetric
  const bool diag = (I == J) && (rb == cb);
  const bool mirror = (I != J) || (rb < cb);
  const int row0 = I * kBTile + 32 * rb, col0 = J * kBTile + 32 * cb;
  float vd[4], vm[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = tid + u * 256, rr = idx >> 5, cc = idx & 31;
    const bool wd = row0 + rr < d && col0 + cc < d && (!diag || rr <= cc);
    const bool wm = col0 + rr < d && row0 + cc < d && (mirror || (diag && cc < rr));
    vd[u] = wd ? S[static_cast<int64_t>(row0 + rr) * d + col0 + cc] : 0.f;
    vm[u] = wm ? S[static_cast<int64_t>(col0 + rr) * d + row0 + cc] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = tid + u * 256, rr = idx >> 5, cc = idx & 31;
    const bool wd = row0 + rr < d && col0 + cc < d && (!diag || rr <= cc);
    const bool wm = col0 + rr < d && row0 + cc < d && (mirror || (diag && cc < rr));
    if (wd) S[static_cast<int64_t>(row0 + rr) * d + col0 + cc] = vd[u] + (D[rr][cc] + Tr[cc][rr]);
    if (wm) S[static_cast<int64_t>(col0 + rr) * d + row0 + cc] = vm[u] + (D[cc][rr] + Tr[rr][cc]);
  }
}

}  // namespace

// fp32 X goes through the three-plane path when the product is large enough
// to repay the split pass (N d^2 >= 4e9) and the planes' partial tiles stay
// modest (d_in <= 8192); it runs X in passes of at most 512 MiB of planes.
constexpr double kPlaneMinWork = 4e9;
constexpr int64_t kPlaneMaxDim = 8192;
constexpr int64_t kPlaneBufBytes = int64_t{512} << 20;

static HessPlan plane_plan(int64_t d_in, int64_t n_tokens, int n_cu) {
  HessPlan pl{};
  pl.planes = true;
  pl.tile = kBTile;
  pl.stage_tokens = kPStage * kPSlots;
  pl.nt = static_cast<int>((d_in + kBTile - 1) / kBTile);
  const int64_t dp = static_cast<int64_t>(pl.nt) * kBTile;
  pl.n_tiles = pl.nt * (pl.nt + 1) + 2 * pl.nt * pl.nt;
  const int64_t per_token = 3 * dp * static_cast<int64_t>(sizeof(uint16_t));
  const int64_t cap = std::max<int64_t>(pl.stage_tokens, (kPlaneBufBytes / per_token) / pl.stage_tokens * pl.stage_tokens);
  pl.chunk = std::min<int64_t>(n_tokens, cap);
  // slice count: time of the partial-tile rounds (about 3 us per tile and
  // 128-token stage) plus the reduction's read of the partials (5 TB/s)
  const int64_t slots = n_cu > 0 ? n_cu : 256;
  const int64_t stages = (pl.chunk + pl.stage_tokens - 1) / pl.stage_tokens;
  const double tile_bytes = static_cast<double>(kBTile) * kBTile * sizeof(float);
  int best = 1;
  double best_cost = 1e300;
  for (int s = 1; s <= std::min<int64_t>(64, stages); ++s) {
    const int64_t waves = (static_cast<int64_t>(pl.n_tiles) * s + slots - 1) / slots;
    const int64_t per = (stages + s - 1) / s;
    const double cost = 3.0 * waves * per + pl.n_tiles * s * tile_bytes / 5e6;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  pl.split_len = ((stages + best - 1) / best) * pl.stage_tokens;
  pl.n_split = static_cast<int>((pl.chunk + pl.split_len - 1) / pl.split_len);
  pl.partial_bytes = static_cast<size_t>(pl.n_tiles) * pl.n_split * static_cast<size_t>(tile_bytes);
  pl.planes_off = (pl.partial_bytes + 255) & ~static_cast<size_t>(255);
  pl.ws_bytes = pl.planes_off + static_cast<size_t>(pl.chunk * per_token);
  return pl;
}

HessPlan hessian_plan(int64_t d_in, int64_t n_tokens, bool bf16, int n_cu) {
  if (!bf16 && d_in <= kPlaneMaxDim && static_cast<double>(n_tokens) * d_in * d_in >= kPlaneMinWork)
    return plane_plan(d_in, n_tokens, n_cu);
  HessPlan pl{};
  pl.tile = bf16 ? kBTile : kFTile;
  pl.stage_tokens = bf16 ? kPStage * kPSlots : kFStage;
  pl.nt = static_cast<int>((d_in + pl.tile - 1) / pl.tile);
  pl.n_tiles = pl.nt * (pl.nt + 1) / 2;
  const int per_cu = bf16 ? 1 : 2;  // resident workgroups per CU (LDS bound)
  const int64_t slots = static_cast<int64_t>(n_cu > 0 ? n_cu : 256) * per_cu;
  const int64_t stages = (n_tokens + pl.stage_tokens - 1) / pl.stage_tokens;
  // choose the slice count that fills whole waves of workgroups, with a mild
  // preference for fewer slices (each slice costs a partial tile in HBM)
  int best = 1;
  double best_score = -1e30;
  const int max_split = static_cast<int>(std::min<int64_t>(64, std::max<int64_t>(1, stages / 4)));
  for (int s = 1; s <= max_split; ++s) {
    const int64_t blocks = static_cast<int64_t>(pl.n_tiles) * s;
    const int64_t waves = (blocks + slots - 1) / slots;
    const double eff = static_cast<double>(blocks) / static_cast<double>(waves * slots);
    const double score = eff - 0.002 * s;
    if (score > best_score + 1e-12) {
      best_score = score;
      best = s;
    }
  }
  pl.n_split = best;
  const int64_t per = (stages + best - 1) / best;
  pl.split_len = per * pl.stage_tokens;
  if (pl.split_len <= 0) pl.split_len = pl.stage_tokens;
  pl.n_split = static_cast<int>(std::max<int64_t>(1, (n_tokens + pl.split_len - 1) / pl.split_len));
  const size_t tile_bytes = static_cast<size_t>(pl.tile) * pl.tile * sizeof(float);
  pl.partial_bytes = static_cast<size_t>(pl.n_tiles) * pl.n_split * tile_bytes;
  pl.ws_bytes = (pl.partial_bytes + 255) & ~static_cast<size_t>(255);
  return pl;
}

hipError_t hessian_launch(const HessPlan& pl, float* S, int64_t d_in, const void* X, bool bf16,
                          int64_t n_tokens, int64_t ldx, void* ws, hipStream_t stream) {
  if (n_tokens <= 0 || d_in <= 0) return hipSuccess;
  HessParams p{};
  p.X = X;
  p.ldx = ldx;
  p.n_tokens = n_tokens;
  p.d_in = static_cast<int32_t>(d_in);
  p.nt = pl.nt;
  p.n_tiles = pl.n_tiles;
  p.n_split = pl.n_split;
  p.split_len = pl.split_len;
  p.partial = static_cast<float*>(ws);
  const int blocks = pl.n_tiles * pl.n_split;
  const int d = static_cast<int>(d_in);
  if (pl.planes) {
    // fp32 X in passes: split a pass into bf16 planes, the plane tiles'
    // partials, then their sum into S
    const int dp = pl.nt * kBTile;
    uint16_t* X3 = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + pl.planes_off);
    p.X = X3;
    p.ldx = 3 * static_cast<int64_t>(dp);
    p.d_in = 3 * dp;
    p.planes = 1;
    for (int64_t c0 = 0; c0 < n_tokens; c0 += pl.chunk) {
      const int64_t len = std::min<int64_t>(pl.chunk, n_tokens - c0);
      p.n_tokens = len;
      // a shorter last pass takes fewer slices, so no slice is empty
      p.n_split = static_cast<int32_t>((len + pl.split_len - 1) / pl.split_len);
      {
        PhaseScope ph(kPhHessian, stream);
        const int64_t work = len * (dp / 4);
        const int grid = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>((work + 255) / 256, 8192)));
        plane_split_kernel<<<grid, 256, 0, stream>>>(static_cast<const float*>(X) + c0 * ldx, ldx, len, d, dp, X3);
        hessian_bf16_pipe_kernel<<<pl.n_tiles * p.n_split, kThreads, 0, stream>>>(p);
      }
      PhaseScope ph(kPhHessReduce, stream);
      const int out_tiles = pl.nt * (pl.nt + 1) / 2;
      plane_reduce_kernel<<<out_tiles * 64, 256, 0, stream>>>(p.partial, p.n_split, pl.nt, d, S);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (bf16) {
    {
      PhaseScope ph(kPhHessian, stream);
      hessian_bf16_pipe_kernel<<<blocks, kThreads, 0, stream>>>(p);
    }
    PhaseScope ph(kPhHessReduce, stream);
    hessian_reduce_kernel<kBTile, 32, 4><<<pl.n_tiles * 64, 256, 0, stream>>>(p.partial, pl.n_split, pl.nt, d, S);
  } else {
    {
      PhaseScope ph(kPhHessian, stream);
      hessian_f32_kernel<<<blocks, kThreads, 0, stream>>>(p);
    }
    PhaseScope ph(kPhHessReduce, stream);
    hessian_reduce_kernel<kFTile, 16, 1><<<pl.n_tiles * 64, 64, 0, stream>>>(p.partial, pl.n_split, pl.nt, d, S);
  }
  return hipGetLastError();
}

}  // namespace gptq
