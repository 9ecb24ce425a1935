// S += X^T X on gfx950 matrix cores.
//
// GPTQ 实战 ch.5, section 5.1.7: the layer Hessian is X X^T (up to a constant)
// estimated from calibration activations.  X arrives token-major
// ([tokens, d_in]), so the contraction runs over the strided token axis.
//
// Work split: the d_in x d_in output is cut into tiles of the upper triangle
// (diagonal tiles computed whole); the token axis is cut into n_split equal
// slices so a launch has enough workgroups for 256 CUs.  Each workgroup owns
// one (tile, slice) pair and writes its fp32 partial tile; the last workgroup
// of a tile to finish (a ticket counter) sums the partials in slice order and
// adds the result to S and to its mirror tile.  The sum order is fixed, so
// the result does not depend on scheduling.
//
// bf16 path: 256x256 tile, 4 waves of 128x128, v_mfma_f32_32x32x16_bf16.
//   Each thread loads an 8-token x 8-channel block (eight 16-byte loads) and
//   transposes it in registers with v_perm_b32, so LDS holds every channel's
//   tokens contiguously: MFMA operands are single ds_read_b128.  A wave's
//   load instruction reads two token rows, 512 contiguous bytes each.  LDS
//   rows are 128 bytes (64 tokens); the 16-byte chunk index is XOR-swizzled
//   with the row index so both the transposing stores and the operand loads
//   are free of bank conflicts.  Double-buffered: 2 x (32 KB + 32 KB).
// fp32 path: 128x128 tile, 4 waves of 64x64, v_mfma_f32_16x16x4_f32, LDS
//   holds [token][channel] rows padded to 144 floats.
#include "gptq_common.h"
#include "gptq_internal.h"

#include <algorithm>

namespace gptq {
namespace {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

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
  int32_t* tickets;
  float* S;
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

// ----------------------------------------------------------------------------
// Split-slice epilogue shared by both paths.  Accumulators are NI x NJ MFMA
// 16x16 tiles per wave; element (i, j, r) of a lane sits at tile row
// rbase + 16 i + 4 (lane >> 4) + r and tile column cbase + 16 j + (lane & 15).
// ----------------------------------------------------------------------------
template <int TILE>
GPTQ_DEV void add_frag_to_S(const HessParams& p, int I, int J, int row0, int col, const f32x4_t& v) {
  // v[r] belongs to tile element (row0 + r, col)
  const int d = p.d_in;
  const int gc = J * TILE + col;
  if (gc >= d) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int gr = I * TILE + row0 + r;
    if (gr < d) {
      p.S[static_cast<int64_t>(gr) * d + gc] += v[r];
      if (I != J) p.S[static_cast<int64_t>(gc) * d + gr] += v[r];
    }
  }
}

// Split-slice epilogue.  The caller has stored its accumulators to its
// partial tile in register order (lane-fastest f32x4 fragments).  The
// accumulators only ever leave through memory stores (which read AGPRs
// directly): arithmetic on them would make the register allocator keep part
// of them in VGPRs across the main loop and shuffle them every stage.
// coord(f, row0, col): tile row of fragment f's first element and its column
// (the 4 elements are 4 consecutive rows).
template <int NF, int TILE, typename Coord>
GPTQ_DEV void finish_tile(const HessParams& p, int t, int I, int J, Coord coord) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int64_t kElems = static_cast<int64_t>(TILE) * TILE;
  fence_release();
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) {
    const int old = (p.n_split == 1) ? 0 : atomicAdd(&p.tickets[t], 1);
    s_last = (old == p.n_split - 1);
  }
  __syncthreads();
  if (!s_last) return;
  fence_acquire();
  // the last slice to arrive sums all slices in slice order, fragment by fragment
  const float* base = p.partial + static_cast<int64_t>(t) * p.n_split * kElems;
  for (int f = 0; f < NF; ++f) {
    const int64_t off = static_cast<int64_t>((wave * NF + f) * 64 + lane) << 2;
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < p.n_split; ++k) sum += *reinterpret_cast<const f32x4_t*>(base + k * kElems + off);
    int row0, col;
    coord(f, row0, col);
    add_frag_to_S<TILE>(p, I, J, row0, col, sum);
  }
}

GPTQ_DEV float* partial_tile(const HessParams& p, int t, int split, int64_t elems) {
  return p.partial + (static_cast<int64_t>(t) * p.n_split + split) * elems;
}

// ============================================================ bf16 path ====
constexpr int kBTile = 256;
constexpr int kBStage = 64;              // tokens per stage = 128 bytes per LDS row
constexpr int kBOpBytes = kBTile * 128;  // one operand stage: 32 KB

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

// Loads tokens [8 tg, 8 tg + 8) of the stage for one 8-channel group: the lane
// offset is 32-bit, the row step is a scalar offset.  A channel group beyond
// d_in (d_in is a multiple of 8) gets an out-of-range offset and reads zeros.
GPTQ_DEV void load_block_bf16(__amdgpu_buffer_rsrc_t rs, int ldx, int tg, int col, int d_in, u32x4_t (&r)[8]) {
  const uint32_t voff = (col < d_in) ? static_cast<uint32_t>((8 * tg * ldx + col) * 2) : 0x80000000u;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, j * ldx * 2, 0);
}

// LDS row m (one channel, 64 tokens = eight 16-byte chunks): logical chunk q is
// stored at q ^ (m & 7) ^ ((m >> 3) & 7).  Both the transposing stores (eight
// rows 8 apart per instruction) and the operand loads (consecutive rows) then
// touch eight distinct bank groups.
GPTQ_DEV int swz(int m, int q) { return q ^ (m & 7) ^ ((m >> 3) & 7); }

// r[j] holds tokens (8 tg + j) x channels (8 cg .. 8 cg + 7); write each channel's
// 8 tokens as one 16-byte chunk (logical chunk tg) of LDS row 8 cg + c.
GPTQ_DEV void store_block_bf16(uint8_t* lds, int cg, int tg, const u32x4_t (&r)[8]) {
#pragma unroll
  for (int pch = 0; pch < 4; ++pch) {
    u32x4_t lo, hi;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lo[q] = __builtin_amdgcn_perm(r[2 * q + 1][pch], r[2 * q][pch], 0x05040100u);
      hi[q] = __builtin_amdgcn_perm(r[2 * q + 1][pch], r[2 * q][pch], 0x07060302u);
    }
    const int m0 = 8 * cg + 2 * pch;
    *reinterpret_cast<u32x4_t*>(lds + m0 * 128 + (swz(m0, tg) << 4)) = lo;
    *reinterpret_cast<u32x4_t*>(lds + (m0 + 1) * 128 + (swz(m0 + 1, tg) << 4)) = hi;
  }
}

// One 64-token stage on v_mfma_f32_32x32x16_bf16: the wave's 128x128 block is
// 4x4 MFMA tiles; per 16 tokens each lane reads one 16-byte chunk (8 tokens of
// one channel) per A and B tile.  32x32 tiles keep the loop free of
// accumulator moves (the allocator handles 16 wide tuples well).
GPTQ_DEV void mfma_stage_bf16(const uint8_t* A, const uint8_t* B, int wm, int wn, int lane,
                              f32x16_t (&acc)[4][4]) {
  const int r32 = lane & 31;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int q = (lane >> 5) + 2 * ks;
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 128 + 32 * i + r32;
      a[i] = *reinterpret_cast<const bf16x8_t*>(A + m * 128 + (swz(m, q) << 4));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = wn * 128 + 32 * j + r32;
      b[j] = *reinterpret_cast<const bf16x8_t*>(B + m * 128 + (swz(m, q) << 4));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kThreads, 1) void hessian_bf16_kernel(HessParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kBOpBytes];
  int t, split, I, J;
  work_item(blockIdx.x, p.n_tiles, p.n_split, t, split);
  tile_coords(t, p.nt, I, J);
  const bool diag = (I == J);
  const int64_t k0 = static_cast<int64_t>(split) * p.split_len;
  const int64_t k1 = min(p.n_tokens, k0 + p.split_len);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // a load instruction covers two token rows, 512 contiguous bytes each
  const int cg = lane & 31, tg = (lane >> 5) + 2 * wave;
  const int colA = I * kBTile + 8 * cg, colB = J * kBTile + 8 * cg;
  const uint16_t* X = static_cast<const uint16_t*>(p.X);

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nstage = (k1 > k0) ? static_cast<int>((k1 - k0 + kBStage - 1) / kBStage) : 0;
  const int ldx = static_cast<int>(p.ldx);
  // diagonal tiles load the same channel block for both operands (an L2 hit):
  // one code path keeps the loop free of branches, which lets the compiler
  // keep the 256 accumulators in fixed AGPRs.  Global loads run two stages
  // ahead of the MFMAs (two register sets), so about two stages of load
  // latency are hidden behind matrix work.
  u32x4_t ra0[8], rb0[8], ra1[8], rb1[8];
  auto load_stage = [&](int s, u32x4_t (&ra)[8], u32x4_t (&rb)[8]) {
    const int64_t t0 = k0 + static_cast<int64_t>(s) * kBStage;
    const int left = static_cast<int>(min<int64_t>(k1 - t0, kBStage));
    const __amdgpu_buffer_rsrc_t rs = stage_rsrc(X + t0 * p.ldx, left, ldx);
    load_block_bf16(rs, ldx, tg, colA, p.d_in, ra);
    load_block_bf16(rs, ldx, tg, colB, p.d_in, rb);
  };
  auto store_stage = [&](int buf, const u32x4_t (&ra)[8], const u32x4_t (&rb)[8]) {
    store_block_bf16(lds[buf][0], cg, tg, ra);
    store_block_bf16(lds[buf][1], cg, tg, rb);
  };
  // stage s lives in LDS buffer s & 1 and, before that, in register set s & 1
  if (nstage > 0) load_stage(0, ra0, rb0);
  if (nstage > 1) load_stage(1, ra1, rb1);
  if (nstage > 0) store_stage(0, ra0, rb0);
  __syncthreads();
  int s = 0;
  for (; s + 3 < nstage; s += 2) {
    load_stage(s + 2, ra0, rb0);
    mfma_stage_bf16(lds[0][0], lds[0][1], wm, wn, lane, acc);
    store_stage(1, ra1, rb1);
    __syncthreads();
    load_stage(s + 3, ra1, rb1);
    mfma_stage_bf16(lds[1][0], lds[1][1], wm, wn, lane, acc);
    store_stage(0, ra0, rb0);
    __syncthreads();
  }
  // tail: at most three stages left, s even; stage s is in LDS 0, s + 1 in set 1
  for (; s < nstage; ++s) {
    const int cur = s & 1;
    if (s + 2 < nstage) {
      if (cur == 0) load_stage(s + 2, ra0, rb0);
      else load_stage(s + 2, ra1, rb1);
    }
    mfma_stage_bf16(lds[cur][0], lds[cur][1], wm, wn, lane, acc);
    if (s + 1 < nstage) {
      if (cur == 0) store_stage(1, ra1, rb1);
      else store_stage(0, ra0, rb0);
    }
    __syncthreads();
  }
  (void)diag;
  // 32x32 accumulator layout: element r of lane l is tile row
  // 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32; stored as 4 fragments of 4 rows
  float* mine = partial_tile(p, t, split, static_cast<int64_t>(kBTile) * kBTile);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<f32x4_t*>(mine + (((wave * 64 + (i * 4 + j) * 4 + e) * 64 + lane) << 2)) =
            f32x4_t{acc[i][j][4 * e], acc[i][j][4 * e + 1], acc[i][j][4 * e + 2], acc[i][j][4 * e + 3]};
  finish_tile<64, kBTile>(p, t, I, J, [&](int f, int& row0, int& col) {
    const int i = f >> 4, j = (f >> 2) & 3, e = f & 3;
    row0 = wm * 128 + 32 * i + 8 * e + 4 * (lane >> 5);
    col = wn * 128 + 32 * j + (lane & 31);
  });
}

// ======================================================= bf16 DMA path ====
// Same tiling and epilogue as hessian_bf16_kernel, but X moves from HBM to LDS
// with buffer_load ... lds (no VGPRs, no register transposition) through a
// ring of four 32-token stages (three in flight while one is consumed), and
// the MFMA operands come out of the token-major LDS tile through
// ds_read_b64_tr_b16.  In a 16-lane group, if lane s points at token
// t0 + (s >> 2), channels m0 + 4 (s & 3) .. +3, lane i receives tokens
// t0 .. t0 + 3 of channel m0 + i: two such reads make one 8-token operand.
// LDS rows (tokens) are 512 bytes; the 16-byte chunk index is XOR-swizzled
// with 2 (row & 3) so the eight chunks one read touches fall in distinct banks.
constexpr int kDStage = 32;               // tokens per stage
constexpr int kDOpBytes = kDStage * 512;  // one operand stage: 16 KB

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

#define GPTQ_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

GPTQ_DEV void dma_operand(__amdgpu_buffer_rsrc_t rs, uint8_t* buf, int ldx, int col0, int d_in, int wave_u,
                          int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = 4 * wave_u + u;               // 1 KB piece: token rows 2q, 2q + 1
    const int row = 2 * q + (lane >> 5);
    const int c = (lane & 31) ^ (2 * (row & 3));  // logical chunk held at this lane's slot
    const int col = col0 + 8 * c;
    const uint32_t voff = (col < d_in) ? static_cast<uint32_t>((row * ldx + col) * 2) : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(buf + q * 1024), 16, voff, 0, 0, 0);
  }
}

GPTQ_DEV bf16x8_t tr_operand(const uint8_t* buf, uint32_t lane_off, int imm) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
  uint8_t* b = const_cast<uint8_t*>(buf) + lane_off + imm;
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)b);
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(b + 4 * 512));
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8_t;
  const s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// lane offsets of the transposed reads for even / odd 32-channel tiles of a wave block
struct TrLane {
  uint32_t off[2];
};
GPTQ_DEV TrLane tr_lane(int lane, int wblock) {
  const int g = lane >> 4, s = lane & 15;
  const int base_row = 8 * (g >> 1) + (s >> 2);
  const int f = 2 * (s >> 2);
  const int cl = 2 * (g & 1) + ((s & 3) >> 1);
  TrLane t;
#pragma unroll
  for (int par = 0; par < 2; ++par)
    t.off[par] = static_cast<uint32_t>(base_row * 512 + (s & 1) * 8 + 16 * ((4 * par + cl) ^ f) + 256 * wblock);
  return t;
}

GPTQ_DEV void mfma_stage_tr(const uint8_t* A, const uint8_t* B, const TrLane& la, const TrLane& lb,
                            f32x16_t (&acc)[4][4]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = tr_operand(A, la.off[i & 1], ks * 16 * 512 + (i >> 1) * 128);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = tr_operand(B, lb.off[j & 1], ks * 16 * 512 + (j >> 1) * 128);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kThreads, 1) void hessian_bf16_dma_kernel(HessParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[kDOpBytes], sB0[kDOpBytes], sA1[kDOpBytes], sB1[kDOpBytes],
      sA2[kDOpBytes], sB2[kDOpBytes], sA3[kDOpBytes], sB3[kDOpBytes];
  int t, split, I, J;
  work_item(blockIdx.x, p.n_tiles, p.n_split, t, split);
  tile_coords(t, p.nt, I, J);
  const int64_t k0 = static_cast<int64_t>(split) * p.split_len;
  const int64_t k1 = min(p.n_tokens, k0 + p.split_len);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int colA = I * kBTile, colB = J * kBTile;
  const int ldx = static_cast<int>(p.ldx);
  const uint16_t* X = static_cast<const uint16_t*>(p.X);
  const TrLane la = tr_lane(lane, wm), lb = tr_lane(lane, wn);

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nstage = (k1 > k0) ? static_cast<int>((k1 - k0 + kDStage - 1) / kDStage) : 0;
  auto issue = [&](int s, uint8_t* bA, uint8_t* bB) {
    const int64_t t0 = k0 + static_cast<int64_t>(s) * kDStage;
    const int left = static_cast<int>(min<int64_t>(k1 - t0, kDStage));
    const __amdgpu_buffer_rsrc_t rs = stage_rsrc(X + t0 * p.ldx, left, ldx);
    dma_operand(rs, bA, ldx, colA, p.d_in, wave, lane);
    dma_operand(rs, bB, ldx, colB, p.d_in, wave, lane);
  };
  auto bufA = [&](int r) { return r == 0 ? sA0 : r == 1 ? sA1 : r == 2 ? sA2 : sA3; };
  auto bufB = [&](int r) { return r == 0 ? sB0 : r == 1 ? sB1 : r == 2 ? sB2 : sB3; };
  int s = 0;
  if (nstage > 6) {
    // steady state: stage s + r lives in ring buffer r and every wait leaves
    // the two stages issued after it in flight.  All issues here are
    // unconditional, which keeps the compiler's own wait tracking exact.
    issue(0, sA0, sB0);
    issue(1, sA1, sB1);
    issue(2, sA2, sB2);
    for (; s + 6 < nstage; s += 4) {
      __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(16));
      __builtin_amdgcn_s_barrier();
      issue(s + 3, sA3, sB3);
      mfma_stage_tr(sA0, sB0, la, lb, acc);
      __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(16));
      __builtin_amdgcn_s_barrier();
      issue(s + 4, sA0, sB0);
      mfma_stage_tr(sA1, sB1, la, lb, acc);
      __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(16));
      __builtin_amdgcn_s_barrier();
      issue(s + 5, sA1, sB1);
      mfma_stage_tr(sA2, sB2, la, lb, acc);
      __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(16));
      __builtin_amdgcn_s_barrier();
      issue(s + 6, sA2, sB2);
      mfma_stage_tr(sA3, sB3, la, lb, acc);
    }
  } else {
    for (int x = 0; x < nstage && x < 3; ++x) issue(x, bufA(x), bufB(x));
  }
  // tail (at most six stages): stage x in buffer x % 4, stages up to s + 2
  // already issued; full waits.  A buffer is refilled only after the barrier
  // that follows everyone's last read of it.
  for (int x = s; x < nstage; ++x) {
    __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(0));
    __builtin_amdgcn_s_barrier();
    if (x + 3 < nstage) issue(x + 3, bufA((x + 3) & 3), bufB((x + 3) & 3));
    mfma_stage_tr(bufA(x & 3), bufB(x & 3), la, lb, acc);
  }
  float* mine = partial_tile(p, t, split, static_cast<int64_t>(kBTile) * kBTile);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<f32x4_t*>(mine + (((wave * 64 + (i * 4 + j) * 4 + e) * 64 + lane) << 2)) =
            f32x4_t{acc[i][j][4 * e], acc[i][j][4 * e + 1], acc[i][j][4 * e + 2], acc[i][j][4 * e + 3]};
  finish_tile<64, kBTile>(p, t, I, J, [&](int f, int& row0, int& col) {
    const int i = f >> 4, j = (f >> 2) & 3, e = f & 3;
    row0 = wm * 128 + 32 * i + 8 * e + 4 * (lane >> 5);
    col = wn * 128 + 32 * j + (lane & 31);
  });
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
  finish_tile<16, kFTile>(p, t, I, J, [&](int f, int& row0, int& col) {
    const int i = f >> 2, j = f & 3;
    row0 = wm * 64 + 16 * i + 4 * (lane >> 4);
    col = wn * 64 + 16 * j + (lane & 15);
  });
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  fill_i32_kernel<<<static_cast<int>(blocks), 256, 0, stream>>>(p, n, v);
  return hipGetLastError();
}

HessPlan hessian_plan(int64_t d_in, int64_t n_tokens, bool bf16, int n_cu) {
  HessPlan pl{};
  pl.tile = bf16 ? kBTile : kFTile;
  pl.stage_tokens = bf16 ? kBStage : kFStage;
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
  pl.ticket_bytes = static_cast<size_t>(pl.n_tiles) * sizeof(int32_t);
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  pl.ws_bytes = up(pl.partial_bytes) + up(pl.ticket_bytes);
  return pl;
}

hipError_t hessian_launch(const HessPlan& pl, float* S, int64_t d_in, const void* X, bool bf16,
                          int64_t n_tokens, int64_t ldx, void* ws, hipStream_t stream) {
  if (n_tokens <= 0 || d_in <= 0) return hipSuccess;
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
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
  p.tickets = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + up(pl.partial_bytes));
  p.S = S;
  if (pl.n_split > 1) {
    hipError_t e = fill_i32(p.tickets, pl.n_tiles, 0, stream);
    if (e != hipSuccess) return e;
  }
  const int blocks = pl.n_tiles * pl.n_split;
  if (bf16)
    hessian_bf16_dma_kernel<<<blocks, kThreads, 0, stream>>>(p);
  else
    hessian_f32_kernel<<<blocks, kThreads, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace gptq
