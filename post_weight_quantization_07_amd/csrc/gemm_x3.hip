// fp32 products on the bf16 matrix cores.
//
// On gfx950 a v_mfma_f32_16x16x4_f32 runs at the fp32 vector rate and holds
// the SIMD's vector ALU while it runs; the bf16 matrix cores are 16 times
// faster per flop and leave the vector ALU to other waves.  An fp32 value x
// splits exactly into three bf16 parts, x = hi + mid + lo: hi = bf16(x), the
// remainder x - hi is exact (Sterbenz), mid = bf16 of it, and what is left
// has at most 6 significant bits, so lo holds it exactly.  A product x y is
// then the sum of the nine part products; the six kept here (hi hi, hi mid,
// mid hi, hi lo, mid mid, lo hi) leave out terms below 2^-24 |x y|, and each
// part product is exact in the fp32 accumulator.  The result has the accuracy
// of an fp32 product (it is not bit-equal to one: the sums round in another
// order).  It serves the GPTQ lazy-batch update W[:, j+B:] -= Err U[j:j+B,
// j+B:] and the products of the factor U = Cholesky(inverse(H)) (GPTQ 实战
// ch.5, section 5.1.8): the Cholesky's updates and the widest levels of the
// triangular inverse (batched, with the triangular operands' zero K range
// skipped per tile).
//
// Operands are given as three planes of bf16 bit patterns in the blocked
// panel layout (x3_offset): A over [M][K], B transposed over [N][K]; C fp32
// row-major.  A block of 128 rows x 16 k is 4 KB contiguous, so one stage of
// one plane of a tile is one contiguous read.
// 128 x 128 output tile per 256-thread workgroup (2 x 2 waves of 64 x 64,
// v_mfma_f32_32x32x16_bf16), 16-k stages (24 KB: both operands, three
// planes) moved to LDS by buffer_load ... lds through a ring of three slots,
// two workgroups a CU (measured at 4096 x 3072 x 1024: 156 us against 194 us
// for one workgroup with a six-slot ring and 163 us for three with two).
// Each wave reads the next stage's operand fragments from LDS while its
// products of the current stage run (two register sets, one fragment read
// between two products): 4-5% faster on the large shapes.  A 256 x 128 tile
// (eight waves, one workgroup a CU) was slower.  Problems with fewer than 512
// such tiles use 64 x 64 tiles (2 x 2 waves of 32 x 32, four workgroups a
// CU): the Cholesky's 128-column products and its smaller trailing updates
// run about twice as fast on them.
#include "gptq_common.h"
#include "gptq_internal.h"

#include <algorithm>

namespace gptq {

namespace {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kT = 128;        // output tile edge
constexpr int kSK = 16;        // k per stage (one MFMA k-step)
constexpr int kSlots = 3;      // ring depth: two stages in flight; two workgroups a CU
constexpr int kSmallBelow = 512;             // fewer 128-tiles than this: 64-tiles

// s_waitcnt immediate: vmcnt(n) and lgkmcnt(0)
#define GPTQ_X3_VMLGK(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0070)

struct X3Params {
  const uint16_t* A;  // 3 planes of [M][K], blocked
  const uint16_t* B;  // 3 planes of [N][K], blocked
  int64_t M, N, K;
  int64_t ldk;        // width of the planes' blocked layout (>= K): the product uses its first K columns
  int64_t sA, sB;     // plane strides in elements
  float* C;
  int64_t ldc;
  float alpha;
  int tiles_m, tiles_n;
  int lower;          // only the tiles on or below the diagonal; nothing written above the 64-block diagonal
  int tri;            // 0 dense; 1 B lower-triangular (a tile skips k below its first column); 2 A
                      // lower-triangular (a tile skips k past its last row)
  int beta0;          // C = alpha A B (C is not read)
  int64_t bA, bB, bC; // batch strides (blockIdx.y) in elements
};

GPTQ_DEV __amdgpu_buffer_rsrc_t x3_rsrc(const uint16_t* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const int64_t cl = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0LL : bytes);
  const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(cl));
  void* b = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, static_cast<short>(0), n, 0x00020000);
}

// One plane of one operand stage: the 4 KB block of 128 rows x 16 k (32
// bytes a row, two 16-byte chunks) is four 1 KB pieces of 32 rows.  Physical
// chunk p of row r in LDS holds logical chunk p ^ ((r >> 3) & 1): an MFMA
// operand read (16 consecutive rows, one chunk each) then covers all 64
// banks; the permutation stays inside each row's 32 bytes, so a piece is
// still one contiguous 1 KB read.  rs spans the tile's 128-row block, st is
// the stage, src the piece in the block, dst the piece's place in LDS.
GPTQ_DEV void x3_dma(__amdgpu_buffer_rsrc_t rs, uint8_t* dst, int st, int src, int lane) {
  const int r = 32 * src + (lane >> 1);
  const int c = (lane & 1) ^ ((r >> 3) & 1);
  const uint32_t voff = static_cast<uint32_t>((st * 2048 + r * 16 + 8 * c) * 2);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 16, voff, 0, 0, 0);
}

// the 8 bf16 of row r, k 8 h .. 8 h + 7 (h = lane >> 5) of a stage plane
GPTQ_DEV bf16x8_t x3_read(const uint8_t* plane, int r, int h) {
  const int pc = h ^ ((r >> 3) & 1);
  return *reinterpret_cast<const bf16x8_t*>(plane + r * 32 + pc * 16);
}

// TS x TS output tile per 256-thread workgroup, 2 x 2 waves of TS/2 x TS/2.
// TS = 128: each wave moves piece w of all six planes of a stage.  TS = 64
// (problems with few 128-tiles): a tile is half a 128-row block; waves 0-1
// move A's two pieces, waves 2-3 B's, three planes each.
template <int TS>
__global__ __launch_bounds__(256, TS == 128 ? 2 : 4) void gemm_x3_kernel(X3Params p) {
  constexpr int kNI = TS / 64;                   // 32 x 32 blocks per wave and dimension
  constexpr int kPlane = TS * kSK * 2;           // bytes of one plane of one operand stage
  constexpr int kSlot = 6 * kPlane;              // A and B, three planes each
  constexpr int kLoads = TS == 128 ? 6 : 3;      // DMA instructions per wave per stage
  constexpr int kFr = 6 * kNI;                   // fragments per wave per stage
  constexpr int kMf = 6 * kNI * kNI;             // products per wave per stage
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kSlots * kSlot];
  // Workgroups go round-robin to the 8 XCDs (b % 8), each with its own L2:
  // the tile list is cut into 8 contiguous ranges, one per XCD, listed in
  // groups of 8 tile rows, column by column inside a group, so the tiles an
  // XCD runs at once share rows of A and columns of B.
  // Lower-tile problems list the tiles (i >= j) row by row.
  // Triangular problems instead list the tiles heaviest first in plain
  // dispatch order, so the round robin gives every XCD an equal share of
  // heavy and light tiles.
  constexpr int kXcd = 8;
  const int b = blockIdx.x, G = p.lower ? p.tiles_m * (p.tiles_m + 1) / 2 : p.tiles_m * p.tiles_n;
  const int x = b % kXcd, xl = b / kXcd;
  const int base = G / kXcd, rem = G % kXcd;
  const int t = x * base + min(x, rem) + xl;
  int tm, tn;
  if (p.tri == 1) {  // k from the tile's first column: the first columns are heaviest
    tn = b / p.tiles_m;
    tm = b % p.tiles_m;
  } else if (p.tri == 2) {  // k up to the tile's last row: the last rows are heaviest
    tm = p.tiles_m - 1 - b / p.tiles_n;
    tn = b % p.tiles_n;
  } else if (p.lower) {
    int i = static_cast<int>((__builtin_sqrtf(8.f * t + 1.f) - 1.f) * 0.5f);
    while (i * (i + 1) / 2 > t) --i;
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    tm = i;
    tn = t - i * (i + 1) / 2;
  } else {
    const int g = t / (8 * p.tiles_n);
    const int rows = min(8, p.tiles_m - 8 * g);
    const int idx = t - g * 8 * p.tiles_n;
    tn = idx / rows;
    tm = 8 * g + idx % rows;
  }
  const int64_t m0 = static_cast<int64_t>(tm) * TS, n0 = static_cast<int64_t>(tn) * TS;
  const int64_t bz = blockIdx.y;
  const uint16_t* Ab = p.A + bz * p.bA;
  const uint16_t* Bb = p.B + bz * p.bB;
  float* Cb = p.C + bz * p.bC;
  // the tile's k range: a lower-triangular operand is zero past it (both
  // ends are multiples of 64, so the stage count stays a multiple of four)
  const int64_t k_lo = p.tri == 1 ? min(n0, p.K) : 0;
  const int64_t k_hi = p.tri == 2 ? min(m0 + TS, p.K) : p.K;
  const int kst0 = static_cast<int>(k_lo / kSK);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // the 128-row block of each operand that holds the tile (rows past M or N
  // are padding), and the tile's first piece in it
  const int64_t ma = m0 & ~int64_t{127}, na = n0 & ~int64_t{127};
  __amdgpu_buffer_rsrc_t ra[3], rb[3];
#pragma unroll
  for (int pl = 0; pl < 3; ++pl) {
    ra[pl] = x3_rsrc(Ab + pl * p.sA + ma * p.ldk, 128 * p.ldk * 2);
    rb[pl] = x3_rsrc(Bb + pl * p.sB + na * p.ldk, 128 * p.ldk * 2);
  }
  const int pa = static_cast<int>(m0 - ma) / 32, pb = static_cast<int>(n0 - na) / 32;
  auto issue = [&](int xs) {  // stage xs of the tile's k range
    uint8_t* d = ring + (xs % kSlots) * kSlot;
    const int st = kst0 + xs;
    if (TS == 128) {
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        x3_dma(ra[pl], d + pl * kPlane + wave * 1024, st, wave, lane);
        x3_dma(rb[pl], d + (3 + pl) * kPlane + wave * 1024, st, wave, lane);
      }
    } else {
      const int c = wave & 1;
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        if (wave < 2)
          x3_dma(ra[pl], d + pl * kPlane + c * 1024, st, pa + c, lane);
        else
          x3_dma(rb[pl], d + (3 + pl) * kPlane + c * 1024, st, pb + c, lane);
      }
    }
  };

  f32x16_t acc[kNI][kNI];
#pragma unroll
  for (int i = 0; i < kNI; ++i)
#pragma unroll
    for (int j = 0; j < kNI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int h = lane >> 5, l32 = lane & 31;
  constexpr int kWT = TS / 2;  // wave tile edge
  // fragments of one stage: a[i][plane], b[j][plane]
  struct Frag { bf16x8_t a[kNI][3], b[kNI][3]; };
  auto read = [&](Frag& f, const uint8_t* d) {
#pragma unroll
    for (int pl = 0; pl < 3; ++pl)
#pragma unroll
      for (int i = 0; i < kNI; ++i) {
        f.a[i][pl] = x3_read(d + pl * kPlane, wm * kWT + 32 * i + l32, h);
        f.b[i][pl] = x3_read(d + (3 + pl) * kPlane, wn * kWT + 32 * i + l32, h);
      }
  };
  auto mfma = [&](const Frag& f) {
    // the six part products, smallest first, each over the independent
    // accumulators in turn
    constexpr int PA[6] = {2, 1, 0, 1, 0, 0}, PB[6] = {0, 1, 2, 0, 1, 0};
#pragma unroll
    for (int q = 0; q < 6; ++q)
#pragma unroll
      for (int i = 0; i < kNI; ++i)
#pragma unroll
        for (int jj = 0; jj < kNI; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i][PA[q]], f.b[jj][PB[q]], acc[i][jj], 0, 0, 0);
  };
  // the next stage's fragment reads spread over this stage's products
  auto interleave = [&]() {
#pragma unroll
    for (int r = 0; r < kFr; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, kMf / kFr, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // K is a multiple of 32, at least 64 (the host checks): an even number of
  // stages, at least four
  const int nstage = static_cast<int>((k_hi - k_lo) / kSK);
  // stage x lives in slot x % kSlots.  Stage y - 1 is computed from registers
  // while stage y is read from LDS; before that read: stage y has landed
  // (with stage y + 1 still in flight) and a barrier (every wave has read
  // stage y - 1 and finished those reads, so its slot takes stage y - 1 +
  // kSlots).
  auto half = [&](int y, const Frag& fc, Frag& fr) {
    if (y - 1 + kSlots < nstage) {
      __builtin_amdgcn_s_waitcnt(GPTQ_X3_VMLGK(kLoads));
      __builtin_amdgcn_s_barrier();
      issue(y - 1 + kSlots);
    } else {
      __builtin_amdgcn_s_waitcnt(GPTQ_X3_VMLGK(0));
      __builtin_amdgcn_s_barrier();
    }
    read(fr, ring + (y % kSlots) * kSlot);
    mfma(fc);
    interleave();
  };
  Frag F0, F1;
  if (nstage > 0) {
  for (int st = 0; st < kSlots && st < nstage; ++st) issue(st);
  __builtin_amdgcn_s_waitcnt(GPTQ_X3_VMLGK(2 * kLoads));  // stage 0 (two more stages issued after it)
  __builtin_amdgcn_s_barrier();
  read(F0, ring);
  for (int xs = 0; xs + 2 < nstage; xs += 2) {
    half(xs + 1, F0, F1);
    half(xs + 2, F1, F0);
  }
  half(nstage - 1, F0, F1);
  mfma(F1);
  }

  // C += alpha acc: accumulator element e of lane l in a 32 x 32 block is row
  // 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32.  Every C value is loaded
  // before the first store, so the loads are in flight together.
  float cv[kNI][kNI][16];
#pragma unroll
  for (int i = 0; i < kNI; ++i)
#pragma unroll
    for (int jj = 0; jj < kNI; ++jj) {
      const int64_t n = n0 + wn * kWT + 32 * jj + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * kWT + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        cv[i][jj][e] = (m < p.M && n < p.N && !p.beta0) ? Cb[m * p.ldc + n] : 0.f;
      }
    }
#pragma unroll
  for (int i = 0; i < kNI; ++i)
#pragma unroll
    for (int jj = 0; jj < kNI; ++jj) {
      const int64_t n = n0 + wn * kWT + 32 * jj + l32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * kWT + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        if (m < p.M && n < p.N && !(p.lower && (m >> 6) < (n >> 6)))
          Cb[m * p.ldc + n] = fmaf(p.alpha, acc[i][jj][e], cv[i][jj][e]);
      }
    }
}

// planes of the transposed block in the blocked layout: element (n, k) of
// plane pl = part pl of src[k][n] for k < K, n < N (src row-major, ld
// elements); 64 x 64 tiles through LDS.  Padding rows n >= N are not written.
__global__ __launch_bounds__(256) void split3_t_kernel(const float* src, int64_t ld, int64_t K, int64_t N,
                                                       uint16_t* out, int64_t plane, int64_t bsrc, int64_t bout) {
  __shared__ float tile[64][65];
  src += blockIdx.z * bsrc;
  out += blockIdx.z * bout;
  const int64_t k0 = static_cast<int64_t>(blockIdx.y) * 64, nb = static_cast<int64_t>(blockIdx.x) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const int64_t k = k0 + r, n = nb + tx;
    tile[r][tx] = (k < K && n < N) ? src[k * ld + n] : 0.f;
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int64_t n = nb + r, k = k0 + tx;
    if (n < N && k < K) {
      uint16_t hh, mm, ll;
      split3(tile[tx][r], hh, mm, ll);
      const int64_t o = x3_offset(n, k, K);
      out[o] = hh;
      out[plane + o] = mm;
      out[2 * plane + o] = ll;
    }
  }
}

// planes of a row-major block in the blocked layout: element (r, k) of
// plane pl = part pl of src[r][k] for r < R, k < K (K a multiple of 16); a
// 256-thread workgroup covers 4 rows x 64 k.  Padding rows are not written.
__global__ __launch_bounds__(256) void split3_rows_kernel(const float* src, int64_t ld, int64_t R, int64_t K,
                                                          uint16_t* out, int64_t plane, int64_t bsrc, int64_t bout) {
  src += blockIdx.z * bsrc;
  out += blockIdx.z * bout;
  const int64_t r = static_cast<int64_t>(blockIdx.y) * 4 + (threadIdx.x >> 6);
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 64 + (threadIdx.x & 63);
  if (r >= R || k >= K) return;
  uint16_t hh, mm, ll;
  split3(src[r * ld + k], hh, mm, ll);
  const int64_t o = x3_offset(r, k, K);
  out[o] = hh;
  out[plane + o] = mm;
  out[2 * plane + o] = ll;
}

}  // namespace

hipError_t gemm_x3(int64_t M, int64_t N, int64_t K, float alpha, const uint16_t* A, int64_t sA, const uint16_t* Bt,
                   int64_t sB, float* C, int64_t ldc, hipStream_t stream, int64_t ldk, bool lower, int tri, bool beta0,
                   int batch, int64_t bA, int64_t bB, int64_t bC) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  if (K % 32 != 0 || K < 64) return hipErrorInvalidValue;  // an even number of stages, at least four
  if (tri != 0 && (lower || K % 64 != 0)) return hipErrorInvalidValue;
  if (ldk <= 0) ldk = K;
  X3Params p{A, Bt, M, N, K, ldk, sA, sB, C, ldc, alpha, 0, 0, lower ? 1 : 0, tri, beta0 ? 1 : 0, bA, bB, bC};
  auto tiles_of = [&](int ts) {
    p.tiles_m = static_cast<int>((M + ts - 1) / ts);
    p.tiles_n = static_cast<int>((N + ts - 1) / ts);
    return lower ? p.tiles_m * (p.tiles_m + 1) / 2 : p.tiles_m * p.tiles_n;
  };
  // 128-tiles while they give every CU two workgroups; 64-tiles below that
  if (tiles_of(kT) * batch >= kSmallBelow) {
    gemm_x3_kernel<kT><<<dim3(tiles_of(kT), batch), 256, 0, stream>>>(p);
  } else {
    gemm_x3_kernel<64><<<dim3(tiles_of(64), batch), 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t split3_t(const float* src, int64_t ld, int64_t K, int64_t N, uint16_t* out, hipStream_t stream, int batch,
                    int64_t bsrc, int64_t bout) {
  if (K <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((N + 63) / 64), static_cast<unsigned>((K + 63) / 64), batch);
  split3_t_kernel<<<grid, 256, 0, stream>>>(src, ld, K, N, out, x3_plane_elems(N, K), bsrc, bout);
  return hipGetLastError();
}

hipError_t split3_rows(const float* src, int64_t ld, int64_t R, int64_t K, uint16_t* out, hipStream_t stream, int batch,
                       int64_t bsrc, int64_t bout) {
  if (R <= 0 || K <= 0 || batch <= 0) return hipSuccess;
  if (K % 16 != 0) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>((K + 63) / 64), static_cast<unsigned>((R + 3) / 4), batch);
  split3_rows_kernel<<<grid, 256, 0, stream>>>(src, ld, R, K, out, x3_plane_elems(R, K), bsrc, bout);
  return hipGetLastError();
}

}  // namespace gptq
