// fp32 GEMM on gfx950 matrix cores (v_mfma_f32_16x16x4_f32).
//
// C[M,N] = alpha * A[M,K] * op(B)[K,N] + beta * C, all row-major.  op(B) is B
// ([K,N]) or, with transB, the transpose of a [N,K] matrix.  Used by the
// Cholesky trailing update, the triangular inverse and the GPTQ lazy-batch
// update W[:, j+B:] -= Err * U[j:j+B, j+B:] (GPTQ 实战 ch.5, section 5.1.8).
//
// 64x64 or 128x128 output tile per 256-thread workgroup (2x2 waves), 32-k
// stages moved HBM -> LDS by buffer_load ... lds through a ring of slots: three
// for 64x64 tiles (three workgroups per CU), two for 128x128 tiles, where one
// stage of MFMA work covers the next stage's loads and the 64 KB ring lets two
// workgroups share a CU (one's prologue and epilogue overlap the other's loop).
// Requirements (checked by the callers): K, N, lda, ldb, ldc multiples of 4 and
// 16-byte aligned base pointers; M arbitrary.  `tri` marks a lower-triangular
// operand (B, or A) whose zero part a tile's K range skips: the triangular
// inverse multiplies by inverted diagonal blocks.
#include "gptq_common.h"
#include "gptq_internal.h"

namespace gptq {
namespace {

constexpr int kBK = 32;  // k per stage

typedef __attribute__((address_space(3))) void lds_void_t;

#define GPTQ_VMCNT(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

struct GemmParams {
  int64_t M, N, K;
  float alpha, beta;
  const float* A;
  int64_t lda, sA;
  const float* B;
  int64_t ldb, sB;
  float* C;
  int64_t ldc, sC;
  int lower_tiles;
  int tri;  // 0: dense; 1: B lower-triangular (k >= n0); 2: A lower-triangular (k < m0 + T)
  int tiles_m, tiles_n, tiles;  // tile grid; tiles per batch entry
  int batch;
};

// Tile of workgroup b.  Workgroups go round-robin to the 8 XCDs (b % 8), each
// with its own L2: for equal tiles the tile list is cut into 8 contiguous
// ranges, one per XCD.  Dense tiles are listed in groups of 8 tile rows,
// column by column inside a group, so the tiles an XCD runs at once share rows
// of A and columns of B.  Lower-tile problems list the tiles (i >= j) row by
// row.
GPTQ_DEV bool gemm_tile(const GemmParams& p, int b, int& z, int& tm, int& tn) {
  constexpr int kXcd = 8;
  const int G = p.tiles * p.batch;
  if (p.tri != 0) {
    // Unequal tiles: listed heaviest first in dispatch order (the batch index
    // fastest), so every XCD gets an even mix and free slots take the
    // heaviest tiles left.  B lower-triangular: work falls with the column;
    // A lower-triangular: it grows with the row.
    if (b >= G) return false;
    const int t = b / p.batch;
    z = b - t * p.batch;
    if (p.tri == 1) {
      tn = t / p.tiles_m;
      tm = t - tn * p.tiles_m;
    } else {
      tm = p.tiles_m - 1 - t / p.tiles_n;
      tn = t % p.tiles_n;
    }
    return true;
  }
  const int x = b % kXcd, l = b / kXcd;
  const int base = G / kXcd, rem = G % kXcd;
  const int q = x * base + min(x, rem) + l;
  if (l >= base + (x < rem ? 1 : 0)) return false;
  z = q / p.tiles;
  const int t = q - z * p.tiles;
  if (p.lower_tiles) {
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
  return true;
}

// Buffer resource over `bytes` bytes at `base`; reads past the end return
// zeros in hardware.  Every field is workgroup-uniform.
GPTQ_DEV __amdgpu_buffer_rsrc_t gemm_rsrc(const float* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  const int64_t cl = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0LL : bytes);
  const int n = __builtin_amdgcn_readfirstlane(static_cast<int>(cl));
  void* b = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, static_cast<short>(0), n, 0x00020000);
}

// k-major operand stage (rows of A, or of B given as [N, K]): T rows x 32 k,
// 128-byte LDS rows; physical 16-byte chunk p of row r holds logical chunk
// p ^ ((r >> 1) & 7), which makes the MFMA operand reads (16 rows x 4 k per
// instruction) cover all 64 banks.  1 KB pieces of 8 rows, T / 32 per wave;
// chunks at or past ke read zeros.
template <int T>
GPTQ_DEV void dma_kmajor(__amdgpu_buffer_rsrc_t rs, uint8_t* slot, int64_t ld, int64_t k0, int64_t ke, int wave,
                         int lane) {
#pragma unroll
  for (int u = 0; u < T / 32; ++u) {
    const int q = (T / 32) * wave + u;
    const int r = 8 * q + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int64_t k = k0 + 4 * c;
    const uint32_t voff = (k < ke) ? static_cast<uint32_t>((r * ld + k) * 4) : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(slot + q * 1024), 16, voff, 0, 0, 0);
  }
}

// row-major B stage ([K, N]): 32 k-rows x T n, 4T-byte LDS rows; physical
// chunk p of k-row r holds logical chunk p ^ (4 (r & 3)).  rs starts at k-row
// k0 of the stage and column 0; columns at or past N read zeros.
template <int T>
GPTQ_DEV void dma_nmajor(__amdgpu_buffer_rsrc_t rs, uint8_t* slot, int64_t ld, int64_t n0, int64_t N, int wave,
                         int lane) {
  constexpr int kRowsPerPiece = 1024 / (4 * T);  // 4 (T = 64) or 2 (T = 128)
  constexpr int kChunks = T / 4;                 // 16-byte chunks per row
#pragma unroll
  for (int u = 0; u < T / 32; ++u) {
    const int q = (T / 32) * wave + u;
    const int r = kRowsPerPiece * q + lane / kChunks;
    const int c = (lane % kChunks) ^ (4 * (r & 3));
    const int64_t n = n0 + 4 * c;
    const uint32_t voff = (n < N) ? static_cast<uint32_t>((r * ld + n) * 4) : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(slot + q * 1024), 16, voff, 0, 0, 0);
  }
}

GPTQ_DEV float lds_f32(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const float*>(base + off);
}

// T x T output tile (T = 64 or 128), 2x2 waves of (T/2) x (T/2) on
// v_mfma_f32_16x16x4_f32.  The operands stream through a ring of S 32-k stages
// (S - 1 in flight), one LDS array per slot so the compiler's wait insertion
// sees no false aliasing.
template <bool TRANS_B, int T>
__global__ __launch_bounds__(256, T == 64 ? 3 : 2) void gemm_f32_kernel(GemmParams p) {
  constexpr int S = (T == 64) ? 3 : 2;  // ring slots
  constexpr int kOp = T * kBK * 4;      // one operand stage
  constexpr int NB = T / 32;            // 16x16 blocks per wave and dimension
  __shared__ __attribute__((aligned(1024))) uint8_t sa0[kOp], sa1[kOp], sa2[S == 3 ? kOp : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sb0[kOp], sb1[kOp], sb2[S == 3 ? kOp : 16];
  int z, tm, tn;
  if (!gemm_tile(p, blockIdx.x, z, tm, tn)) return;
  const int64_t m0 = static_cast<int64_t>(tm) * T;
  const int64_t n0 = static_cast<int64_t>(tn) * T;
  const float* A = p.A + z * p.sA;
  const float* B = p.B + z * p.sB;
  float* C = p.C + z * p.sC;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // K range of this tile: a lower-triangular operand is zero outside it
  int64_t kb = 0, ke = p.K;
  if (p.tri == 1) kb = n0;
  if (p.tri == 2) ke = min(p.K, m0 + T);
  const int nstage = (ke > kb) ? static_cast<int>((ke - kb + kBK - 1) / kBK) : 0;

  // C rows of this wave's block as float4 (row-contiguous), read two stages
  // before the end of the K loop: late enough that the workgroups starting
  // together do not all pull their C tiles at once, early enough that they
  // land during the last products.  A load instruction covers kCRows rows;
  // lane l takes row l / (T / 8), columns 4 (l % (T / 8)).
  constexpr int kC4 = T / 8;            // float4 per block row
  constexpr int kCRows = 64 / kC4;      // rows per instruction
  constexpr int kCLoads = (T / 2) / kCRows;
  f32x4_t cpre[kCLoads];
  const bool use_c = p.beta != 0.f;
  auto load_c = [&]() {
#pragma unroll
    for (int u = 0; u < kCLoads; ++u) {
      const int64_t m = m0 + wm * (T / 2) + u * kCRows + lane / kC4;
      const int64_t n = n0 + wn * (T / 2) + 4 * (lane % kC4);
      cpre[u] = (m < p.M && n < p.N) ? *reinterpret_cast<const f32x4_t*>(C + m * p.ldc + n)
                                     : f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  };

  f32x4_t acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const __amdgpu_buffer_rsrc_t rsA = gemm_rsrc(A + m0 * p.lda, min<int64_t>(p.M - m0, T) * p.lda * 4);
  const __amdgpu_buffer_rsrc_t rsBt =
      gemm_rsrc(B + (TRANS_B ? n0 * p.ldb : 0), TRANS_B ? min<int64_t>(p.N - n0, T) * p.ldb * 4 : 0);
  auto issue = [&](int s, uint8_t* da, uint8_t* db) {
    const int64_t k0 = kb + static_cast<int64_t>(s) * kBK;
    dma_kmajor<T>(rsA, da, p.lda, k0, ke, wave, lane);
    if (TRANS_B) {
      dma_kmajor<T>(rsBt, db, p.ldb, k0, ke, wave, lane);
    } else {
      const int64_t rows = min<int64_t>(ke - k0, kBK);
      dma_nmajor<T>(gemm_rsrc(B + k0 * p.ldb, rows * p.ldb * 4), db, p.ldb, n0, p.N, wave, lane);
    }
  };
  constexpr int kLoadsPerStage = 2 * (T / 32);  // DMA instructions per wave per stage

  // operand read offsets (bytes within a stage)
  uint32_t abase[NB], asw[NB], bbase[NB], bsw[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int r = wm * (T / 2) + 16 * i + (lane & 15);
    abase[i] = static_cast<uint32_t>(r * 128 + (lane >> 4) * 4);
    asw[i] = static_cast<uint32_t>(((r >> 1) & 7) * 16);
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int nn = wn * (T / 2) + 16 * j + (lane & 15);
    const int kk = lane >> 4;
    if (TRANS_B) {
      bbase[j] = static_cast<uint32_t>(nn * 128 + kk * 4);
      bsw[j] = static_cast<uint32_t>(((nn >> 1) & 7) * 16);
    } else {
      bbase[j] = static_cast<uint32_t>(kk * (4 * T) + (((nn >> 2) ^ (4 * kk)) * 16) + (nn & 3) * 4);
      bsw[j] = 0;
    }
  }
  auto compute = [&](const uint8_t* da, const uint8_t* db) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // half a stage of operands first, then its MFMAs
      float a[kBK / 8][NB], b[kBK / 8][NB];
#pragma unroll
      for (int tt = 0; tt < kBK / 8; ++tt) {
        const int t = h * (kBK / 8) + tt;
#pragma unroll
        for (int i = 0; i < NB; ++i) a[tt][i] = lds_f32(da, abase[i] + ((16u * t) ^ asw[i]));
#pragma unroll
        for (int j = 0; j < NB; ++j)
          b[tt][j] = TRANS_B ? lds_f32(db, bbase[j] + ((16u * t) ^ bsw[j]))
                             : lds_f32(db, bbase[j] + static_cast<uint32_t>(16 * T) * t);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep these reads above the MFMAs
#pragma unroll
      for (int tt = 0; tt < kBK / 8; ++tt)
#pragma unroll
        for (int i = 0; i < NB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[tt][i], b[tt][j], acc[i][j], 0, 0, 0);
    }
  };
  // Stage x lives in slot x % S.  Before computing stage x: wait until its
  // loads have landed (the loads issued after them may stay in flight: stage
  // x + 1 when S = 3, and C when it went out after stage x), barrier (all
  // waves' pieces are in; everyone is done with slot (x - 1) % S), then refill
  // that slot with stage x + S - 1; C follows the refill of step cst.
  const int cst = max(0, nstage - 2);
  auto step = [&](int x, const uint8_t* da, const uint8_t* db, uint8_t* na, uint8_t* nb) {
    if (x >= nstage) return;
    int later = (S == 3 && x + 1 < nstage) ? kLoadsPerStage : 0;
    if (use_c && cst <= x - 1 && cst >= x - (S - 1)) later += kCLoads;
    if (later == 0) __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(0));
    else if (later == kLoadsPerStage) __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(kLoadsPerStage));
    else if (later == kCLoads) __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(kCLoads));
    else __builtin_amdgcn_s_waitcnt(GPTQ_VMCNT(kCLoads + kLoadsPerStage));
    __builtin_amdgcn_s_barrier();
    if (x + S - 1 < nstage) issue(x + S - 1, na, nb);
    if (use_c && x == cst) load_c();
    compute(da, db);
  };
  if (nstage > 0) issue(0, sa0, sb0);
  else if (use_c) load_c();
  if constexpr (S == 3) {
    if (nstage > 1) issue(1, sa1, sb1);
    for (int s = 0; s < nstage; s += 3) {
      step(s, sa0, sb0, sa2, sb2);
      step(s + 1, sa1, sb1, sa0, sb0);
      step(s + 2, sa2, sb2, sa1, sb1);
    }
  } else {
    for (int s = 0; s < nstage; s += 2) {
      step(s, sa0, sb0, sa1, sb1);
      step(s + 1, sa1, sb1, sa0, sb0);
    }
  }
  // epilogue: each wave stages its (T/2) x (T/2) block in its own LDS slot
  // array (row-major; T = 128: 64-float rows, column bits 4-5 XOR-ed with
  // row bits 2-3; T = 64: rows padded to 36 floats), then writes C as float4
  // rows.  Accumulator element (i, j, e) is block row 16 i + 4 (lane >> 4) + e,
  // column 16 j + (lane & 15).  Lower-tile problems never write above the
  // 64-block diagonal.
  constexpr int kP = (T == 128) ? 64 : 36;
  auto xr = [&](int row) { return (T == 128) ? 16 * ((row >> 2) & 3) : 0; };
  __syncthreads();  // every wave is done with the ring
  float* stg = reinterpret_cast<float*>(S == 3 ? (wave == 0 ? sa0 : wave == 1 ? sa1 : wave == 2 ? sa2 : sb0)
                                              : (wave == 0 ? sa0 : wave == 1 ? sa1 : wave == 2 ? sb0 : sb1));
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * i + 4 * (lane >> 4) + e, col = 16 * j + (lane & 15);
        stg[row * kP + (col ^ xr(row))] = acc[i][j][e];
      }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
  for (int u = 0; u < kCLoads; ++u) {
    const int row = u * kCRows + lane / kC4, c4 = lane % kC4;
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stg + row * kP + ((4 * c4) ^ xr(row)));
    const int64_t m = m0 + wm * (T / 2) + row;
    const int64_t n = n0 + wn * (T / 2) + 4 * c4;
    const bool upper = p.lower_tiles && (m >> 6) < (n >> 6);
    if (m < p.M && n < p.N && !upper) {
      f32x4_t out = p.alpha * v;
      if (use_c) out += p.beta * cpre[u];
      *reinterpret_cast<f32x4_t*>(C + m * p.ldc + n) = out;
    }
  }
}

}  // namespace

hipError_t gemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const float* A, int64_t lda,
                    int64_t sA, const float* B, int64_t ldb, int64_t sB, bool transB, float beta,
                    float* C, int64_t ldc, int64_t sC, int batch, bool lower_tiles, int tri,
                    hipStream_t stream) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  GemmParams p{M, N, K, alpha, beta, A, lda, sA, B, ldb, sB, C, ldc, sC, lower_tiles ? 1 : 0, tri, 0, 0, 0, batch};
  // 128x128 tiles halve the operand bytes per flop; used when they still give
  // every CU a tile.  Lower-tile problems are square (the Cholesky update).
  auto count = [&](int T) {
    const int tm = static_cast<int>((M + T - 1) / T), tn = static_cast<int>((N + T - 1) / T);
    return lower_tiles ? tm * (tm + 1) / 2 : tm * tn;
  };
  // triangular operands make tiles unequal: small tiles, heaviest first, balance them
  const bool big = tri == 0 && static_cast<int64_t>(count(128)) * batch >= 256;
  const int T = big ? 128 : 64;
  p.tiles_m = static_cast<int>((M + T - 1) / T);
  p.tiles_n = static_cast<int>((N + T - 1) / T);
  p.tiles = count(T);
  const unsigned blocks = static_cast<unsigned>(static_cast<int64_t>(p.tiles) * batch);
  if (transB) {
    if (big) gemm_f32_kernel<true, 128><<<blocks, 256, 0, stream>>>(p);
    else gemm_f32_kernel<true, 64><<<blocks, 256, 0, stream>>>(p);
  } else {
    if (big) gemm_f32_kernel<false, 128><<<blocks, 256, 0, stream>>>(p);
    else gemm_f32_kernel<false, 64><<<blocks, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace gptq
