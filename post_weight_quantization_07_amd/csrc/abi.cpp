// C ABI of the GPTQ layer solve: argument checks, workspace sizing and the
// launch sequence of each call.  Declarations and contracts: include/gptq.h.
#include "../../include/gptq.h"

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gptq_internal.h"

namespace {

constexpr int kBlock = 128;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

gptq_status from_hip(hipError_t e) { return e == hipSuccess ? GPTQ_OK : GPTQ_ERR_HIP; }

bool bits_ok(int32_t b) { return b == 2 || b == 3 || b == 4 || b == 8; }

// size limits of every call: channels and output rows up to 2^20 (an H of
// that size would take 4 TiB), tokens up to 2^40; beyond them no size
// computation of the library can overflow
constexpr int64_t kMaxDim = int64_t{1} << 20;
constexpr int64_t kMaxTokens = int64_t{1} << 40;
bool dim_ok(int64_t v) { return v > 0 && v <= kMaxDim; }
bool tokens_ok(int64_t n) { return n >= 0 && n <= kMaxTokens; }

// d_in % (32 / bits) == 0, and d_in % 32 == 0 for 3 bits: whole words per row
bool packable(int64_t d_in, int32_t bits) {
  if (!bits_ok(bits) || d_in <= 0) return false;
  const int64_t m = (bits == 3) ? 32 : 32 / bits;
  return d_in % m == 0;
}

}  // namespace

extern "C" {

const char* gptq_status_string(int32_t s) {
  switch (s) {
    case GPTQ_OK: return "ok";
    case GPTQ_ERR_INVALID_ARG: return "invalid argument";
    case GPTQ_ERR_NOT_SPD: return "damped Hessian is not positive definite";
    case GPTQ_ERR_HIP: return "HIP runtime error";
    case GPTQ_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case GPTQ_ERR_TOO_LARGE: return "the call needs more scratch memory than the library's fixed buffer holds";
  }
  return "unknown status";
}

gptq_status gptq_config_validate(const gptq_config* c) {
  if (!c) return GPTQ_ERR_INVALID_ARG;
  if (!bits_ok(c->bits)) return GPTQ_ERR_INVALID_ARG;
  if (!(c->group_size == -1 || c->group_size > 0)) return GPTQ_ERR_INVALID_ARG;
  if (!(c->damp_percent > 0.0f && c->damp_percent < 1.0f)) return GPTQ_ERR_INVALID_ARG;
  if (c->block_size != kBlock) return GPTQ_ERR_INVALID_ARG;
  if (c->group_size > 0 && !(kBlock % c->group_size == 0 || c->group_size % kBlock == 0))
    return GPTQ_ERR_INVALID_ARG;
  return GPTQ_OK;
}

size_t gptq_hessian_workspace_size(int64_t d_in, int64_t n_tokens, int32_t xt) {
  if (!dim_ok(d_in) || !tokens_ok(n_tokens) || (xt != GPTQ_F32 && xt != GPTQ_BF16)) return 0;
  return gptq::hessian_plan(d_in, n_tokens, xt == GPTQ_BF16, device_cus()).ws_bytes;
}

gptq_status gptq_hessian_accumulate(float* S, int64_t d_in, const void* X, int32_t xt, int64_t n_tokens,
                                    int64_t ldx, void* ws, size_t ws_bytes, void* stream) {
  if (!S || !dim_ok(d_in) || !tokens_ok(n_tokens) || (xt != GPTQ_F32 && xt != GPTQ_BF16)) return GPTQ_ERR_INVALID_ARG;
  if (n_tokens == 0) return GPTQ_OK;
  const bool bf16 = (xt == GPTQ_BF16);
  const int64_t vec = bf16 ? 8 : 4;
  if (!X || d_in % vec != 0 || ldx < d_in || ldx % vec != 0 || !aligned16(X) || !aligned16(S))
    return GPTQ_ERR_INVALID_ARG;
  if (ldx > (int64_t{1} << 24)) return GPTQ_ERR_INVALID_ARG;  // 32-bit in-stage offsets
  const gptq::HessPlan plan = gptq::hessian_plan(d_in, n_tokens, bf16, device_cus());
  if (!ws || ws_bytes < plan.ws_bytes || !aligned256(ws)) return GPTQ_ERR_WORKSPACE;
  return from_hip(gptq::hessian_launch(plan, S, d_in, X, bf16, n_tokens, ldx, ws,
                                       static_cast<hipStream_t>(stream)));
}

size_t gptq_prepare_workspace_size(int64_t d_in) {
  if (!dim_ok(d_in)) return 0;
  return gptq::prepare_layout(d_in).ws_bytes;
}

gptq_status gptq_prepare_hinv(float* S_to_H, int64_t d_in, int64_t n_total, const gptq_config* cfg, float* U,
                              int32_t* perm, int32_t* info_dev, void* ws, size_t ws_bytes, void* stream) {
  if (!S_to_H || !U || !perm || !info_dev || !dim_ok(d_in) || n_total <= 0) return GPTQ_ERR_INVALID_ARG;
  if (gptq_config_validate(cfg) != GPTQ_OK) return GPTQ_ERR_INVALID_ARG;
  if (d_in % 4 != 0 || !aligned16(S_to_H) || !aligned16(U)) return GPTQ_ERR_INVALID_ARG;
  const gptq::PrepLayout lay = gptq::prepare_layout(d_in);
  if (!ws || ws_bytes < lay.ws_bytes || !aligned256(ws)) return GPTQ_ERR_WORKSPACE;
  return from_hip(gptq::prepare_launch(S_to_H, d_in, n_total, cfg->damp_percent, cfg->desc_act != 0, U, perm,
                                       info_dev, ws, static_cast<hipStream_t>(stream)));
}

size_t gptq_workspace_size(int64_t d_out, int64_t d_in, const gptq_config* cfg) {
  if (!dim_ok(d_out) || !dim_ok(d_in) || gptq_config_validate(cfg) != GPTQ_OK) return 0;
  return gptq::quant_layout(d_out, d_in, gptq::quant_planes(cfg->group_size, cfg->static_groups != 0)).ws_bytes;
}

gptq_status gptq_quantize_layer(const void* W, int32_t wt, int64_t d_out, int64_t d_in, const float* U,
                                const int32_t* perm, const gptq_config* cfg, uint8_t* codes, float* scales,
                                int32_t* zeros, int32_t* g_idx, float* Q_or_null, float* row_loss_or_null,
                                void* ws, size_t ws_bytes, void* stream) {
  if (gptq_config_validate(cfg) != GPTQ_OK) return GPTQ_ERR_INVALID_ARG;
  if (!W || !U || !codes || !scales || !zeros || !g_idx || !dim_ok(d_out) || !dim_ok(d_in)) return GPTQ_ERR_INVALID_ARG;
  if (wt != GPTQ_F32 && wt != GPTQ_BF16) return GPTQ_ERR_INVALID_ARG;
  if (cfg->desc_act && !perm) return GPTQ_ERR_INVALID_ARG;
  if (!packable(d_in, cfg->bits)) return GPTQ_ERR_INVALID_ARG;
  if (!aligned16(U) || !aligned16(codes) || (Q_or_null && !aligned16(Q_or_null))) return GPTQ_ERR_INVALID_ARG;
  const gptq::QuantLayout lay =
      gptq::quant_layout(d_out, d_in, gptq::quant_planes(cfg->group_size, cfg->static_groups != 0));
  if (!ws || ws_bytes < lay.ws_bytes || !aligned256(ws)) return GPTQ_ERR_WORKSPACE;
  return from_hip(gptq::quantize_launch(W, wt == GPTQ_BF16, d_out, d_in, U, perm, cfg->bits, cfg->group_size,
                                        cfg->sym != 0, cfg->static_groups != 0, codes, scales, zeros, g_idx,
                                        Q_or_null, row_loss_or_null, ws, static_cast<hipStream_t>(stream),
                                        cfg->desc_act == 0));
}

gptq_status gptq_pack(const uint8_t* codes, int64_t d_out, int64_t d_in, int32_t bits, int32_t* qweight,
                      void* stream) {
  if (!codes || !qweight || !dim_ok(d_out) || !dim_ok(d_in)) return GPTQ_ERR_INVALID_ARG;
  if (!packable(d_in, bits)) return GPTQ_ERR_INVALID_ARG;
  return from_hip(gptq::pack_launch(codes, d_out, d_in, bits, qweight, static_cast<hipStream_t>(stream)));
}

size_t gptq_dequant_workspace_size(int64_t m, int64_t d_in, int64_t d_out) {
  if (m <= 0 || !tokens_ok(m) || !dim_ok(d_in) || !dim_ok(d_out) || d_in % 32 != 0) return 0;
  return gptq::dequant_workspace_bytes(m, d_in, d_out);
}

gptq_status gptq_dequant_matmul(const void* x, int32_t xt, int64_t m, int64_t d_in, const int32_t* qweight,
                                const float* scales, const int32_t* zeros, const int32_t* g_idx, int32_t bits,
                                int64_t d_out, int32_t n_groups, float* y, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!x || !qweight || !scales || !zeros || !g_idx || !y) return GPTQ_ERR_INVALID_ARG;
  if (m <= 0 || !tokens_ok(m) || !dim_ok(d_out) || !dim_ok(d_in) || d_in % 32 != 0 || n_groups <= 0)
    return GPTQ_ERR_INVALID_ARG;
  if (!bits_ok(bits) || (xt != GPTQ_F32 && xt != GPTQ_BF16)) return GPTQ_ERR_INVALID_ARG;
  // qweight and scales / zeros are addressed with 32-bit byte offsets
  if (d_in / 32 * bits * d_out * 4 >= (int64_t{1} << 31) || int64_t{n_groups} * d_out * 4 >= (int64_t{1} << 31))
    return GPTQ_ERR_INVALID_ARG;
  const size_t need = gptq::dequant_workspace_bytes(m, d_in, d_out);
  if (need > 0 && (!ws || ws_bytes < need || !aligned256(ws))) return GPTQ_ERR_WORKSPACE;
  return from_hip(gptq::dequant_matmul_launch(x, xt == GPTQ_BF16, m, d_in, qweight, scales, zeros, g_idx, bits, d_out,
                                              n_groups, y, ws, static_cast<hipStream_t>(stream)));
}

size_t gptq_dequant_scratch_bytes(void) { return gptq::kDequantScratchBytes; }

size_t gptq_dequant_noalloc_need(int64_t m, int32_t xt, int64_t d_in, int32_t bits, int64_t d_out) {
  if (m <= 0 || !tokens_ok(m) || !dim_ok(d_in) || !dim_ok(d_out) || d_in % 32 != 0 || !bits_ok(bits)) return 0;
  if (xt != GPTQ_F32 && xt != GPTQ_BF16) return 0;
  return gptq::dequant_partial_bytes(m, d_in, d_out, xt == GPTQ_BF16, bits);
}

gptq_status gptq_dequant_matmul_noalloc(const void* x, int32_t xt, int64_t m, int64_t d_in,
                                        const int32_t* qweight, const float* scales, const int32_t* zeros,
                                        const int32_t* g_idx, int32_t bits, int64_t d_out, int32_t n_groups,
                                        float* y, void* stream) {
  if (!x || !qweight || !scales || !zeros || !g_idx || !y) return GPTQ_ERR_INVALID_ARG;
  if (m <= 0 || !tokens_ok(m) || !dim_ok(d_out) || !dim_ok(d_in) || d_in % 32 != 0 || n_groups <= 0)
    return GPTQ_ERR_INVALID_ARG;
  if (!bits_ok(bits) || (xt != GPTQ_F32 && xt != GPTQ_BF16)) return GPTQ_ERR_INVALID_ARG;
  if (d_in / 32 * bits * d_out * 4 >= (int64_t{1} << 31) || int64_t{n_groups} * d_out * 4 >= (int64_t{1} << 31))
    return GPTQ_ERR_INVALID_ARG;
  if (gptq::dequant_partial_bytes(m, d_in, d_out, xt == GPTQ_BF16, bits) > gptq::kDequantScratchBytes)
    return GPTQ_ERR_TOO_LARGE;
  void* ws = nullptr;
  const gptq_status st = from_hip(gptq::dequant_scratch(&ws));
  if (st != GPTQ_OK) return st;
  return from_hip(gptq::dequant_matmul_launch(x, xt == GPTQ_BF16, m, d_in, qweight, scales, zeros, g_idx, bits, d_out,
                                              n_groups, y, ws, static_cast<hipStream_t>(stream)));
}

gptq_status gptq_dequant_order(const int32_t* qweight, const int32_t* g_idx, int32_t bits, int64_t d_in,
                               int64_t d_out, int32_t* qweight_out, int32_t* g_idx_out, int32_t* order,
                               void* stream) {
  if (!qweight || !g_idx || !qweight_out || !g_idx_out || !order) return GPTQ_ERR_INVALID_ARG;
  if (!dim_ok(d_out) || !dim_ok(d_in) || d_in % 32 != 0 || !bits_ok(bits)) return GPTQ_ERR_INVALID_ARG;
  if (d_in / 32 * bits * d_out * 4 >= (int64_t{1} << 31)) return GPTQ_ERR_INVALID_ARG;
  return from_hip(gptq::dequant_order_launch(qweight, g_idx, bits, d_in, d_out, qweight_out, g_idx_out, order,
                                             static_cast<hipStream_t>(stream)));
}

size_t gptq_dequant_ordered_workspace_size(int64_t m, int64_t d_in, int64_t d_out) {
  if (m <= 0 || !tokens_ok(m) || !dim_ok(d_in) || !dim_ok(d_out) || d_in % 32 != 0) return 0;
  return gptq::dequant_ordered_workspace_bytes(m, d_in, d_out);
}

gptq_status gptq_dequant_matmul_ordered(const void* x, int32_t xt, int64_t m, int64_t d_in,
                                        const int32_t* qweight, const float* scales, const int32_t* zeros,
                                        const int32_t* g_idx, const int32_t* order, int32_t bits, int64_t d_out,
                                        int32_t n_groups, float* y, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !qweight || !scales || !zeros || !g_idx || !order || !y) return GPTQ_ERR_INVALID_ARG;
  if (m <= 0 || !tokens_ok(m) || !dim_ok(d_out) || !dim_ok(d_in) || d_in % 32 != 0 || n_groups <= 0)
    return GPTQ_ERR_INVALID_ARG;
  if (!bits_ok(bits) || (xt != GPTQ_F32 && xt != GPTQ_BF16)) return GPTQ_ERR_INVALID_ARG;
  if (d_in / 32 * bits * d_out * 4 >= (int64_t{1} << 31) || int64_t{n_groups} * d_out * 4 >= (int64_t{1} << 31))
    return GPTQ_ERR_INVALID_ARG;
  const size_t need = gptq::dequant_ordered_workspace_bytes(m, d_in, d_out);
  if (!ws || ws_bytes < need || !aligned256(ws)) return GPTQ_ERR_WORKSPACE;
  return from_hip(gptq::dequant_matmul_ordered_launch(x, xt == GPTQ_BF16, m, d_in, qweight, scales, zeros, g_idx,
                                                      order, bits, d_out, n_groups, y, ws,
                                                      static_cast<hipStream_t>(stream)));
}

gptq_status gptq_phase_timing(int32_t enable) { return from_hip(gptq::phase_timing_set(enable != 0)); }

int32_t gptq_phase_count(void) { return gptq::kNumPhases; }

const char* gptq_phase_name(int32_t phase) { return gptq::phase_name(phase); }

gptq_status gptq_phase_read(float* ms, int32_t* launches, int32_t n) {
  if (!ms || !launches || n <= 0) return GPTQ_ERR_INVALID_ARG;
  return from_hip(gptq::phase_timing_read(ms, launches, n));
}

}  // extern "C"
