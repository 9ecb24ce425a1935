// Host-side driver for the sanitizer build of the C ABI (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only).  Every call below either
// returns an error before anything touches a GPU, or is a pure size query; the
// driver checks the status codes and exits non-zero on a mismatch.  No GPU is
// needed or used.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "gptq.h"

static int g_fail = 0;

#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);    \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

static gptq_config cfg(int bits, int g, float damp, int desc, int stat, int sym, int block) {
  gptq_config c;
  c.bits = bits;
  c.group_size = g;
  c.damp_percent = damp;
  c.desc_act = desc;
  c.static_groups = stat;
  c.sym = sym;
  c.block_size = block;
  return c;
}

int main() {
  const int64_t big = std::numeric_limits<int64_t>::max();
  void* fake = reinterpret_cast<void*>(static_cast<uintptr_t>(1) << 20);  // never dereferenced
  void* fake_mis = reinterpret_cast<void*>((static_cast<uintptr_t>(1) << 20) + 4);
  const gptq_config good = cfg(4, 128, 0.01f, 0, 0, 1, 128);

  // configuration rules
  EXPECT(gptq_config_validate(&good) == GPTQ_OK);
  EXPECT(gptq_config_validate(nullptr) == GPTQ_ERR_INVALID_ARG);
  const int bad_bits[] = {0, 1, 5, 7, 16, -4, std::numeric_limits<int>::min(), std::numeric_limits<int>::max()};
  for (int b : bad_bits) {
    gptq_config c = cfg(b, 128, 0.01f, 0, 0, 1, 128);
    EXPECT(gptq_config_validate(&c) == GPTQ_ERR_INVALID_ARG);
  }
  const int bad_groups[] = {0, -2, 48, 96, 200, std::numeric_limits<int>::min(), std::numeric_limits<int>::max()};
  for (int g : bad_groups) {
    gptq_config c = cfg(4, g, 0.01f, 0, 0, 1, 128);
    EXPECT(gptq_config_validate(&c) == GPTQ_ERR_INVALID_ARG);
  }
  const float bad_damp[] = {0.f, 1.f, -0.5f, 2.f, std::numeric_limits<float>::quiet_NaN(),
                            std::numeric_limits<float>::infinity()};
  for (float d : bad_damp) {
    gptq_config c = cfg(4, 128, d, 0, 0, 1, 128);
    EXPECT(gptq_config_validate(&c) == GPTQ_ERR_INVALID_ARG);
  }
  gptq_config c64 = cfg(4, 128, 0.01f, 0, 0, 1, 64);
  EXPECT(gptq_config_validate(&c64) == GPTQ_ERR_INVALID_ARG);

  // status strings: every code, and one past the end
  for (int s = 0; s <= 6; ++s) EXPECT(gptq_status_string(s) != nullptr);
  EXPECT(std::strcmp(gptq_status_string(99), "unknown status") == 0);
  EXPECT(std::strcmp(gptq_status_string(-1), "unknown status") == 0);

  // size queries at and past the limits: no overflow, 0 for what cannot be served
  const int64_t dims[] = {-1, 0, 1, 7, 8, 31, 32, 4096, 28672, int64_t{1} << 20, int64_t{1} << 31, int64_t{1} << 40,
                          big};
  for (int64_t d : dims) {
    for (int64_t n : dims) {
      (void)gptq_hessian_workspace_size(d, n, GPTQ_BF16);
      (void)gptq_hessian_workspace_size(d, n, GPTQ_F32);
      (void)gptq_workspace_size(n, d, &good);
      (void)gptq_dequant_workspace_size(n, d, 4096);
      (void)gptq_dequant_workspace_size(4, d, n);
      (void)gptq_dequant_ordered_workspace_size(n, d, 4096);
      for (int b : {2, 3, 4, 8, 5}) (void)gptq_dequant_noalloc_need(n, GPTQ_BF16, d, b, 4096);
    }
    (void)gptq_prepare_workspace_size(d);
  }
  EXPECT(gptq_hessian_workspace_size(0, 10, GPTQ_BF16) == 0);
  EXPECT(gptq_hessian_workspace_size(big, 10, GPTQ_BF16) == 0);
  EXPECT(gptq_prepare_workspace_size(big) == 0);
  EXPECT(gptq_workspace_size(big, big, &good) == 0);
  EXPECT(gptq_dequant_workspace_size(4, big, 4096) == 0);
  EXPECT(gptq_dequant_ordered_workspace_size(big, 4096, 4096) == 0);
  EXPECT(gptq_hessian_workspace_size(4096, 262144, GPTQ_BF16) > 0);
  EXPECT(gptq_prepare_workspace_size(4096) > 0);

  // the calls: rejected on the host before any launch
  float* S = static_cast<float*>(fake);
  EXPECT(gptq_hessian_accumulate(nullptr, 64, fake, GPTQ_BF16, 10, 64, fake, 1 << 20, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(S, 0, fake, GPTQ_BF16, 10, 64, fake, 1 << 20, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(S, 60, fake, GPTQ_BF16, 10, 64, fake, 1 << 20, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(S, 64, fake, GPTQ_BF16, 10, 32, fake, 1 << 20, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(S, 64, fake_mis, GPTQ_BF16, 10, 64, fake, 1 << 20, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(S, 64, fake, 7, 10, 64, fake, 1 << 20, nullptr) ==
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(S, 64, fake, GPTQ_BF16, -1, 64, fake, 1 << 20, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(S, big, fake, GPTQ_BF16, 10, big, fake, 1 << 20, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_hessian_accumulate(S, 64, fake, GPTQ_BF16, 0, 64, nullptr, 0, nullptr) == GPTQ_OK);  // no tokens
  EXPECT(gptq_hessian_accumulate(S, 64, fake, GPTQ_BF16, 10, 64, nullptr, 0, nullptr) == GPTQ_ERR_WORKSPACE);
  EXPECT(gptq_hessian_accumulate(S, 64, fake, GPTQ_BF16, 10, 64, fake_mis, 1 << 20, nullptr) == GPTQ_ERR_WORKSPACE);

  int32_t* ip = static_cast<int32_t*>(fake);
  EXPECT(gptq_prepare_hinv(nullptr, 64, 10, &good, S, ip, ip, fake, 1 << 24, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv(S, 64, 0, &good, S, ip, ip, fake, 1 << 24, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv(S, 62, 10, &good, S, ip, ip, fake, 1 << 24, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv(S, 64, 10, nullptr, S, ip, ip, fake, 1 << 24, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv(S, big, 10, &good, S, ip, ip, fake, 1 << 24, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_prepare_hinv(S, 64, 10, &good, S, ip, ip, fake, 16, nullptr) == GPTQ_ERR_WORKSPACE);

  uint8_t* codes = static_cast<uint8_t*>(fake);
  EXPECT(gptq_quantize_layer(fake, GPTQ_BF16, 8, 60, S, ip, &good, codes, S, ip, ip, nullptr, nullptr, fake, 1 << 24,
                             nullptr) == GPTQ_ERR_INVALID_ARG);  // d_in % 8
  gptq_config c3 = cfg(3, 32, 0.01f, 0, 0, 1, 128);
  EXPECT(gptq_quantize_layer(fake, GPTQ_BF16, 8, 48, S, ip, &c3, codes, S, ip, ip, nullptr, nullptr, fake, 1 << 24,
                             nullptr) == GPTQ_ERR_INVALID_ARG);  // 3 bits needs d_in % 32
  gptq_config cdesc = cfg(4, 128, 0.01f, 1, 0, 1, 128);
  EXPECT(gptq_quantize_layer(fake, GPTQ_BF16, 8, 64, S, nullptr, &cdesc, codes, S, ip, ip, nullptr, nullptr, fake,
                             1 << 24, nullptr) == GPTQ_ERR_INVALID_ARG);  // act-order without perm
  EXPECT(gptq_quantize_layer(fake, GPTQ_BF16, big, big, S, ip, &good, codes, S, ip, ip, nullptr, nullptr, fake,
                             1 << 24, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_quantize_layer(fake, GPTQ_BF16, 8, 64, S, ip, &good, codes, S, ip, ip, nullptr, nullptr, fake, 16,
                             nullptr) == GPTQ_ERR_WORKSPACE);

  EXPECT(gptq_pack(codes, 8, 60, 4, ip, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_pack(codes, 8, 64, 5, ip, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_pack(codes, 0, 64, 4, ip, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_pack(nullptr, 8, 64, 4, ip, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_pack(codes, big, big, 4, ip, nullptr) == GPTQ_ERR_INVALID_ARG);

  float* y = static_cast<float*>(fake);
  EXPECT(gptq_dequant_matmul(fake, GPTQ_BF16, 4, 48, ip, S, ip, ip, 4, 64, 1, y, fake, 1 << 20, nullptr) ==
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_dequant_matmul(fake, GPTQ_BF16, 4, 64, ip, S, ip, ip, 4, 64, 0, y, fake, 1 << 20, nullptr) ==
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_dequant_matmul(fake, GPTQ_BF16, big, 64, ip, S, ip, ip, 4, 64, 1, y, fake, 1 << 20, nullptr) ==
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_dequant_matmul(fake, GPTQ_BF16, 4, big / 2, ip, S, ip, ip, 4, 64, 1, y, fake, 1 << 20, nullptr) ==
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_dequant_matmul(fake, GPTQ_BF16, 4, 4096, ip, S, ip, ip, 4, 4096, 32, y, fake, 16, nullptr) ==
         GPTQ_ERR_WORKSPACE);
  EXPECT(gptq_dequant_matmul_noalloc(fake, GPTQ_BF16, 4, 48, ip, S, ip, ip, 4, 64, 1, y, nullptr) ==
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_dequant_matmul_noalloc(fake, GPTQ_F32, 16, 8192, ip, S, ip, ip, 4, 28672, 64, y, nullptr) ==
         GPTQ_ERR_TOO_LARGE);
  EXPECT(gptq_dequant_matmul_noalloc(fake, GPTQ_BF16, big, 4096, ip, S, ip, ip, 4, 4096, 32, y, nullptr) ==
         GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_dequant_order(ip, ip, 4, 48, 64, ip, ip, ip, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_dequant_order(ip, ip, 4, big / 2, big / 2, ip, ip, ip, nullptr) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_dequant_matmul_ordered(fake, GPTQ_BF16, 4, 4096, ip, S, ip, ip, nullptr, 4, 4096, 32, y, fake, 1 << 26,
                                     nullptr) == GPTQ_ERR_INVALID_ARG);

  // phase timing bookkeeping (host only: nothing recorded, nothing to wait for)
  EXPECT(gptq_phase_count() > 0);
  for (int p = 0; p < gptq_phase_count(); ++p) EXPECT(gptq_phase_name(p) != nullptr);
  EXPECT(gptq_phase_name(-1) == nullptr && gptq_phase_name(gptq_phase_count()) == nullptr);
  float ms[16];
  int32_t cnt[16];
  EXPECT(gptq_phase_read(nullptr, cnt, 4) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_phase_read(ms, cnt, 0) == GPTQ_ERR_INVALID_ARG);
  EXPECT(gptq_phase_timing(1) == GPTQ_OK);
  EXPECT(gptq_phase_read(ms, cnt, 16) == GPTQ_OK);
  EXPECT(gptq_phase_timing(0) == GPTQ_OK);
  for (int p = 0; p < gptq_phase_count(); ++p) EXPECT(cnt[p] == 0 && ms[p] == 0.f);

  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("abi sanitize driver: all checks passed\n");
  return 0;
}
