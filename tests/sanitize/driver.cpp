// Exercises the C-ABI entry points' argument validation under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only; the kernel launchers are stubs that count
// calls).  Pointers are fake device addresses: validation only compares and offsets them.
// Each case states the status it must return; extreme sizes check that the size arithmetic
// of the validators is free of overflow (UBSan aborts on signed overflow).
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "../../include/mmdit.h"

extern int g_launches;

static int g_fail = 0, g_cases = 0;
#define EXPECT(call, want)                                                                       \
  do {                                                                                           \
    ++g_cases;                                                                                   \
    const int got_ = (call);                                                                     \
    if ((want) >= 0 ? got_ != (want) : got_ == 0) {                                              \
      std::printf("FAIL line %d: %s -> %d (want %d): %s\n", __LINE__, #call, got_, (want),       \
                  mmdit_last_error());                                                           \
      ++g_fail;                                                                                  \
    }                                                                                            \
  } while (0)
static void* fk(uintptr_t a) { return reinterpret_cast<void*>(a); }
static float* ff(uintptr_t a) { return reinterpret_cast<float*>(a); }

int main() {
  const int OK = MMDIT_OK, ANYERR = -1;
  const int64_t BIG = std::numeric_limits<int64_t>::max();
  void *p = fk(0x10000), *o = fk(0x900000), *o2 = fk(0xA00000);

  // ---- modulate_ln
  EXPECT(mmdit_modulate_ln(p, MMDIT_BF16, nullptr, MMDIT_BF16, nullptr, nullptr, ff(0x20000), ff(0x30000), 3072, o,
                           MMDIT_BF16, 1, 4, 3072, 1e-6f, nullptr), OK);
  EXPECT(mmdit_modulate_ln(p, MMDIT_BF16, nullptr, MMDIT_BF16, nullptr, nullptr, ff(0x20000), ff(0x30000), 3072, o,
                           MMDIT_BF16, 1, 4, 3004, 1e-6f, nullptr), MMDIT_ERR_SHAPE);
  EXPECT(mmdit_modulate_ln(p, MMDIT_BF16, p, MMDIT_BF16, nullptr, nullptr, ff(0x20000), ff(0x30000), 3072, o,
                           MMDIT_BF16, 1, 4, 3072, 1e-6f, nullptr), MMDIT_ERR_NULL);
  EXPECT(mmdit_modulate_ln(p, MMDIT_BF16, nullptr, MMDIT_BF16, nullptr, nullptr, ff(0x20000), ff(0x30000), 3072, p,
                           MMDIT_BF16, 1, 4, 3072, 1e-6f, nullptr), MMDIT_ERR_ALIAS);
  EXPECT(mmdit_modulate_ln(p, MMDIT_BF16, nullptr, MMDIT_BF16, nullptr, nullptr, ff(0x20000), ff(0x30000), 3072, o,
                           MMDIT_BF16, BIG, BIG, 3072, 1e-6f, nullptr), ANYERR);

  // ---- qk_norm_rope
  mmdit_rope3d rope{2, 2, 2, 16, 56, 56, 10000.f};
  mmdit_rope3d bad_rope{2, 2, 2, 16, 55, 57, 10000.f};
  mmdit_rope3d huge_rope{BIG, BIG, 2, 16, 56, 56, 10000.f};
  EXPECT(mmdit_qk_norm_rope(p, fk(0x20000), MMDIT_BF16, 384, p, p, MMDIT_BF16, 0, p, fk(0x20000), MMDIT_BF16, 384, 1,
                            8, 1, 128, 1e-6f, &rope, nullptr), OK);                       // in place
  EXPECT(mmdit_qk_norm_rope(p, fk(0x20000), MMDIT_BF16, 384, p, p, MMDIT_BF16, 0, p, fk(0x20000), MMDIT_BF16, 384, 1,
                            8, 1, 128, 1e-6f, &bad_rope, nullptr), MMDIT_ERR_SHAPE);
  EXPECT(mmdit_qk_norm_rope(p, fk(0x20000), MMDIT_BF16, 384, p, p, MMDIT_BF16, 0, fk(0x10080), fk(0x20000), MMDIT_BF16,
                            384, 1, 8, 1, 128, 1e-6f, &rope, nullptr), MMDIT_ERR_ALIAS);
  EXPECT(mmdit_qk_norm_rope(p, fk(0x20000), MMDIT_BF16, 384, p, p, MMDIT_BF16, 0, p, fk(0x20000), MMDIT_BF16, 384, 1,
                            8, 1, 128, 1e-6f, &huge_rope, nullptr), ANYERR);
  EXPECT(mmdit_qk_norm_rope(p, fk(0x20000), MMDIT_BF16, BIG, p, p, MMDIT_BF16, 0, o, o2, MMDIT_BF16, BIG, BIG, BIG,
                            1, 128, 1e-6f, nullptr, nullptr), ANYERR);

  // ---- joint attention (workspace, no-alloc, 8-bit)
  auto ja = [&](int64_t nv, int64_t nc, int64_t stride, int64_t B, int64_t H, void* ov, void* oc, float* lse,
                void* ws, size_t wsb) {
    return mmdit_joint_attention(p, p, p, nv, p, p, p, nc, MMDIT_BF16, MMDIT_BF16, stride, B, H, 128, 0.088f, ov, oc,
                                 MMDIT_F32, stride, lse, ws, wsb, nullptr);
  };
  EXPECT(ja(10, 3, 256, 1, 2, o, o2, nullptr, nullptr, 0), OK);
  EXPECT(ja(10, 3, 256, 1, 2, o, o2, nullptr, fk(0xB00000), 1 << 20), OK);
  EXPECT(ja(10, 3, 256, 1, 2, o, o2, nullptr, p, 1 << 20), MMDIT_ERR_ALIAS);
  EXPECT(ja(10, 3, 256, 1, 2, o, o2, ff(0xC00000), fk(0xC00000), 256), MMDIT_ERR_ALIAS);
  EXPECT(ja(10, 3, 256, 1, 2, p, o2, nullptr, nullptr, 0), MMDIT_ERR_ALIAS);
  EXPECT(ja(BIG, BIG, BIG, BIG, BIG, o, o2, nullptr, nullptr, 0), ANYERR);
  EXPECT(ja(BIG / 2, 3, 256, 3, 2, o, o2, nullptr, nullptr, 0), ANYERR);
  EXPECT(mmdit_joint_attention_noalloc(p, p, p, 10, p, p, p, 3, MMDIT_BF16, MMDIT_BF16, 256, 1, 2, 128, 0.088f, p, o2,
                                       MMDIT_F32, 256, nullptr, nullptr), ANYERR);       // alias, or no device
  EXPECT(mmdit_cast(p, MMDIT_BF16, fk(0x90000000), MMDIT_F16, 1000, nullptr), OK);
  EXPECT(mmdit_cast(p, MMDIT_BF16, p, MMDIT_F16, 1000, nullptr), OK);                       // in place
  EXPECT(mmdit_cast(p, MMDIT_F32, p, MMDIT_F16, 1000, nullptr), MMDIT_ERR_ALIAS);
  EXPECT(mmdit_cast(p, MMDIT_BF16, fk(0x90000000), MMDIT_F16, BIG, nullptr), ANYERR);
  mmdit_attn8_stream st{fk(0x10000000), ff(0x20000000), fk(0x30000000), ff(0x40000000), fk(0x50000000)};
  EXPECT(mmdit_attn8_quantize(p, p, p, 100, nullptr, nullptr, nullptr, 0, MMDIT_BF16, 3072, 1, 24, 128, &st, nullptr,
                              ff(0x60000000), nullptr), OK);
  EXPECT(mmdit_attn8_quantize(p, p, p, BIG, nullptr, nullptr, nullptr, 0, MMDIT_BF16, 3072, BIG, 24, 128, &st,
                              nullptr, ff(0x60000000), nullptr), ANYERR);
  EXPECT(mmdit_joint_attention_8bit(&st, 100, nullptr, 0, ff(0x60000000), 1, 24, 128, 0.088f, fk(0x70000000), nullptr,
                                    MMDIT_F32, 3072, nullptr, nullptr, 0, nullptr), OK);
  EXPECT(mmdit_joint_attention_8bit(&st, 100, nullptr, 0, ff(0x60000000), 1, 24, 128, 0.088f, fk(0x10000000), nullptr,
                                    MMDIT_F32, 3072, nullptr, nullptr, 0, nullptr), MMDIT_ERR_ALIAS);
  EXPECT(mmdit_joint_attention_8bit(&st, BIG, nullptr, 0, ff(0x60000000), BIG, BIG, 128, 0.088f, fk(0x70000000),
                                    nullptr, MMDIT_F32, 3072, nullptr, nullptr, 0, nullptr), ANYERR);

  // ---- linear, FP8, modulation, timestep path, Lite regrouping
  EXPECT(mmdit_linear(p, fk(0x20000), MMDIT_BF16, nullptr, MMDIT_BF16, o, MMDIT_BF16, 10, 256, 128, MMDIT_EPI_NONE,
                      nullptr, MMDIT_F32, nullptr, 0, 10, nullptr), OK);
  EXPECT(mmdit_linear(p, fk(0x20000), MMDIT_BF16, nullptr, MMDIT_BF16, o, MMDIT_BF16, 10, 256, 100, MMDIT_EPI_NONE,
                      nullptr, MMDIT_F32, nullptr, 0, 10, nullptr), MMDIT_ERR_SHAPE);
  EXPECT(mmdit_linear(p, fk(0x20000), MMDIT_BF16, nullptr, MMDIT_BF16, o, MMDIT_BF16, BIG, BIG, 1 << 20,
                      MMDIT_EPI_NONE, nullptr, MMDIT_F32, nullptr, 0, 10, nullptr), ANYERR);
  EXPECT(mmdit_quantize_fp8(p, MMDIT_BF16, 4, 16, 1, o, ff(0xA00000), nullptr), OK);
  EXPECT(mmdit_quantize_fp8(p, MMDIT_BF16, BIG, BIG, 1, o, ff(0xA00000), nullptr), ANYERR);
  EXPECT(mmdit_linear_fp8(p, ff(0xB00000), fk(0x20000), ff(0xB00100), nullptr, MMDIT_BF16, o, MMDIT_F32, 10, 256,
                          128, MMDIT_EPI_NONE, nullptr, MMDIT_F32, nullptr, 0, 10, nullptr), OK);
  EXPECT(mmdit_linear_fp8(p, ff(0xB00000), fk(0x20000), ff(0xB00100), nullptr, MMDIT_BF16, o, MMDIT_F32, BIG, BIG,
                          BIG - 63, MMDIT_EPI_NONE, nullptr, MMDIT_F32, nullptr, 0, 10, nullptr), ANYERR);
  EXPECT(mmdit_modulation(p, nullptr, fk(0x20000), MMDIT_BF16, ff(0x900000), 1, 18432, 1536, nullptr), OK);
  EXPECT(mmdit_modulation(p, nullptr, fk(0x20000), MMDIT_BF16, ff(0x900000), BIG, BIG, BIG, nullptr), ANYERR);
  EXPECT(mmdit_timestep_embed(ff(0x10000), 2, fk(0x20000), nullptr, fk(0x20000), nullptr, fk(0x20000), nullptr,
                              MMDIT_BF16, 256, 3072, 16, 10000.f, ff(0x90000000), ff(0xA0000000), ff(0xB0000000),
                              nullptr), OK);
  EXPECT(mmdit_timestep_embed(ff(0x10000), BIG, p, nullptr, p, nullptr, p, nullptr, MMDIT_BF16, 256, BIG & ~7, 16,
                              10000.f, ff(0x900000), ff(0xA00000), ff(0xB00000), nullptr), ANYERR);
  EXPECT(mmdit_lite_merge(p, MMDIT_BF16, p, nullptr, MMDIT_BF16, fk(0x90000000), MMDIT_F32, 1, 21, 30, 52, 3072,
                          nullptr), OK);
  EXPECT(mmdit_lite_unpatchify(p, MMDIT_BF16, p, nullptr, MMDIT_BF16, fk(0x90000000), MMDIT_F32, BIG, BIG, 30, 52,
                               3072, nullptr), ANYERR);

  // ---- block: workspace arithmetic and validation
  mmdit_block_dims d{3072, 24, 128, 12288, 1536, 1e-6f, 1e-6f, 0, MMDIT_BF16, MMDIT_F16};
  const size_t need = mmdit_block_workspace_bytes(&d, 1, 32760, 512);
  ++g_cases;
  if (need == 0) { std::printf("FAIL: block workspace of the 480p block is 0\n"); ++g_fail; }
  ++g_cases;
  if (mmdit_block_workspace_bytes(&d, BIG, BIG, BIG) != 0) {
    // a size that cannot be represented must be refused, not wrapped
    std::printf("FAIL: block workspace of an unrepresentable size is not 0\n"); ++g_fail;
  }
  size_t offs[2 * MMDIT_WS_COUNT];
  EXPECT(mmdit_block_workspace_offsets(&d, 1, 32760, 512, offs), OK);
  mmdit_stream_weights w;
  std::memset(&w, 0, sizeof(w));
  mmdit_rope3d grid{21, 30, 52, 16, 56, 56, 10000.f};
  EXPECT(mmdit_block_fwd(&d, &w, &w, p, p, MMDIT_BF16, p, MMDIT_BF16, &grid, 512, o, o2, MMDIT_F32, fk(0x100000),
                         1024, 1, nullptr), MMDIT_ERR_NULL);
  void** ws = reinterpret_cast<void**>(&w);
  for (size_t i = 0; i < sizeof(w) / sizeof(void*); ++i) ws[i] = fk(0x20000);
  EXPECT(mmdit_block_fwd(&d, &w, &w, p, p, MMDIT_BF16, p, MMDIT_BF16, &grid, 512, o, o2, MMDIT_F32, fk(0x100000),
                         1024, 1, nullptr), MMDIT_ERR_WORKSPACE);
  EXPECT(mmdit_block_fwd(&d, &w, &w, p, p, MMDIT_BF16, p, MMDIT_BF16, &grid, 512, o, o2, MMDIT_F32, fk(0x100000),
                         need, 1, nullptr), OK);
  EXPECT(mmdit_block_fwd(&d, &w, &w, p, p, MMDIT_BF16, p, MMDIT_BF16, &huge_rope, 512, o, o2, MMDIT_F32,
                         fk(0x100000), need, BIG, nullptr), ANYERR);

  std::printf("%d cases, %d failures, %d launches reached\n", g_cases, g_fail, g_launches);
  if (g_fail == 0) std::printf("ALL OK\n");
  return g_fail ? 1 : 0;
}
