// Host-only stand-ins for the kernel launchers, so that the C-ABI entry points' argument
// validation can be built with AddressSanitizer / UndefinedBehaviorSanitizer and run on a
// machine without a GPU: every launcher only counts its calls and reports success.
#include "../../video_diffusion_transformer_mmdit_amd/csrc/common.h"

int g_launches = 0;

namespace mmdit {
int launch_modulate_ln(const void*, int, const void*, int, const float*, float*, const float*, const float*, int64_t,
                       void*, int, int64_t, int64_t, int64_t, float, hipStream_t) { ++g_launches; return MMDIT_OK; }
int launch_qk_norm_rope(const void*, const void*, int, int64_t, const void*, const void*, int, int64_t, void*, void*,
                        int, int64_t, int64_t, int64_t, int64_t, float, const mmdit_rope3d*, hipStream_t) {
  ++g_launches; return MMDIT_OK;
}
int launch_joint_attention(const void*, const void*, const void*, int64_t, const void*, const void*, const void*,
                           int64_t, int, int, int64_t, int64_t, int64_t, float, void*, void*, int, int64_t, float*,
                           hipStream_t, float*, size_t) { ++g_launches; return MMDIT_OK; }
size_t joint_attention_split_bytes(int64_t, int64_t, int64_t, int64_t, int, bool) { return 0; }
int launch_lite_regroup(int, const void*, const void*, const void*, int, void*, int, int, int64_t, int64_t, int64_t,
                        int64_t, int64_t, hipStream_t) { ++g_launches; return MMDIT_OK; }
int launch_linear(const GemmProblem*, int, int, int, int, int64_t, int64_t, int, int, hipStream_t, float*, size_t) {
  ++g_launches; return MMDIT_OK;
}
int launch_attn8_quantize(const void* const*, const void* const*, const void* const*, const int64_t*, int, int64_t,
                          int64_t, int64_t, const mmdit_attn8_stream* const*, float*, hipStream_t) {
  ++g_launches; return MMDIT_OK;
}
int launch_joint_attention_8bit(const mmdit_attn8_stream* const*, const int64_t*, const float*, int64_t, int64_t, float,
                                void*, void*, int, int64_t, float*, hipStream_t, float*, size_t) {
  ++g_launches; return MMDIT_OK;
}
int launch_quantize_fp8(const void*, int, int64_t, int64_t, int, uint8_t*, float*, hipStream_t) { ++g_launches; return MMDIT_OK; }
int launch_modulation(const void*, const void*, const void*, int, float*, int64_t, int64_t, int64_t, hipStream_t) {
  ++g_launches; return MMDIT_OK;
}
int launch_timestep_embed(const float*, int64_t, const void*, const void*, const void*, const void*, const void*,
                          const void*, int, int64_t, int64_t, int64_t, float, float*, float*, float*, hipStream_t) {
  ++g_launches; return MMDIT_OK;
}
int launch_convert_bf16_to_f16(const void*, void*, int64_t, hipStream_t) { ++g_launches; return MMDIT_OK; }
int launch_cast(const void*, int, void*, int, int64_t, hipStream_t) { ++g_launches; return MMDIT_OK; }
}  // namespace mmdit
