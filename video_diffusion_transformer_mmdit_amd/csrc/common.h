// Shared helpers of the gfx950 MMDiT kernels: 16-bit conversions, vector types, error
// plumbing.  Device code is written for CDNA4 wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <initializer_list>
#include <string>

#include "../../include/mmdit.h"

namespace mmdit {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Unpack the two bf16 halves of a 32-bit word.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return f32_to_f16_bits(a) | (f32_to_f16_bits(b) << 16);
}
// Range guard for the f16 intermediates (GEMM outputs, LN-modulated activations): a value
// beyond the f16 range saturates at +-65504 instead of rounding to infinity, which would turn
// into NaN downstream (LayerNorm, attention); NaN stays NaN.
__device__ __forceinline__ float sat_f16(float v) { return fabsf(v) > 65504.0f ? copysignf(65504.0f, v) : v; }
__device__ __forceinline__ float lo_f16(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hi_f16(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Load 8 consecutive elements of dtype DT (0 f32, 1 bf16, 2 f16) as floats.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&v)[8]) {
  if constexpr (DT == MMDIT_F32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == MMDIT_BF16) { v[2 * i] = lo_bf16(ws[i]); v[2 * i + 1] = hi_bf16(ws[i]); }
      else { v[2 * i] = lo_f16(ws[i]); v[2 * i + 1] = hi_f16(ws[i]); }
    }
  }
}

// Store 8 consecutive floats as dtype DT.
template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t idx, const float (&v)[8]) {
  if constexpr (DT == MMDIT_F32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + idx);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 w;
    if constexpr (DT == MMDIT_BF16) {
      w.x = pack_bf16x2(v[0], v[1]); w.y = pack_bf16x2(v[2], v[3]);
      w.z = pack_bf16x2(v[4], v[5]); w.w = pack_bf16x2(v[6], v[7]);
    } else {
      w.x = pack_f16x2(v[0], v[1]); w.y = pack_f16x2(v[2], v[3]);
      w.z = pack_f16x2(v[4], v[5]); w.w = pack_f16x2(v[6], v[7]);
    }
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx) = w;
  }
}

template <int DT>
__device__ __forceinline__ float load1(const void* base, int64_t idx) {
  if constexpr (DT == MMDIT_F32) return static_cast<const float*>(base)[idx];
  else if constexpr (DT == MMDIT_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  else return (float)static_cast<const _Float16*>(base)[idx];
}

template <int DT>
__device__ __forceinline__ void store1(void* base, int64_t idx, float v) {
  if constexpr (DT == MMDIT_F32) static_cast<float*>(base)[idx] = v;
  else if constexpr (DT == MMDIT_BF16) static_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_bf16_bits(v);
  else static_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_f16_bits(v);
}

// Sum over groups of `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
  return v;
}

// ------------------------------------------------------------------ host-side errors
void set_error(const std::string& msg);
int fail(int status, const std::string& msg);
int check_launch(const char* what);

inline int dtype_size(int dt) { return dt == MMDIT_F32 ? 4 : dt == MMDIT_FP8_E4M3 ? 1 : 2; }

// Compute units of the current device (queried once per device; 256 on MI355X).  The split-tail
// heuristics size a launch's last round by it: one persistent-size workgroup per CU.
int device_cu_count();
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Size guard of the argument validators: every extent lies in [0, 2^31) and their product
// (a zero extent counting as one) stays below 2^40, so that the validators' byte-span
// arithmetic on such products cannot overflow int64.
inline bool extents_ok(std::initializer_list<int64_t> xs) {
  int64_t p = 1;
  for (const int64_t x : xs) {
    if (x < 0 || x >= ((int64_t)1 << 31)) return false;
    if (__builtin_mul_overflow(p, x > 0 ? x : (int64_t)1, &p) || p >= ((int64_t)1 << 40)) return false;
  }
  return true;
}

// Internal launchers (validated arguments only).
int launch_modulate_ln(const void* x, int x_dtype, const void* branch, int branch_dtype,
                       const float* gate, float* x_out, const float* shift, const float* scale,
                       int64_t mod_stride, void* y, int y_dtype, int64_t B, int64_t N, int64_t C,
                       float eps, hipStream_t stream);
int launch_qk_norm_rope(const void* q, const void* k, int in_dtype, int64_t in_stride,
                        const void* q_scale, const void* k_scale, int scale_dtype,
                        int64_t scale_head_stride, void* q_out, void* k_out, int out_dtype,
                        int64_t out_stride, int64_t B, int64_t N, int64_t H, float eps,
                        const mmdit_rope3d* rope, hipStream_t stream);
int launch_joint_attention(const void* q_vis, const void* k_vis, const void* v_vis, int64_t n_vis,
                           const void* q_cond, const void* k_cond, const void* v_cond,
                           int64_t n_cond, int qk_dtype, int v_dtype, int64_t in_stride, int64_t B, int64_t H,
                           float softmax_scale, void* o_vis, void* o_cond, int out_dtype,
                           int64_t out_stride, float* lse, hipStream_t stream, float* split_ws = nullptr,
                           size_t split_ws_bytes = 0);

// Bytes of key-range results the attention's split tail uses with an unlimited workspace (0:
// the call does not split).
size_t joint_attention_split_bytes(int64_t n_vis, int64_t n_cond, int64_t B, int64_t H, int qk_dtype, bool has_lse);

struct GemmProblem {
  const void* x;      // [M, K]
  const void* w;      // [N, K]
  const void* bias;   // [N] or null
  void* y;            // [M, N]
  const void* res;    // [M, N] (gated residual) or null
  const float* gate;  // [B, N] slices (gated residual) or null
  int64_t M;
  int64_t gate_stride;
  int64_t rows_per_batch;
  const float* x_scale;  // FP8 operands: [M] per-row scale of x
  const float* w_scale;  // FP8 operands: [1] scale of all of W
};
// Operand layouts of the GEMM kernel: plain row-major x and y, or the Lite 2x2 regrouping.
enum { GEMM_PLAIN = 0, GEMM_GATHER_X = 1, GEMM_SCATTER_Y = 2 };
int launch_lite_regroup(int layout, const void* x, const void* w, const void* bias, int bias_dtype, void* y,
                        int in_dtype, int y_dtype, int64_t B, int64_t T, int64_t H, int64_t W, int64_t C,
                        hipStream_t stream);
// Runs one or two problems with equal N, K, dtypes and epilogue in one launch.
// split_ws (optional, split_ws_bytes long): f32 scratch for the split tail (up to 64 MiB).
int launch_linear(const GemmProblem* probs, int nprobs, int x_dtype, int bias_dtype, int y_dtype,
                  int64_t N, int64_t K, int epilogue, int res_dtype, hipStream_t stream,
                  float* split_ws = nullptr, size_t split_ws_bytes = 0);
int launch_attn8_quantize(const void* const* q, const void* const* k, const void* const* v, const int64_t* n,
                          int in_dtype, int64_t stride, int64_t B, int64_t H, const mmdit_attn8_stream* const* out,
                          float* v_scale, hipStream_t stream);
int launch_joint_attention_8bit(const mmdit_attn8_stream* const* seg, const int64_t* n, const float* v_scale,
                                int64_t B, int64_t H, float softmax_scale, void* o_vis, void* o_cond, int out_dtype,
                                int64_t out_stride, float* lse, hipStream_t stream, float* split_ws = nullptr,
                                size_t split_ws_bytes = 0);
// FP8 E4M3 quantization with a scale per row (per_row) or one for the whole tensor.
int launch_quantize_fp8(const void* x, int x_dtype, int64_t rows, int64_t cols, int per_row, uint8_t* q,
                        float* scales, hipStream_t stream);
int launch_modulation(const void* w_mod, const void* b_mod, const void* tvec, int t_dtype,
                      float* mod, int64_t B, int64_t C6, int64_t Dt, hipStream_t stream);
int launch_timestep_embed(const float* t, int64_t B, const void* w1, const void* b1, const void* w2,
                          const void* b2, const void* w3, const void* b3, int w_dtype, int64_t freq_dim,
                          int64_t hidden_dim, int64_t Dt, float max_period, float* hidden, float* temb,
                          float* tvec, hipStream_t stream);
int launch_convert_bf16_to_f16(const void* src, void* dst, int64_t n, hipStream_t stream);
int launch_cast(const void* src, int src_dtype, void* dst, int dst_dtype, int64_t n, hipStream_t stream);

}  // namespace mmdit
