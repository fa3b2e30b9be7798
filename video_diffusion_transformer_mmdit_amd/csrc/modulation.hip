// Per-(block, stream) modulation Linear: mod = W_mod tvec + b_mod, mapping the shared
// timestep bottleneck straight to six C-vectors (Vimoo 1.0 notes, sections 2.2 and 2.4).
//
// A GEMV over a [6C, Dt] bf16 matrix: bound by reading W_mod from HBM once (56.6 MB per
// stream at C = 3072, Dt = 1536).  tvec is staged in LDS as f32; one wave64 computes
// ROWS_PER_WAVE output rows with 16-byte loads along each row and a butterfly reduction.
// Also here: the bf16 -> f16 copy used when the FFN runs on f16 operands.
#include "common.h"

namespace mmdit {

constexpr int MOD_THREADS = 256;
constexpr int MOD_ROWS_PER_WAVE = 4;
constexpr int MOD_MAX_T = 16384;  // B * Dt floats staged in LDS (64 KiB)

template <int TDT>
__global__ __launch_bounds__(MOD_THREADS) void modulation_kernel(
    const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias, const void* __restrict__ tvec,
    float* __restrict__ mod, int B, int64_t R, int Dt) {
  __shared__ float tv[MOD_MAX_T];
  for (int i = threadIdx.x; i < B * Dt; i += MOD_THREADS) tv[i] = load1<TDT>(tvec, i);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int64_t row0 = ((int64_t)blockIdx.x * (MOD_THREADS / 64) + (threadIdx.x >> 6)) * MOD_ROWS_PER_WAVE;
  const int nch = Dt >> 3;
  for (int b = 0; b < B; ++b) {
    float acc[MOD_ROWS_PER_WAVE];
#pragma unroll
    for (int r = 0; r < MOD_ROWS_PER_WAVE; ++r) acc[r] = 0.f;
    for (int ch = lane; ch < nch; ch += 64) {
      float t8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t8[e] = tv[b * Dt + ch * 8 + e];
#pragma unroll
      for (int r = 0; r < MOD_ROWS_PER_WAVE; ++r) {
        const int64_t row = row0 + r;
        if (row < R) {
          float w8[8];
          load8<MMDIT_BF16>(w, row * Dt + ch * 8, w8);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r] = fmaf(w8[e], t8[e], acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < MOD_ROWS_PER_WAVE; ++r) {
      const float s = group_sum<64>(acc[r]);
      const int64_t row = row0 + r;
      if (lane == 0 && row < R) mod[b * R + row] = s + (bias ? bf16_bits_to_f32(bias[row]) : 0.f);
    }
  }
}

int launch_modulation(const void* w_mod, const void* b_mod, const void* tvec, int t_dtype,
                      float* mod, int64_t B, int64_t C6, int64_t Dt, hipStream_t stream) {
  if (B == 0 || C6 == 0) return MMDIT_OK;
  if (B * Dt > MOD_MAX_T) return fail(MMDIT_ERR_SHAPE, "modulation: B * Dt exceeds 16384");
  const int64_t rows_per_block = (MOD_THREADS / 64) * MOD_ROWS_PER_WAVE;
  const dim3 grid((unsigned)((C6 + rows_per_block - 1) / rows_per_block));
  const uint16_t* w = static_cast<const uint16_t*>(w_mod);
  const uint16_t* b = static_cast<const uint16_t*>(b_mod);
  if (t_dtype == MMDIT_BF16)
    modulation_kernel<MMDIT_BF16><<<grid, MOD_THREADS, 0, stream>>>(w, b, tvec, mod, (int)B, C6, (int)Dt);
  else if (t_dtype == MMDIT_F32)
    modulation_kernel<MMDIT_F32><<<grid, MOD_THREADS, 0, stream>>>(w, b, tvec, mod, (int)B, C6, (int)Dt);
  else
    return fail(MMDIT_ERR_DTYPE, "modulation: tvec must be f32 or bf16");
  return check_launch("modulation");
}

// bf16 -> f16, 8 elements per thread (n a multiple of 8).
__global__ __launch_bounds__(256) void convert_bf16_f16_kernel(const uint16_t* __restrict__ src,
                                                               uint16_t* __restrict__ dst, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float v[8];
  load8<MMDIT_BF16>(src, i * 8, v);
  store8<MMDIT_F16>(dst, i * 8, v);
}

int launch_convert_bf16_to_f16(const void* src, void* dst, int64_t n, hipStream_t stream) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return MMDIT_OK;
  convert_bf16_f16_kernel<<<dim3((unsigned)((n8 + 255) / 256)), 256, 0, stream>>>(
      static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), n8);
  return check_launch("convert_bf16_f16");
}

}  // namespace mmdit
