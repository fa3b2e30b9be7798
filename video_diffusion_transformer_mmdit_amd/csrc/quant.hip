// FP8 E4M3 quantization of activations (one scale per token row) and of weights (one scale
// per tensor), the scaling the Wan report uses for its FP8 GEMMs (section 4.4.3).
//
//   s = amax / 448 (f32; an all-zero group takes s = 1),  code = E4M3(clamp(x * (1/s), +-448))
//
// with round-to-nearest-even in the hardware conversion (v_cvt_pk_fp8_f32).  Bound by HBM:
// per row one read of x and one write of the codes.  Rows go to one wave each, 8 elements
// per lane per step; rows of 3072 or 12288 16-bit values stay in registers between the amax
// and the coding pass, other rows are read a second time (from cache when still there).
#include "common.h"

namespace mmdit {

constexpr float FP8_MAX = 448.f;

__device__ __forceinline__ float fp8_scale(float amax) { return amax > 0.f ? amax / FP8_MAX : 1.f; }

// Four floats (already within +-448) to four E4M3 codes, first value in the low byte.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float clamp_fp8(float v) { return fminf(fmaxf(v, -FP8_MAX), FP8_MAX); }

// codes of eight values at q[idx .. idx + 7]
__device__ __forceinline__ void store_codes8(float (&v)[8], float inv, uint8_t* q, int64_t idx) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = clamp_fp8(v[e] * inv);
  *reinterpret_cast<uint2*>(q + idx) = make_uint2(pack_fp8x4(v[0], v[1], v[2], v[3]), pack_fp8x4(v[4], v[5], v[6], v[7]));
}

template <int DT>
__device__ __forceinline__ void quant8(const void* x, int64_t idx, float inv, uint8_t* q) {
  float v[8];
  load8<DT>(x, idx, v);
  store_codes8(v, inv, q, idx);
}

// Eight 16-bit values of one 16-byte chunk as floats (as load8 widens them).
template <int DT>
__device__ __forceinline__ void widen8(const uint4& w, float (&v)[8]) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (DT == MMDIT_BF16) { v[2 * i] = lo_bf16(ws[i]); v[2 * i + 1] = hi_bf16(ws[i]); }
    else { v[2 * i] = lo_f16(ws[i]); v[2 * i + 1] = hi_f16(ws[i]); }
  }
}

// Per-row quantization of 16-bit rows of 512 * CPL values: each lane keeps its CPL chunks in
// registers between the amax and the coding pass, so the row crosses HBM once (the generic
// kernel below re-reads it, from cache when it is still there).
template <int DT, int CPL>
__global__ __launch_bounds__(256) void quant_rows_reg_kernel(const void* __restrict__ x, int64_t rows,
                                                             uint8_t* __restrict__ q, float* __restrict__ scales) {
  constexpr int COLS = 512 * CPL;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t base = row * COLS;
  uint4 raw[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i)
    raw[i] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + base + (lane + 64 * i) * 8);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    float v[8];
    widen8<DT>(raw[i], v);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float s = fp8_scale(amax);
  const float inv = 1.f / s;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    float v[8];
    widen8<DT>(raw[i], v);
    store_codes8(v, inv, q, base + (lane + 64 * i) * 8);
  }
  if (lane == 0) scales[row] = s;
}

template <int DT>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ x, int64_t rows, int cols,
                                                         uint8_t* __restrict__ q, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nch = cols >> 3;
  const int64_t base = row * cols;
  float amax = 0.f;
  for (int ch = lane; ch < nch; ch += 64) {
    float v[8];
    load8<DT>(x, base + ch * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float s = fp8_scale(amax);
  const float inv = 1.f / s;
  for (int ch = lane; ch < nch; ch += 64) quant8<DT>(x, base + ch * 8, inv, q);
  if (lane == 0) scales[row] = s;
}

__global__ void zero1_kernel(float* p) { *p = 0.f; }

// amax over the whole tensor into *amax (float bits; non-negative floats order as unsigned)
template <int DT>
__global__ __launch_bounds__(256) void amax_kernel(const void* __restrict__ x, int64_t n8, float* __restrict__ amax) {
  __shared__ float red[4];
  float m = 0.f;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n8; c += (int64_t)gridDim.x * 256) {
    float v[8];
    load8<DT>(x, c * 8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(m));
  }
}

template <int DT>
__global__ __launch_bounds__(256) void quant_tensor_kernel(const void* __restrict__ x, int64_t n8,
                                                           const float* __restrict__ amax, uint8_t* __restrict__ q) {
  const float inv = 1.f / fp8_scale(*amax);
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < n8; c += (int64_t)gridDim.x * 256)
    quant8<DT>(x, c * 8, inv, q);
}

__global__ void amax_to_scale_kernel(float* p) { *p = fp8_scale(*p); }

template <int DT>
static int quant_go(const void* x, int64_t rows, int64_t cols, int per_row, uint8_t* q, float* scales,
                    hipStream_t stream) {
  if (per_row) {
    const dim3 grid((unsigned)((rows + 3) / 4));
    if constexpr (DT != MMDIT_F32) {
      if (cols == 512 * 6) {
        quant_rows_reg_kernel<DT, 6><<<grid, 256, 0, stream>>>(x, rows, q, scales);
        return check_launch("quantize_fp8 rows");
      }
      if (cols == 512 * 24) {
        quant_rows_reg_kernel<DT, 24><<<grid, 256, 0, stream>>>(x, rows, q, scales);
        return check_launch("quantize_fp8 rows");
      }
    }
    quant_rows_kernel<DT><<<grid, 256, 0, stream>>>(x, rows, (int)cols, q, scales);
    return check_launch("quantize_fp8 rows");
  }
  const int64_t n8 = rows * cols / 8;
  const unsigned blocks = (unsigned)(n8 / 256 + 1 < 2048 ? n8 / 256 + 1 : 2048);
  zero1_kernel<<<1, 1, 0, stream>>>(scales);
  amax_kernel<DT><<<blocks, 256, 0, stream>>>(x, n8, scales);
  quant_tensor_kernel<DT><<<blocks, 256, 0, stream>>>(x, n8, scales, q);
  amax_to_scale_kernel<<<1, 1, 0, stream>>>(scales);
  return check_launch("quantize_fp8 tensor");
}

int launch_quantize_fp8(const void* x, int x_dtype, int64_t rows, int64_t cols, int per_row, uint8_t* q,
                        float* scales, hipStream_t stream) {
  if (rows == 0) return MMDIT_OK;
  if (x_dtype == MMDIT_F32) return quant_go<MMDIT_F32>(x, rows, cols, per_row, q, scales, stream);
  if (x_dtype == MMDIT_BF16) return quant_go<MMDIT_BF16>(x, rows, cols, per_row, q, scales, stream);
  return quant_go<MMDIT_F16>(x, rows, cols, per_row, q, scales, stream);
}

}  // namespace mmdit
