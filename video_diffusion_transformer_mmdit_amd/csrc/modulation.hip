// Per-(block, stream) modulation Linear: mod = W_mod tvec + b_mod, mapping the shared
// timestep bottleneck straight to six C-vectors (Vimoo 1.0 notes, sections 2.2 and 2.4).
//
// A GEMV over a [6C, Dt] bf16 matrix: bound by reading W_mod from HBM once (56.6 MB per
// stream at C = 3072, Dt = 1536; 0.59 MB with the 16-wide bottleneck of the Lite model,
// section 2.4).  The input vector is staged in LDS as f32; groups of lanes walk the rows
// in 16-byte loads and finish with a butterfly reduction.
// Also here: the timestep path that produces tvec (section 2.2) from the same GEMV, and the
// bf16 -> f16 copy used when the FFN runs on f16 operands.
#include "common.h"

namespace mmdit {

constexpr int MOD_THREADS = 256;
constexpr int MOD_MAX_T = 16384;  // floats of the input vectors staged in LDS (64 KiB)

// How the staged input vector is made from the kernel's `x` argument.
enum { GEMV_IN_PLAIN = 0,      // x[b, k] as stored (dtype TDT)
       GEMV_IN_SILU = 1,       // SiLU(x[b, k]), x f32
       GEMV_IN_SINUSOID = 2 }; // sinusoidal embedding of the timestep x[b] (f32), K entries

// y[b, r] = sum_k W[r, k] * in[b, k] + bias[r] for a [R, K] row-major matrix W of dtype
// WDT (bias the same dtype, or null).  Each group of LPR lanes owns ROWS rows and walks
// them in 16-byte chunks; LPR < 64 serves short rows (K / 8 < 64) without idle lanes.
// Consecutive row groups are consecutive in memory, so a wave reads one contiguous span.
template <int IN, int TDT, int WDT, int LPR, int ROWS>
__global__ __launch_bounds__(MOD_THREADS) void gemv_kernel(
    const void* __restrict__ w, const void* __restrict__ bias, const void* __restrict__ x,
    float* __restrict__ y, int B, int64_t R, int K, double log_max_period) {
  constexpr int GROUPS = 64 / LPR;
  extern __shared__ float tv[];   // B * K floats
  for (int i = threadIdx.x; i < B * K; i += MOD_THREADS) {
    float v;
    if constexpr (IN == GEMV_IN_PLAIN) {
      v = load1<TDT>(x, i);
    } else if constexpr (IN == GEMV_IN_SILU) {
      const float u = static_cast<const float*>(x)[i];
      v = u / (1.f + __expf(-u));
    } else {
      // Entry j < K/2: cos(t f_j); entry K/2 + j: sin(t f_j); f_j = max_period^(-j/(K/2)).
      // The angle reaches ~1e3 rad, so it is formed and reduced in double.
      const int b = i / K, j = i - b * K, half = K >> 1;
      const int jj = j < half ? j : j - half;
      const double ang = (double)static_cast<const float*>(x)[b] *
                         exp(-log_max_period * (double)jj / (double)half);
      v = (float)(j < half ? cos(ang) : sin(ang));
    }
    tv[i] = v;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int sub = lane / LPR, sl = lane % LPR;
  const int64_t row0 =
      (((int64_t)blockIdx.x * (MOD_THREADS / 64) + (threadIdx.x >> 6)) * GROUPS + sub) * ROWS;
  const int nch = K >> 3;
  for (int b = 0; b < B; ++b) {
    float acc[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[r] = 0.f;
    for (int ch = sl; ch < nch; ch += LPR) {
      float t8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t8[e] = tv[b * K + ch * 8 + e];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const int64_t row = row0 + r;
        if (row < R) {
          float w8[8];
          load8<WDT>(w, row * K + ch * 8, w8);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r] = fmaf(w8[e], t8[e], acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      const float s = group_sum<LPR>(acc[r]);
      const int64_t row = row0 + r;
      if (sl == 0 && row < R) y[b * R + row] = s + (bias ? load1<WDT>(bias, row) : 0.f);
    }
  }
}

template <int IN, int TDT, int WDT>
static int gemv_dispatch(const void* w, const void* bias, const void* x, float* y, int64_t B,
                         int64_t R, int64_t K, double log_max_period, hipStream_t stream) {
  const int64_t nch = K / 8;
  int lpr = 64;
  if (nch < 64) {
    lpr = 1;
    while (lpr * 2 <= nch) lpr *= 2;
  }
  // four rows per lane group while that still leaves two workgroups per CU, else one
  const int rows = (R / ((MOD_THREADS / 64) * (64 / lpr) * 4) >= 512) ? 4 : 1;
  const int64_t rows_per_block = (MOD_THREADS / 64) * (64 / lpr) * rows;
  const dim3 grid((unsigned)((R + rows_per_block - 1) / rows_per_block));
  // The input vectors of at most MOD_MAX_T / K batch items fit in LDS at once.
  const int64_t bmax = MOD_MAX_T / K;
  for (int64_t b0 = 0; b0 < B; b0 += bmax) {
    const int bn = (int)(B - b0 < bmax ? B - b0 : bmax);
    const void* xb;
    if constexpr (IN == GEMV_IN_SINUSOID) xb = static_cast<const float*>(x) + b0;
    else xb = static_cast<const char*>(x) + b0 * K * (TDT == MMDIT_F32 ? 4 : 2);
    float* yb = y + b0 * R;
    const size_t lds = (size_t)bn * K * sizeof(float);
#define GEMV_CASE(L)                                                                                       \
    case L:                                                                                                \
      if (rows == 4) gemv_kernel<IN, TDT, WDT, L, 4><<<grid, MOD_THREADS, lds, stream>>>(w, bias, xb, yb, bn, R, (int)K, log_max_period); \
      else gemv_kernel<IN, TDT, WDT, L, 1><<<grid, MOD_THREADS, lds, stream>>>(w, bias, xb, yb, bn, R, (int)K, log_max_period); \
      break;
    switch (lpr) {
      GEMV_CASE(1) GEMV_CASE(2) GEMV_CASE(4) GEMV_CASE(8) GEMV_CASE(16) GEMV_CASE(32) GEMV_CASE(64)
    }
#undef GEMV_CASE
    const int st = check_launch("gemv");
    if (st) return st;
  }
  return MMDIT_OK;
}

int launch_modulation(const void* w_mod, const void* b_mod, const void* tvec, int t_dtype,
                      float* mod, int64_t B, int64_t C6, int64_t Dt, hipStream_t stream) {
  if (B == 0 || C6 == 0) return MMDIT_OK;
  if (Dt > MOD_MAX_T) return fail(MMDIT_ERR_SHAPE, "modulation: Dt exceeds 16384");
  if (t_dtype == MMDIT_BF16)
    return gemv_dispatch<GEMV_IN_PLAIN, MMDIT_BF16, MMDIT_BF16>(w_mod, b_mod, tvec, mod, B, C6, Dt, 0.0, stream);
  if (t_dtype == MMDIT_F32)
    return gemv_dispatch<GEMV_IN_PLAIN, MMDIT_F32, MMDIT_BF16>(w_mod, b_mod, tvec, mod, B, C6, Dt, 0.0, stream);
  return fail(MMDIT_ERR_DTYPE, "modulation: tvec must be f32 or bf16");
}

// Timestep conditioning: hidden = W1 sinusoid(t) + b1; temb = W2 SiLU(hidden) + b2;
// tvec = W3 SiLU(temb) + b3.  Three dependent GEMVs (each needs all of the previous one's
// output), each bound by reading its weight matrix once.
int launch_timestep_embed(const float* t, int64_t B, const void* w1, const void* b1, const void* w2,
                          const void* b2, const void* w3, const void* b3, int w_dtype, int64_t freq_dim,
                          int64_t hidden_dim, int64_t Dt, float max_period, float* hidden, float* temb,
                          float* tvec, hipStream_t stream) {
  if (B == 0) return MMDIT_OK;
  const double lmp = log((double)max_period);
  int st;
  if (w_dtype == MMDIT_BF16) {
    if ((st = gemv_dispatch<GEMV_IN_SINUSOID, MMDIT_F32, MMDIT_BF16>(w1, b1, t, hidden, B, hidden_dim, freq_dim, lmp, stream))) return st;
    if ((st = gemv_dispatch<GEMV_IN_SILU, MMDIT_F32, MMDIT_BF16>(w2, b2, hidden, temb, B, hidden_dim, hidden_dim, 0.0, stream))) return st;
    return gemv_dispatch<GEMV_IN_SILU, MMDIT_F32, MMDIT_BF16>(w3, b3, temb, tvec, B, Dt, hidden_dim, 0.0, stream);
  }
  if ((st = gemv_dispatch<GEMV_IN_SINUSOID, MMDIT_F32, MMDIT_F32>(w1, b1, t, hidden, B, hidden_dim, freq_dim, lmp, stream))) return st;
  if ((st = gemv_dispatch<GEMV_IN_SILU, MMDIT_F32, MMDIT_F32>(w2, b2, hidden, temb, B, hidden_dim, hidden_dim, 0.0, stream))) return st;
  return gemv_dispatch<GEMV_IN_SILU, MMDIT_F32, MMDIT_F32>(w3, b3, temb, tvec, B, Dt, hidden_dim, 0.0, stream);
}

// Elementwise dtype change, 8 elements per thread with 16-byte accesses; the last n % 8
// elements one per thread of the last workgroup.  Rounding to 16 bits is to nearest even.
template <int IN, int OUT>
__global__ __launch_bounds__(256) void cast_kernel(const void* __restrict__ src, void* __restrict__ dst,
                                                   int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n8 = n / 8;
  if (i < n8) {
    float v[8];
    load8<IN>(src, i * 8, v);
    store8<OUT>(dst, i * 8, v);
  } else if (i - n8 < n % 8) {
    const int64_t e = n8 * 8 + (i - n8);
    store1<OUT>(dst, e, load1<IN>(src, e));
  }
}

template <int IN, int OUT>
static int cast_go(const void* src, void* dst, int64_t n, hipStream_t stream) {
  const int64_t threads = n / 8 + n % 8;
  if (threads == 0) return MMDIT_OK;
  cast_kernel<IN, OUT><<<dim3((unsigned)((threads + 255) / 256)), 256, 0, stream>>>(src, dst, n);
  return check_launch("cast");
}

int launch_cast(const void* src, int src_dtype, void* dst, int dst_dtype, int64_t n, hipStream_t stream) {
#define MMDIT_CAST(I, O) if (src_dtype == I && dst_dtype == O) return cast_go<I, O>(src, dst, n, stream)
  MMDIT_CAST(MMDIT_BF16, MMDIT_F16); MMDIT_CAST(MMDIT_F16, MMDIT_BF16);
  MMDIT_CAST(MMDIT_BF16, MMDIT_F32); MMDIT_CAST(MMDIT_F16, MMDIT_F32);
  MMDIT_CAST(MMDIT_F32, MMDIT_BF16); MMDIT_CAST(MMDIT_F32, MMDIT_F16);
#undef MMDIT_CAST
  return fail(MMDIT_ERR_DTYPE, "cast: unsupported dtype pair");
}

int launch_convert_bf16_to_f16(const void* src, void* dst, int64_t n, hipStream_t stream) {
  return cast_go<MMDIT_BF16, MMDIT_F16>(src, dst, n, stream);
}

}  // namespace mmdit
