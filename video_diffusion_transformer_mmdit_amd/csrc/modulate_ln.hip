// LayerNorm with timestep shift/scale, optionally after a gated residual.
//
// Vimoo 1.0 notes, section 2.2: LayerNorm precedes the attention and FFN transforms, with
// shift and scale supplied by the timestep modulation, and gates weighting each branch's
// residual update.  Here  x' = x + gate * branch  (optional),  y = LN(x') (1 + scale) + shift.
//
// One wave64 owns one token row: the row (C <= 8192) lives in registers, each lane holding
// CPL chunks of 8 channels loaded as 16-byte vectors, so the row is read from HBM exactly
// once and the mean / variance are two in-register passes plus wave butterflies.
#include "common.h"

namespace mmdit {

constexpr int MLN_THREADS = 256;  // 4 rows per block

template <int WIDTH>
__device__ __forceinline__ float wave_sum(float v) { return group_sum<WIDTH>(v); }

template <int XDT, int BDT, int YDT, int CPL, bool BRANCH, bool XOUT>
__global__ __launch_bounds__(MLN_THREADS) void modulate_ln_kernel(
    const void* __restrict__ x, const void* __restrict__ branch, const float* __restrict__ gate,
    float* __restrict__ x_out, const float* __restrict__ shift, const float* __restrict__ scale,
    int64_t mod_stride, void* __restrict__ y, int64_t rows, int64_t n_per_batch, int C, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (MLN_THREADS / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t b = row / n_per_batch;
  const int nchunks = C >> 3;
  const int64_t base = row * C;
  const float* sh = shift + b * mod_stride;
  const float* sc = scale + b * mod_stride;

  // Every chunk load is issued before any is used: a load under a bounds branch waited for its
  // data before the branch closed, so the row's loads went out one at a time.  Chunks past the
  // row's end load its last chunk and are then zeroed.
  float v[CPL][8];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int ch = lane + 64 * i;
    load8<XDT>(x, base + (ch < nchunks ? ch : nchunks - 1) * 8, v[i]);
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nchunks) {
      if constexpr (BRANCH) {
        float br[8], gt[8];
        load8<BDT>(branch, base + ch * 8, br);
        load8<MMDIT_F32>(gate + b * mod_stride, ch * 8, gt);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] = fmaf(gt[e], br[e], v[i][e]);
      }
      if constexpr (XOUT) store8<MMDIT_F32>(x_out, base + ch * 8, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += v[i][e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    }
  }
  const float mean = wave_sum<64>(sum) / (float)C;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    if (lane + 64 * i < nchunks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[i][e] - mean;
        sq = fmaf(d, d, sq);
      }
    }
  }
  const float rstd = rsqrtf(wave_sum<64>(sq) / (float)C + eps);
  // shift and scale of chunk i + 1 are loaded while chunk i is finished and stored
  auto mod_load = [&](int i, float (&s8)[8], float (&c8)[8]) {
    const int ch = lane + 64 * i;
    const int chc = ch < nchunks ? ch : nchunks - 1;
    load8<MMDIT_F32>(sh, chc * 8, s8);
    load8<MMDIT_F32>(sc, chc * 8, c8);
  };
  float s8n[8], c8n[8];
  mod_load(0, s8n, c8n);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int ch = lane + 64 * i;
    float s8[8], c8[8], o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { s8[e] = s8n[e]; c8[e] = c8n[e]; }
    if (i + 1 < CPL) mod_load(i + 1, s8n, c8n);
    if (ch < nchunks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] = fmaf((v[i][e] - mean) * rstd, 1.0f + c8[e], s8[e]);
        if constexpr (YDT == MMDIT_F16) o[e] = sat_f16(o[e]);
      }
      store8<YDT>(y, base + ch * 8, o);
    }
  }
}

template <int XDT, int BDT, int YDT, int CPL>
static void mln_dispatch_flags(bool br, bool xo, dim3 grid, hipStream_t st, const void* x,
                               const void* branch, const float* gate, float* x_out,
                               const float* shift, const float* scale, int64_t ms, void* y,
                               int64_t rows, int64_t n, int C, float eps) {
#define MLN_GO(B_, X_)                                                                        \
  modulate_ln_kernel<XDT, BDT, YDT, CPL, B_, X_><<<grid, MLN_THREADS, 0, st>>>(                \
      x, branch, gate, x_out, shift, scale, ms, y, rows, n, C, eps)
  if (br && xo) MLN_GO(true, true);
  else if (br) MLN_GO(true, false);
  else if (xo) MLN_GO(false, true);
  else MLN_GO(false, false);
#undef MLN_GO
}

template <int XDT, int BDT, int YDT>
static void mln_dispatch_cpl(int cpl, bool br, bool xo, dim3 grid, hipStream_t st,
                             const void* x, const void* branch, const float* gate, float* x_out,
                             const float* shift, const float* scale, int64_t ms, void* y,
                             int64_t rows, int64_t n, int C, float eps) {
#define MLN_CPL(K)                                                                             \
  if (cpl <= K) {                                                                              \
    mln_dispatch_flags<XDT, BDT, YDT, K>(br, xo, grid, st, x, branch, gate, x_out, shift, scale, \
                                         ms, y, rows, n, C, eps);                              \
    return;                                                                                    \
  }
  MLN_CPL(1) MLN_CPL(2) MLN_CPL(4) MLN_CPL(6) MLN_CPL(8) MLN_CPL(12) MLN_CPL(16)
#undef MLN_CPL
}

int launch_modulate_ln(const void* x, int x_dtype, const void* branch, int branch_dtype,
                       const float* gate, float* x_out, const float* shift, const float* scale,
                       int64_t mod_stride, void* y, int y_dtype, int64_t B, int64_t N, int64_t C,
                       float eps, hipStream_t stream) {
  const int64_t rows = B * N;
  if (rows == 0) return MMDIT_OK;
  const int cpl = (int)((C / 8 + 63) / 64);
  const dim3 grid((unsigned)((rows + 3) / 4));
  const bool br = branch != nullptr, xo = x_out != nullptr;
  const int bdt = br ? branch_dtype : MMDIT_BF16;
  const int c = (int)C;
#define MLN_CASE(X, BD, Y)                                                                   \
  if (x_dtype == X && bdt == BD && y_dtype == Y) {                                           \
    mln_dispatch_cpl<X, BD, Y>(cpl, br, xo, grid, stream, x, branch, gate, x_out, shift,     \
                               scale, mod_stride, y, rows, N, c, eps);                       \
    return check_launch("modulate_ln");                                                      \
  }
  MLN_CASE(MMDIT_BF16, MMDIT_BF16, MMDIT_BF16)
  MLN_CASE(MMDIT_BF16, MMDIT_BF16, MMDIT_F16)
  MLN_CASE(MMDIT_BF16, MMDIT_BF16, MMDIT_F32)
  MLN_CASE(MMDIT_BF16, MMDIT_F32, MMDIT_BF16)
  MLN_CASE(MMDIT_BF16, MMDIT_F32, MMDIT_F16)
  MLN_CASE(MMDIT_F32, MMDIT_BF16, MMDIT_BF16)
  MLN_CASE(MMDIT_F32, MMDIT_BF16, MMDIT_F16)
  MLN_CASE(MMDIT_F32, MMDIT_BF16, MMDIT_F32)
  MLN_CASE(MMDIT_F32, MMDIT_F32, MMDIT_BF16)
  MLN_CASE(MMDIT_F32, MMDIT_F32, MMDIT_F16)
  MLN_CASE(MMDIT_F32, MMDIT_F32, MMDIT_F32)
#undef MLN_CASE
  return fail(MMDIT_ERR_DTYPE, "modulate_ln: unsupported dtype combination");
}

}  // namespace mmdit
