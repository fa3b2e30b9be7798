// y = epilogue(x W^T + bias): the per-stream projections of the MMDiT block (QKV, output,
// FFN up with GELU, FFN down with the gated residual), Vimoo 1.0 notes section 2.2; their
// cost is the linear term of the Wan report's workload model (section 4.3.1).
//
// gfx950 design:
//   - 256 x 256 output tile per workgroup of 8 wave64s arranged 2 (M) x 4 (N); each wave
//     owns 128 x 64 = 4 x 2 tiles of v_mfma_f32_32x32x16_{bf16,f16} (128 fp32 accumulators).
//   - K advances 64 at a time through two LDS stages of 2 x 32 KiB (A rows and W rows,
//     both K-contiguous, so both MFMA operands are plain 16-byte LDS reads).  The next
//     stage's global loads are issued before the current stage's MFMAs and written to the
//     other LDS buffer afterwards: one barrier per K step.
//   - LDS rows are 128 B; the 16-byte chunk index is XOR-swizzled with (row / 2) % 8 so the
//     32-row fragment reads and the row-wise stores both spread over all 64 banks.
//   - Tiles are renumbered so that each XCD (workgroups go round-robin over the 8 XCDs) owns
//     a contiguous run of tiles, and runs are rastered in groups of 8 M-tiles, keeping the
//     A and W panels that concurrent workgroups of one XCD share inside its L2.
//   - Epilogues are applied on the accumulators before the only store of y.
#include "common.h"

namespace mmdit {

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int GTHREADS = 512;
constexpr int GROUP_M = 8;
constexpr int G_LDS_STAGE = (GBM + GBN) * GBK * 2;  // bytes per stage (64 KiB)

struct GemmArgs {
  GemmProblem p[2];
  int64_t tiles0;    // tiles of problem 0
  int64_t tiles;     // total tiles
  int64_t N, K;
};

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

template <int IN_DT>
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  if constexpr (IN_DT == MMDIT_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erff(v * 0.70710678118654752440f));
}

template <int IN_DT, int BIAS_DT, int Y_DT, int EPI, int RES_DT>
__global__ __launch_bounds__(GTHREADS) void gemm_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * G_LDS_STAGE];

  // ---- tile selection: XCD-contiguous runs, grouped raster inside a problem
  int64_t t = blockIdx.x;
  if ((args.tiles & 7) == 0) t = (t & 7) * (args.tiles >> 3) + (t >> 3);
  const int pi = t < args.tiles0 ? 0 : 1;
  if (pi) t -= args.tiles0;
  const GemmProblem& P = args.p[pi];
  const int64_t M = P.M, N = args.N, K = args.K;
  const int64_t nTm = (M + GBM - 1) / GBM, nTn = (N + GBN - 1) / GBN;
  const int64_t per_group = (int64_t)GROUP_M * nTn;
  const int64_t grp = t / per_group;
  const int64_t first_m = grp * GROUP_M;
  const int64_t gm = (nTm - first_m) < GROUP_M ? (nTm - first_m) : GROUP_M;
  const int64_t in_grp = t - grp * per_group;
  const int64_t tm = first_m + in_grp % gm;
  const int64_t tn = in_grp / gm;
  const int64_t m0 = tm * GBM, n0 = tn * GBN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;

  const uint16_t* X = static_cast<const uint16_t*>(P.x);
  const uint16_t* W = static_cast<const uint16_t*>(P.w);

  // ---- global -> register staging: 4 A chunks + 4 W chunks of 16 B per thread
  uint4 ra[4], rb[4];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + GTHREADS * i;
      const int r = ch >> 3, cc = ch & 7;
      const int64_t am = m0 + r, bn = n0 + r;
      ra[i] = am < M ? *reinterpret_cast<const uint4*>(X + am * K + k0 + cc * 8) : make_uint4(0, 0, 0, 0);
      rb[i] = bn < N ? *reinterpret_cast<const uint4*>(W + bn * K + k0 + cc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* sa = lds + buf * G_LDS_STAGE;
    uint8_t* sb = sa + GBM * GBK * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + GTHREADS * i;
      const int r = ch >> 3, cc = ch & 7;
      const int off = r * 128 + ((cc ^ swz(r)) << 4);
      *reinterpret_cast<uint4*>(sa + off) = ra[i];
      *reinterpret_cast<uint4*>(sb + off) = rb[i];
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = (int)(K / GBK);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((int64_t)(kt + 1) * GBK);
    const uint8_t* sa = lds + buf * G_LDS_STAGE;
    const uint8_t* sb = sa + GBM * GBK * 2;
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      uint4 af[4], bfr[2];
      const int chunk = 2 * ks + g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + i * 32 + l32;
        af[i] = *reinterpret_cast<const uint4*>(sa + r * 128 + ((chunk ^ swz(r)) << 4));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + l32;
        bfr[j] = *reinterpret_cast<const uint4*>(sb + r * 128 + ((chunk ^ swz(r)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32<IN_DT>(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 8*(e/4) + 4*g + e%4 of each 32 x 32 tile, column l32
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + wn * 64 + j * 32 + l32;
    if (n >= N) continue;
    const float bias = P.bias ? load1<BIAS_DT>(P.bias, n) : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
        if (m >= M) continue;
        float v = acc[i][j][e] + bias;
        if constexpr (EPI == MMDIT_EPI_GELU) v = gelu_erf(v);
        if constexpr (EPI == MMDIT_EPI_GATED_RES) {
          const int64_t b = m / P.rows_per_batch;
          v = load1<RES_DT>(P.res, m * N + n) + P.gate[b * P.gate_stride + n] * v;
        }
        store1<Y_DT>(P.y, m * N + n, v);
      }
    }
  }
}

template <int IN_DT, int BIAS_DT, int Y_DT, int EPI, int RES_DT>
static void gemm_go(const GemmArgs& a, hipStream_t st) {
  gemm_kernel<IN_DT, BIAS_DT, Y_DT, EPI, RES_DT><<<dim3((unsigned)a.tiles), GTHREADS, 0, st>>>(a);
}

int launch_linear(const GemmProblem* probs, int nprobs, int x_dtype, int bias_dtype, int y_dtype,
                  int64_t N, int64_t K, int epilogue, int res_dtype, hipStream_t stream) {
  GemmArgs a{};
  const int64_t nTn = (N + GBN - 1) / GBN;
  int64_t tiles[2] = {0, 0};
  for (int i = 0; i < nprobs; ++i) {
    a.p[i] = probs[i];
    tiles[i] = ((probs[i].M + GBM - 1) / GBM) * nTn;
  }
  a.tiles0 = tiles[0];
  a.tiles = tiles[0] + tiles[1];
  a.N = N;
  a.K = K;
  if (a.tiles == 0) return MMDIT_OK;
  if (a.tiles > 0x7fffffff) return fail(MMDIT_ERR_SHAPE, "linear: too many tiles");
  const int bdt = bias_dtype == MMDIT_F32 ? MMDIT_F32 : MMDIT_BF16;
#define GEMM_CASE(IN, Y, EPI, RES)                                                            \
  if (x_dtype == IN && y_dtype == Y && epilogue == EPI && (EPI != MMDIT_EPI_GATED_RES || res_dtype == RES)) { \
    if (bdt == MMDIT_F32) gemm_go<IN, MMDIT_F32, Y, EPI, RES>(a, stream);                      \
    else gemm_go<IN, MMDIT_BF16, Y, EPI, RES>(a, stream);                                      \
    return check_launch("linear");                                                            \
  }
#define GEMM_IN(IN)                                                                           \
  GEMM_CASE(IN, MMDIT_BF16, MMDIT_EPI_NONE, MMDIT_F32)                                        \
  GEMM_CASE(IN, MMDIT_F16, MMDIT_EPI_NONE, MMDIT_F32)                                         \
  GEMM_CASE(IN, MMDIT_F32, MMDIT_EPI_NONE, MMDIT_F32)                                         \
  GEMM_CASE(IN, MMDIT_BF16, MMDIT_EPI_GELU, MMDIT_F32)                                        \
  GEMM_CASE(IN, MMDIT_F16, MMDIT_EPI_GELU, MMDIT_F32)                                         \
  GEMM_CASE(IN, MMDIT_F32, MMDIT_EPI_GELU, MMDIT_F32)                                         \
  GEMM_CASE(IN, MMDIT_F32, MMDIT_EPI_GATED_RES, MMDIT_F32)                                    \
  GEMM_CASE(IN, MMDIT_F32, MMDIT_EPI_GATED_RES, MMDIT_BF16)                                   \
  GEMM_CASE(IN, MMDIT_BF16, MMDIT_EPI_GATED_RES, MMDIT_F32)                                   \
  GEMM_CASE(IN, MMDIT_BF16, MMDIT_EPI_GATED_RES, MMDIT_BF16)
  GEMM_IN(MMDIT_BF16)
  GEMM_IN(MMDIT_F16)
#undef GEMM_IN
#undef GEMM_CASE
  return fail(MMDIT_ERR_DTYPE, "linear: unsupported dtype / epilogue combination");
}

}  // namespace mmdit
