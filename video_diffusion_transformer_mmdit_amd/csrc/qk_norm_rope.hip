// Fused per-head QK RMSNorm + 3D RoPE (one pass over HBM).
//
// Vimoo 1.0 notes, section 2.2: Q and K are RMS-normalised inside each head with their own
// learned scales; visual Q/K are then rotated by a 3D RoPE whose 128 head dims are split
// 16/56/56 over (t, h, w); conditioning tokens are not rotated.  Seaweed-7B, section 3.4,
// fuses QK-Norm and RoPE into one kernel because both are bound by memory traffic.
//
// Work decomposition (HBM-bound, ~4 bytes moved per element per tensor for bf16):
//   - a block of 256 threads owns TPB whole tokens (all heads of q and of k);
//   - one thread owns one 16-byte chunk of 8 dims = 4 rotation pairs of one head row, so a
//     head row of 128 dims is 16 consecutive lanes and its sum of squares is a 16-lane
//     butterfly;
//   - thread t always handles the same chunk column (t % 16) of every head row it visits,
//     so the 64 (cos, sin) pairs of a token are computed once per block into LDS, in
//     double-precision angle arithmetic with range reduction before the fp32 sincos.
#include "common.h"

namespace mmdit {

struct RopeTable {
  double freq[64];   // base^(-2j/d_band) of each rotation pair
  int32_t axis[64];  // 0 = t, 1 = h, 2 = w, -1 = no rotation
  int64_t T, H, W;
};

constexpr int QKN_THREADS = 256;
constexpr int QKN_D = 128;

template <int IN_DT, int OUT_DT, int SC_DT, bool ROPE>
__global__ __launch_bounds__(QKN_THREADS) void qk_norm_rope_kernel(
    const void* __restrict__ q, const void* __restrict__ k, int64_t in_stride,
    const void* __restrict__ q_scale, const void* __restrict__ k_scale, int64_t scale_head_stride,
    void* q_out, void* k_out, int64_t out_stride, int64_t n_tokens_total, int64_t n_per_batch,
    int heads, int tpb, float eps, RopeTable rope) {
  __shared__ float2 cs[QKN_THREADS];  // [tpb][64] (cos, sin); tpb * 64 <= 256
  const int tid = threadIdx.x;
  const int64_t tok0 = (int64_t)blockIdx.x * tpb;

  if constexpr (ROPE) {
    if (tid < tpb * 64) {
      const int64_t tok = tok0 + tid / 64;
      const int p = tid % 64;
      float c = 1.f, s = 0.f;
      if (tok < n_tokens_total && rope.axis[p] >= 0) {
        const int64_t n = tok % n_per_batch;
        const int64_t hw = rope.H * rope.W;
        const int64_t pos3[3] = {n / hw, (n / rope.W) % rope.H, n % rope.W};
        const double ang = (double)pos3[rope.axis[p]] * rope.freq[p];
        const double two_pi = 6.283185307179586476925286766559;
        const double r = ang - rint(ang * (1.0 / two_pi)) * two_pi;
        sincosf((float)r, &s, &c);
      }
      cs[tid] = make_float2(c, s);
    }
    __syncthreads();
  }

  const int cpt = 32 * heads;          // 16-byte chunks per token (q and k)
  const int c = tid & 15;              // chunk column: dims 8c .. 8c+7
  for (int j = tid; j < tpb * cpt; j += QKN_THREADS) {
    const int tl = j / cpt;
    const int rem = j - tl * cpt;
    const int which = rem / (16 * heads);   // 0: q, 1: k
    const int head = (rem >> 4) % heads;
    const int64_t tok = tok0 + tl;
    const bool valid = tok < n_tokens_total;   // uniform over each 16-lane group
    const int64_t tok_c = valid ? tok : 0;
    const void* src = which ? k : q;
    void* dst = which ? k_out : q_out;
    const void* g = which ? k_scale : q_scale;

    float x[8];
    load8<IN_DT>(src, tok_c * in_stride + head * QKN_D + c * 8, x);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
    ss = group_sum<16>(ss);
    const float rstd = rsqrtf(ss * (1.0f / QKN_D) + eps);
    float gv[8];
    load8<SC_DT>(g, head * scale_head_stride + c * 8, gv);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = x[i] * rstd * gv[i];
    if constexpr (ROPE) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2 r = cs[tl * 64 + c * 4 + i];
        const float x0 = x[2 * i], x1 = x[2 * i + 1];
        x[2 * i] = x0 * r.x - x1 * r.y;
        x[2 * i + 1] = x0 * r.y + x1 * r.x;
      }
    }
    if (valid) store8<OUT_DT>(dst, tok * out_stride + head * QKN_D + c * 8, x);
  }
}

template <int IN_DT, int OUT_DT, int SC_DT>
static void launch_qkn_t(bool rope, dim3 grid, hipStream_t st, const void* q, const void* k,
                         int64_t in_stride, const void* qs, const void* ks, int64_t shs, void* qo,
                         void* ko, int64_t out_stride, int64_t ntot, int64_t nper, int heads,
                         int tpb, float eps, const RopeTable& tab) {
  if (rope)
    qk_norm_rope_kernel<IN_DT, OUT_DT, SC_DT, true><<<grid, QKN_THREADS, 0, st>>>(
        q, k, in_stride, qs, ks, shs, qo, ko, out_stride, ntot, nper, heads, tpb, eps, tab);
  else
    qk_norm_rope_kernel<IN_DT, OUT_DT, SC_DT, false><<<grid, QKN_THREADS, 0, st>>>(
        q, k, in_stride, qs, ks, shs, qo, ko, out_stride, ntot, nper, heads, tpb, eps, tab);
}

int launch_qk_norm_rope(const void* q, const void* k, int in_dtype, int64_t in_stride,
                        const void* q_scale, const void* k_scale, int scale_dtype,
                        int64_t scale_head_stride, void* q_out, void* k_out, int out_dtype,
                        int64_t out_stride, int64_t B, int64_t N, int64_t H, float eps,
                        const mmdit_rope3d* rope, hipStream_t stream) {
  const int64_t ntot = B * N;
  if (ntot == 0) return MMDIT_OK;
  RopeTable tab{};
  if (rope) {
    const int32_t d[3] = {rope->d_t, rope->d_h, rope->d_w};
    int p = 0;
    for (int a = 0; a < 3; ++a)
      for (int j = 0; j < d[a] / 2; ++j, ++p) {
        tab.axis[p] = a;
        tab.freq[p] = pow((double)rope->base, -2.0 * j / (double)d[a]);
      }
    for (; p < 64; ++p) { tab.axis[p] = -1; tab.freq[p] = 0.0; }
    tab.T = rope->T; tab.H = rope->H; tab.W = rope->W;
  }
  const int cpt = 32 * (int)H;
  const int tpb = cpt >= QKN_THREADS ? 1 : (QKN_THREADS / cpt > 4 ? 4 : QKN_THREADS / cpt);  // cs[] holds 4 tokens
  const dim3 grid((unsigned)((ntot + tpb - 1) / tpb));
  const bool r = rope != nullptr;
  const int h = (int)H;
#define QKN_CASE(I, O, S)                                                                   \
  if (in_dtype == I && out_dtype == O && scale_dtype == S) {                                \
    launch_qkn_t<I, O, S>(r, grid, stream, q, k, in_stride, q_scale, k_scale,               \
                          scale_head_stride, q_out, k_out, out_stride, ntot, N, h, tpb, eps, \
                          tab);                                                             \
    return check_launch("qk_norm_rope");                                                    \
  }
  QKN_CASE(MMDIT_BF16, MMDIT_BF16, MMDIT_BF16)
  QKN_CASE(MMDIT_BF16, MMDIT_BF16, MMDIT_F32)
  QKN_CASE(MMDIT_BF16, MMDIT_F16, MMDIT_BF16)
  QKN_CASE(MMDIT_BF16, MMDIT_F16, MMDIT_F32)
  QKN_CASE(MMDIT_BF16, MMDIT_F32, MMDIT_BF16)
  QKN_CASE(MMDIT_BF16, MMDIT_F32, MMDIT_F32)
  QKN_CASE(MMDIT_F32, MMDIT_F32, MMDIT_F32)
  QKN_CASE(MMDIT_F32, MMDIT_F32, MMDIT_BF16)
  QKN_CASE(MMDIT_F32, MMDIT_BF16, MMDIT_F32)
  QKN_CASE(MMDIT_F32, MMDIT_BF16, MMDIT_BF16)
  QKN_CASE(MMDIT_F16, MMDIT_F16, MMDIT_BF16)
  QKN_CASE(MMDIT_F16, MMDIT_F16, MMDIT_F32)
  QKN_CASE(MMDIT_F16, MMDIT_F32, MMDIT_BF16)
  QKN_CASE(MMDIT_F16, MMDIT_F32, MMDIT_F32)
#undef QKN_CASE
  return fail(MMDIT_ERR_DTYPE, "qk_norm_rope: unsupported dtype combination");
}

}  // namespace mmdit
