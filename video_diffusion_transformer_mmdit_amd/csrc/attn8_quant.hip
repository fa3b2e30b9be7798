// Operand preparation of the 8-bit joint attention (Wan report, section 4.4.3: INT8 for
// S = Q K^T, FP8 E4M3 for O = P V):
//   - Q^ codes with one INT8 scale per (token, head);
//   - K^ codes with one INT8 scale per (head, block of 64 consecutive keys of a stream), the
//     attention kernel's key tile;
//   - V codes with one E4M3 scale per (head, channel) over the keys of both streams, stored
//     transposed (channel-major) so that the P V product reads V^T rows directly, with the
//     keys of each 64-key tile in the order the kernel's probability registers hold them.
// Scales are amax / qmax in f32 (an all-zero group takes 1); codes come from x * (1/s) in
// f32: rint then clamp to +-127 for INT8, clamp to +-448 then v_cvt_pk_fp8_f32 for E4M3.
// Bound by HBM: Q, K, V read once (V twice: amax, then codes), codes written once.
#include "common.h"

namespace mmdit {

constexpr int A8_TILE = 64;      // keys per tile / per K scale block
constexpr int A8_D = 128;

// Position of tile key k inside its 64-byte V^T row: the kernel's lane group g of a 32-key
// half h holds keys 32h + 8i + 4g + c (i, c = 0..3) as bytes 16(2h + g) + 4i + c.
__device__ __forceinline__ int a8_vpos(int k) {
  const int h = k >> 5, i = (k >> 3) & 3, g = (k >> 2) & 1, c = k & 3;
  return 16 * (2 * h + g) + 4 * i + c;
}

__device__ __forceinline__ uint32_t pack_i8x4(const float (&v)[8], int o, float inv) {
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float r = fminf(fmaxf(rintf(v[o + e] * inv), -127.f), 127.f);
    w |= ((uint32_t)(int)r & 0xffu) << (8 * e);
  }
  return w;
}

// The four 8-value chunks of a thread's 32 dims of one token row, every load issued before
// any use (a load under a branch waited for its data before the branch closed); a row past
// the stream's end reads its last row and is zeroed.
template <int DT>
__device__ __forceinline__ void load_dims32(const void* p, int64_t elem, bool valid, float (&x)[4][8]) {
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) load8<DT>(p, elem + 8 * ch, x[ch]);
  if (!valid) {
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
#pragma unroll
      for (int e = 0; e < 8; ++e) x[ch][e] = 0.f;
  }
}

// One workgroup per (64-token block, head, batch item) of one stream.  Thread t owns token
// t / 4 of the block and dims [32 (t % 4), +32).
template <int DT>
__global__ __launch_bounds__(256) void attn8_qk_quant_kernel(const void* __restrict__ q, const void* __restrict__ k,
                                                             int64_t stride, int64_t n, int H, int8_t* __restrict__ q8,
                                                             float* __restrict__ sq, int8_t* __restrict__ k8,
                                                             float* __restrict__ sk) {
  __shared__ float red[4];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nblk = gridDim.x;
  const int tok = threadIdx.x >> 2, qtr = threadIdx.x & 3;
  const int64_t row = (int64_t)blk * A8_TILE + tok;
  const bool valid = row < n;
  const int64_t src = (b * n + (valid ? row : n - 1)) * stride + h * A8_D + 32 * qtr;
  float qv[4][8], kv[4][8];
  float qa = 0.f, ka = 0.f;
  load_dims32<DT>(q, src, valid, qv);
  load_dims32<DT>(k, src, valid, kv);
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qa = fmaxf(qa, fabsf(qv[ch][e]));
      ka = fmaxf(ka, fabsf(kv[ch][e]));
    }
  }
  // Q: amax over the token's four threads
  qa = fmaxf(qa, __shfl_xor(qa, 1, 64));
  qa = fmaxf(qa, __shfl_xor(qa, 2, 64));
  // K: amax over the block
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ka = fmaxf(ka, __shfl_xor(ka, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ka;
  __syncthreads();
  ka = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s_q = qa > 0.f ? qa / 127.f : 1.f, s_k = ka > 0.f ? ka / 127.f : 1.f;
  const float iq = 1.f / s_q, ik = 1.f / s_k;
  if (valid) {
    const int64_t dst = ((b * n + row) * H + h) * A8_D + 32 * qtr;
    uint4 w[2], u[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      w[hh] = make_uint4(pack_i8x4(qv[2 * hh], 0, iq), pack_i8x4(qv[2 * hh], 4, iq),
                         pack_i8x4(qv[2 * hh + 1], 0, iq), pack_i8x4(qv[2 * hh + 1], 4, iq));
      u[hh] = make_uint4(pack_i8x4(kv[2 * hh], 0, ik), pack_i8x4(kv[2 * hh], 4, ik),
                         pack_i8x4(kv[2 * hh + 1], 0, ik), pack_i8x4(kv[2 * hh + 1], 4, ik));
    }
    *reinterpret_cast<uint4*>(q8 + dst) = w[0];
    *reinterpret_cast<uint4*>(q8 + dst + 16) = w[1];
    *reinterpret_cast<uint4*>(k8 + dst) = u[0];
    *reinterpret_cast<uint4*>(k8 + dst + 16) = u[1];
    if (qtr == 0) sq[((int64_t)b * H + h) * n + row] = s_q;
  }
  if (threadIdx.x == 0) sk[((int64_t)b * H + h) * nblk + blk] = s_k;
}

__global__ void attn8_zero_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// Per-channel amax of V over one 64-token block, merged into amax[b, h, :] with an atomic max
// on the float bits (non-negative floats order as unsigned integers).
template <int DT>
__global__ __launch_bounds__(256) void attn8_v_amax_kernel(const void* __restrict__ v, int64_t stride, int64_t n,
                                                           int H, float* __restrict__ amax) {
  __shared__ float red[4][A8_D];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tok = threadIdx.x >> 2, qtr = threadIdx.x & 3;
  const int64_t row = (int64_t)blk * A8_TILE + tok;
  float m[32];
  {
    float x[4][8];
    load_dims32<DT>(v, (b * n + (row < n ? row : n - 1)) * stride + h * A8_D + 32 * qtr, row < n, x);
#pragma unroll
    for (int ch = 0; ch < 4; ++ch)
#pragma unroll
      for (int e = 0; e < 8; ++e) m[8 * ch + e] = fabsf(x[ch][e]);
  }
  // lanes 4 apart hold the same dims of other tokens
#pragma unroll
  for (int o = 4; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < 32; ++e) m[e] = fmaxf(m[e], __shfl_xor(m[e], o, 64));
  if ((threadIdx.x & 63) < 4) {
#pragma unroll
    for (int e = 0; e < 32; ++e) red[threadIdx.x >> 6][32 * qtr + e] = m[e];
  }
  __syncthreads();
  if (threadIdx.x < A8_D) {
    const int d = threadIdx.x;
    const float r = fmaxf(fmaxf(red[0][d], red[1][d]), fmaxf(red[2][d], red[3][d]));
    atomicMax(reinterpret_cast<unsigned int*>(amax + ((int64_t)b * H + h) * A8_D + d), __float_as_uint(r));
  }
}

// E4M3 codes of one 64-token block of V, written channel-major into v8t[b, h, d, np] with the
// tile's keys at a8_vpos (padding keys past n are zero codes).
template <int DT>
__global__ __launch_bounds__(256) void attn8_v_quant_kernel(const void* __restrict__ v, int64_t stride, int64_t n,
                                                            int H, const float* __restrict__ amax,
                                                            uint8_t* __restrict__ v8t, int64_t np) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[A8_D * A8_TILE];
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tok = threadIdx.x >> 2, qtr = threadIdx.x & 3;
  const int64_t row = (int64_t)blk * A8_TILE + tok;
  const float* am = amax + ((int64_t)b * H + h) * A8_D + 32 * qtr;
  const int pos = a8_vpos(tok);
  float xv[4][8];
  load_dims32<DT>(v, (b * n + (row < n ? row : n - 1)) * stride + h * A8_D + 32 * qtr, row < n, xv);
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    const float (&x)[8] = xv[ch];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float a0 = am[8 * ch + e], a1 = am[8 * ch + e + 1];
      const float s0 = a0 > 0.f ? a0 / 448.f : 1.f, s1 = a1 > 0.f ? a1 / 448.f : 1.f;
      const float y0 = fminf(fmaxf(x[e] * (1.f / s0), -448.f), 448.f);
      const float y1 = fminf(fmaxf(x[e + 1] * (1.f / s1), -448.f), 448.f);
      const int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
      const int d = 32 * qtr + 8 * ch + e;
      tile[d * A8_TILE + pos] = (uint8_t)(w & 0xff);
      tile[(d + 1) * A8_TILE + pos] = (uint8_t)((w >> 8) & 0xff);
    }
  }
  __syncthreads();
  uint8_t* base = v8t + ((int64_t)b * H + h) * A8_D * np + (int64_t)blk * A8_TILE;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = threadIdx.x + 256 * i;   // 512 chunks of 16 bytes: 128 rows x 4
    const int d = c >> 2, part = c & 3;
    *reinterpret_cast<uint4*>(base + d * np + 16 * part) = *reinterpret_cast<const uint4*>(tile + d * A8_TILE + 16 * part);
  }
}

__global__ void attn8_v_scale_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = p[i] > 0.f ? p[i] / 448.f : 1.f;
}

template <int DT>
static int attn8_quant_go(const void* const* q, const void* const* k, const void* const* v, const int64_t* n,
                          int64_t stride, int64_t B, int64_t H, const mmdit_attn8_stream* const* out, float* v_scale,
                          hipStream_t stream) {
  const int64_t nsv = B * H * A8_D;
  attn8_zero_kernel<<<dim3((unsigned)((nsv + 255) / 256)), 256, 0, stream>>>(v_scale, nsv);
  for (int s = 0; s < 2; ++s) {
    if (n[s] == 0) continue;
    const dim3 grid((unsigned)((n[s] + A8_TILE - 1) / A8_TILE), (unsigned)H, (unsigned)B);
    attn8_qk_quant_kernel<DT><<<grid, 256, 0, stream>>>(q[s], k[s], stride, n[s], (int)H, static_cast<int8_t*>(out[s]->q8),
                                                        out[s]->q_scale, static_cast<int8_t*>(out[s]->k8), out[s]->k_scale);
    attn8_v_amax_kernel<DT><<<grid, 256, 0, stream>>>(v[s], stride, n[s], (int)H, v_scale);
  }
  for (int s = 0; s < 2; ++s) {
    if (n[s] == 0) continue;
    const dim3 grid((unsigned)((n[s] + A8_TILE - 1) / A8_TILE), (unsigned)H, (unsigned)B);
    const int64_t np = grid.x * (int64_t)A8_TILE;
    attn8_v_quant_kernel<DT><<<grid, 256, 0, stream>>>(v[s], stride, n[s], (int)H, v_scale,
                                                       static_cast<uint8_t*>(out[s]->v8t), np);
  }
  attn8_v_scale_kernel<<<dim3((unsigned)((nsv + 255) / 256)), 256, 0, stream>>>(v_scale, nsv);
  return check_launch("attn8_quantize");
}

int launch_attn8_quantize(const void* const* q, const void* const* k, const void* const* v, const int64_t* n,
                          int in_dtype, int64_t stride, int64_t B, int64_t H, const mmdit_attn8_stream* const* out,
                          float* v_scale, hipStream_t stream) {
  if (B == 0 || H == 0 || n[0] + n[1] == 0) return MMDIT_OK;
  if (in_dtype == MMDIT_BF16) return attn8_quant_go<MMDIT_BF16>(q, k, v, n, stride, B, H, out, v_scale, stream);
  if (in_dtype == MMDIT_F16) return attn8_quant_go<MMDIT_F16>(q, k, v, n, stride, B, H, out, v_scale, stream);
  return attn8_quant_go<MMDIT_F32>(q, k, v, n, stride, B, H, out, v_scale, stream);
}

}  // namespace mmdit
