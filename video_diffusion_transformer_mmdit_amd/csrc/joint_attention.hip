// Joint non-causal attention over [conditioning | visual] tokens, split back per stream.
//
// Vimoo 1.0 notes, section 2.2: the two streams' projected sequences are concatenated for
// one attention and the result is split back; the DiT attention is non-causal (Wan report
// reading guide).  Its cost is 4*N^2*D per head (Wan report, section 4.3.1), the dominant
// term of the block.  The concatenation is never materialised: key / query index j < n_cond
// reads the conditioning tensors, j >= n_cond the visual ones.
//
// 16-bit MFMA flash kernel (gfx950):
//   - workgroup = 4 wave64s = 128 queries of one (batch, head); each wave owns 32 queries.
//   - The wave computes S^T = K Q^T with v_mfma_f32_32x32x16_{f16,bf16} (A = 32 keys x 16 dims
//     from LDS, B = the wave's Q held in registers for the whole kernel).  In the S^T
//     accumulator layout every lane holds one query (lane % 32) and 16 keys, so the online
//     softmax statistics are per-lane scalars and only the row max needs one exchange
//     between the two half-waves per tile; the row sum is combined once at the end.
//   - P^T comes straight from those accumulators (converted to f16) as the B operand of
//     O^T = V^T P^T; O^T accumulates 128 dims x 32 queries per wave in registers.
//   - K and V tiles of 64 keys are staged in LDS (2 stages x 32 KiB).  K rows are stored
//     as is with an XOR swizzle; V is transposed on the way in (register 4x2 byte shuffles,
//     8-byte LDS stores) so each lane reads its 8 keys of one dim as a single 16-byte LDS
//     read, with keys permuted inside each 16-key group to match the accumulator layout.
//   - exp2 with log2(e) * softmax_scale folded into one FMA per score.
//   - Precision: S = Q K^T runs on the operand type of Q and K (f16 or bf16); P is rounded
//     to f16 (P lies in [0, 1], where f16 keeps 3 more mantissa bits than bf16) and PV runs
//     on f16 MFMA, so a bf16 V is converted to f16 while it is staged into LDS.
//
// fp32 path: a plain wave-per-query VALU kernel with the same online softmax, used for the
// fp32 workload (small sizes).
#include "common.h"

namespace mmdit {

constexpr int ATT_D = 128;
constexpr int ATT_BM = 128;
constexpr int ATT_BN = 64;
constexpr int ATT_THREADS = 256;
constexpr int ATT_K_BYTES = ATT_BN * ATT_D * 2;   // 16 KiB
constexpr int ATT_V_BYTES = ATT_D * ATT_BN * 2;   // 16 KiB
constexpr int ATT_STAGE = ATT_K_BYTES + ATT_V_BYTES;

struct AttnArgs {
  const uint16_t* q[2];   // [0] cond, [1] vis
  const uint16_t* k[2];
  const uint16_t* v[2];
  void* o[2];
  float* lse;
  int64_t n_cond, n_vis, N;
  int64_t in_stride, out_stride;
  int H;
  int nqt;
  float scale_log2;       // softmax_scale * log2(e)
};

__device__ __forceinline__ const uint16_t* row_ptr(const uint16_t* const* base, int64_t j,
                                                   int64_t n_cond, int64_t n_vis, int64_t b,
                                                   int64_t stride, int h) {
  return j < n_cond ? base[0] + (b * n_cond + j) * stride + h * ATT_D
                    : base[1] + (b * n_vis + (j - n_cond)) * stride + h * ATT_D;
}

template <int DT>
__device__ __forceinline__ f32x16 mfma16(const uint4& a, const uint4& b, const f32x16& c) {
  if constexpr (DT == MMDIT_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two bf16 in one word -> the same two values as f16 in one word.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16x2(lo_bf16(w), hi_bf16(w));
}

// Physical 8-byte slot (0..15) of the V^T row for key quad `qd` (keys 4qd .. 4qd+3) of a
// 64-key tile.  Inside each group of 16 keys the quads are stored in order 0, 2, 1, 3 so
// that lane half g reads keys {16s+4g .. +3, 16s+8+4g .. +3} as one 16-byte slot 2s+g,
// which is the key order of the S^T accumulator; the 16-byte slot is XOR-swizzled by
// (d / 2) % 8.
__device__ __forceinline__ int vt_slot8(int qd, int d) {
  const int r = qd & 3;
  const int logical = (qd & ~3) | (((r & 1) << 1) | (r >> 1));
  return logical ^ (((d >> 1) & 7) << 1);
}

template <int QK_DT, int V_DT, int OUT_DT, bool LSE>
__global__ __launch_bounds__(ATT_THREADS) void joint_attn_mfma_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * ATT_STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int qt = blockIdx.x % a.nqt;
  const int bh = blockIdx.x / a.nqt;
  const int h = bh % a.H;
  const int64_t b = bh / a.H;
  const int64_t N = a.N;

  // ---- this lane's query row, held as the B operand (8 k-steps of 16 dims)
  const int64_t qi = (int64_t)qt * ATT_BM + wave * 32 + l32;
  uint4 qf[8];
  if (qi < N) {
    const uint16_t* qp = row_ptr(a.q, qi, a.n_cond, a.n_vis, b, a.in_stride, h);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const uint4*>(qp + ks * 16 + g * 8);
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = make_uint4(0, 0, 0, 0);
  }

  // ---- K / V tile staging.  K: thread owns chunks tid + 256 i (key = chunk / 16, 16-byte
  // column chunk % 16).  V: thread owns key quad tid % 16 and dim chunk tid / 16.
  uint4 rk[4], rv[4];
  const int v_qd = tid & 15, v_dc = tid >> 4;
  auto gload = [&](int64_t j0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + ATT_THREADS * i;
      const int64_t j = j0 + (ch >> 4);
      rk[i] = j < N ? *reinterpret_cast<const uint4*>(
                          row_ptr(a.k, j, a.n_cond, a.n_vis, b, a.in_stride, h) + (ch & 15) * 8)
                    : make_uint4(0, 0, 0, 0);
      const int64_t jv = j0 + v_qd * 4 + i;
      rv[i] = jv < N ? *reinterpret_cast<const uint4*>(
                           row_ptr(a.v, jv, a.n_cond, a.n_vis, b, a.in_stride, h) + v_dc * 8)
                     : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* sk = lds + buf * ATT_STAGE;
    uint8_t* sv = sk + ATT_K_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + ATT_THREADS * i;
      const int key = ch >> 4, cc = ch & 15;
      *reinterpret_cast<uint4*>(sk + key * 256 + ((cc ^ (key & 15)) << 4)) = rk[i];
    }
    // transpose 4 keys x 8 dims: word for dim 2m+e holds the 4 keys' values of that dim
    uint32_t w0[4] = {rv[0].x, rv[0].y, rv[0].z, rv[0].w};
    uint32_t w1[4] = {rv[1].x, rv[1].y, rv[1].z, rv[1].w};
    uint32_t w2[4] = {rv[2].x, rv[2].y, rv[2].z, rv[2].w};
    uint32_t w3[4] = {rv[3].x, rv[3].y, rv[3].z, rv[3].w};
    if constexpr (V_DT == MMDIT_BF16) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        w0[m] = bf16x2_to_f16x2(w0[m]); w1[m] = bf16x2_to_f16x2(w1[m]);
        w2[m] = bf16x2_to_f16x2(w2[m]); w3[m] = bf16x2_to_f16x2(w3[m]);
      }
    }
    uint2 col[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      col[2 * m] = make_uint2((w0[m] & 0xffffu) | (w1[m] << 16), (w2[m] & 0xffffu) | (w3[m] << 16));
      col[2 * m + 1] = make_uint2((w0[m] >> 16) | (w1[m] & 0xffff0000u),
                                  (w2[m] >> 16) | (w3[m] & 0xffff0000u));
    }
    // odd dim chunks store their 8 dims in swapped pair order so that one store
    // instruction covers both parities of d (both halves of the LDS banks)
    const bool swp = v_dc & 1;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int rr = r ^ (swp ? 1 : 0);
      const int d = v_dc * 8 + rr;
      const uint2 val = swp ? col[r ^ 1] : col[r];
      *reinterpret_cast<uint2*>(sv + d * 128 + (vt_slot8(v_qd, d) << 3)) = val;
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
  float m_run = -INFINITY;   // running max of scaled logits (log2 domain)
  float l_run = 0.f;         // this lane's partial row sum

  const int ntiles = (int)((N + ATT_BN - 1) / ATT_BN);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int jt = 0; jt < ntiles; ++jt) {
    const int buf = jt & 1;
    const int64_t j0 = (int64_t)jt * ATT_BN;
    if (jt + 1 < ntiles) gload(j0 + ATT_BN);
    const uint8_t* sk = lds + buf * ATT_STAGE;
    const uint8_t* sv = sk + ATT_K_BYTES;

    // S^T (64 keys x 32 queries) = K Q^T
    f32x16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[st][e] = 0.f;
      const int key = st * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint4 kf = *reinterpret_cast<const uint4*>(sk + key * 256 + (((2 * ks + g) ^ (key & 15)) << 4));
        s[st] = mfma16<QK_DT>(kf, qf[ks], s[st]);
      }
    }
    // mask keys past the end (last tile only)
    if (j0 + ATT_BN > N) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t j = j0 + st * 32 + 8 * (e >> 2) + 4 * g + (e & 3);
          if (j >= N) s[st][e] = -INFINITY;
        }
    }
    float mx = s[0][0];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[st][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
    uint4 pf[4];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = exp2f(fmaf(s[st][e], a.scale_log2, -m_new));
        psum += p[e];
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        pf[st * 2 + hh] = make_uint4(pack_f16x2(p[8 * hh + 0], p[8 * hh + 1]),
                                     pack_f16x2(p[8 * hh + 2], p[8 * hh + 3]),
                                     pack_f16x2(p[8 * hh + 4], p[8 * hh + 5]),
                                     pack_f16x2(p[8 * hh + 6], p[8 * hh + 7]));
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;

    // O^T (128 dims x 32 queries) += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = dt * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 vf = *reinterpret_cast<const uint4*>(sv + d * 128 + (((2 * ks + g) ^ ((d >> 1) & 7)) << 4));
        o[dt] = mfma16<MMDIT_F16>(vf, pf[ks], o[dt]);
      }
    }
    if (jt + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- finish: combine the two half-wave partial sums, normalise, store
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qi >= N) return;
  const float inv = 1.0f / l_tot;
  const int s_idx = qi < a.n_cond ? 0 : 1;
  const int64_t row = qi < a.n_cond ? b * a.n_cond + qi : b * a.n_vis + (qi - a.n_cond);
  void* obase = a.o[s_idx];
  const int64_t ooff = row * a.out_stride + (int64_t)h * ATT_D;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int d0 = dt * 32 + 8 * e4 + 4 * g;
      const float v0 = o[dt][4 * e4 + 0] * inv, v1 = o[dt][4 * e4 + 1] * inv;
      const float v2 = o[dt][4 * e4 + 2] * inv, v3 = o[dt][4 * e4 + 3] * inv;
      if constexpr (OUT_DT == MMDIT_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(obase) + ooff + d0) = make_float4(v0, v1, v2, v3);
      } else if constexpr (OUT_DT == MMDIT_BF16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(obase) + ooff + d0) =
            make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(obase) + ooff + d0) =
            make_uint2(pack_f16x2(v0, v1), pack_f16x2(v2, v3));
      }
    }
  if constexpr (LSE) {
    if (g == 0) a.lse[(b * a.H + h) * N + qi] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
  }
}

// ------------------------------------------------------------------ fp32 VALU path
struct AttnArgsF32 {
  const float* q[2];
  const float* k[2];
  const float* v[2];
  void* o[2];
  float* lse;
  int64_t n_cond, n_vis, N;
  int64_t in_stride, out_stride;
  int H;
  float scale;
};

__device__ __forceinline__ const float* row_ptr_f32(const float* const* base, int64_t j, int64_t n_cond,
                                                    int64_t n_vis, int64_t b, int64_t stride, int h) {
  return j < n_cond ? base[0] + (b * n_cond + j) * stride + h * ATT_D
                    : base[1] + (b * n_vis + (j - n_cond)) * stride + h * ATT_D;
}

template <int OUT_DT, bool LSE>
__global__ __launch_bounds__(64) void joint_attn_f32_kernel(AttnArgsF32 a) {
  __shared__ float qs[ATT_D];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const int64_t qi = blockIdx.x % a.N;
  const int bh = (int)(blockIdx.x / a.N);
  const int h = bh % a.H;
  const int64_t b = bh / a.H;
  const float* qp = row_ptr_f32(a.q, qi, a.n_cond, a.n_vis, b, a.in_stride, h);
  qs[2 * lane] = qp[2 * lane];
  qs[2 * lane + 1] = qp[2 * lane + 1];
  __syncthreads();
  float m_run = -INFINITY, l_run = 0.f, o0 = 0.f, o1 = 0.f;
  for (int64_t j0 = 0; j0 < a.N; j0 += 64) {
    const int64_t j = j0 + lane;
    float sv = -INFINITY;
    if (j < a.N) {
      const float* kp = row_ptr_f32(a.k, j, a.n_cond, a.n_vis, b, a.in_stride, h);
      float dot = 0.f;
      for (int d = 0; d < ATT_D; ++d) dot = fmaf(qs[d], kp[d], dot);
      sv = dot * a.scale;
    }
    float mx = sv;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = expf(m_run - m_new);
    const float p = expf(sv - m_new);
    l_run = l_run * alpha + group_sum<64>(p);
    m_run = m_new;
    __syncthreads();
    ps[lane] = p;
    __syncthreads();
    o0 *= alpha;
    o1 *= alpha;
    const int64_t jend = (a.N - j0) < 64 ? (a.N - j0) : 64;
    for (int jj = 0; jj < jend; ++jj) {
      const float* vp = row_ptr_f32(a.v, j0 + jj, a.n_cond, a.n_vis, b, a.in_stride, h);
      o0 = fmaf(ps[jj], vp[2 * lane], o0);
      o1 = fmaf(ps[jj], vp[2 * lane + 1], o1);
    }
  }
  const int s_idx = qi < a.n_cond ? 0 : 1;
  const int64_t row = qi < a.n_cond ? b * a.n_cond + qi : b * a.n_vis + (qi - a.n_cond);
  const int64_t off = row * a.out_stride + (int64_t)h * ATT_D + 2 * lane;
  store1<OUT_DT>(a.o[s_idx], off, o0 / l_run);
  store1<OUT_DT>(a.o[s_idx], off + 1, o1 / l_run);
  if constexpr (LSE) {
    if (lane == 0) a.lse[(b * a.H + h) * a.N + qi] = m_run + logf(l_run);
  }
}

template <int QK, int V>
static int attn_go(const AttnArgs& a, dim3 grid, int out_dtype, bool has_lse, hipStream_t stream) {
#define ATT_GO(O, L) joint_attn_mfma_kernel<QK, V, O, L><<<grid, ATT_THREADS, 0, stream>>>(a)
  if (out_dtype == MMDIT_F32) { if (has_lse) ATT_GO(MMDIT_F32, true); else ATT_GO(MMDIT_F32, false); }
  else if (out_dtype == MMDIT_BF16) { if (has_lse) ATT_GO(MMDIT_BF16, true); else ATT_GO(MMDIT_BF16, false); }
  else if (out_dtype == MMDIT_F16) { if (has_lse) ATT_GO(MMDIT_F16, true); else ATT_GO(MMDIT_F16, false); }
  else return fail(MMDIT_ERR_DTYPE, "joint_attention: bad out dtype");
#undef ATT_GO
  return check_launch("joint_attention");
}

int launch_joint_attention(const void* q_vis, const void* k_vis, const void* v_vis, int64_t n_vis,
                           const void* q_cond, const void* k_cond, const void* v_cond,
                           int64_t n_cond, int qk_dtype, int v_dtype, int64_t in_stride, int64_t B, int64_t H,
                           float softmax_scale, void* o_vis, void* o_cond, int out_dtype,
                           int64_t out_stride, float* lse, hipStream_t stream) {
  const int64_t N = n_vis + n_cond;
  if (B == 0 || H == 0 || N == 0) return MMDIT_OK;
  const bool has_lse = lse != nullptr;
  if (qk_dtype != MMDIT_F32) {
    AttnArgs a{};
    a.q[0] = static_cast<const uint16_t*>(q_cond); a.q[1] = static_cast<const uint16_t*>(q_vis);
    a.k[0] = static_cast<const uint16_t*>(k_cond); a.k[1] = static_cast<const uint16_t*>(k_vis);
    a.v[0] = static_cast<const uint16_t*>(v_cond); a.v[1] = static_cast<const uint16_t*>(v_vis);
    a.o[0] = o_cond; a.o[1] = o_vis;
    a.lse = lse;
    a.n_cond = n_cond; a.n_vis = n_vis; a.N = N;
    a.in_stride = in_stride; a.out_stride = out_stride;
    a.H = (int)H;
    a.nqt = (int)((N + ATT_BM - 1) / ATT_BM);
    a.scale_log2 = softmax_scale * 1.44269504088896340736f;
    const int64_t blocks = (int64_t)a.nqt * H * B;
    if (blocks > 0x7fffffff) return fail(MMDIT_ERR_SHAPE, "joint_attention: grid too large");
    const dim3 grid((unsigned)blocks);
    if (qk_dtype == MMDIT_F16 && v_dtype == MMDIT_F16) return attn_go<MMDIT_F16, MMDIT_F16>(a, grid, out_dtype, has_lse, stream);
    if (qk_dtype == MMDIT_F16 && v_dtype == MMDIT_BF16) return attn_go<MMDIT_F16, MMDIT_BF16>(a, grid, out_dtype, has_lse, stream);
    if (qk_dtype == MMDIT_BF16 && v_dtype == MMDIT_BF16) return attn_go<MMDIT_BF16, MMDIT_BF16>(a, grid, out_dtype, has_lse, stream);
    if (qk_dtype == MMDIT_BF16 && v_dtype == MMDIT_F16) return attn_go<MMDIT_BF16, MMDIT_F16>(a, grid, out_dtype, has_lse, stream);
    return fail(MMDIT_ERR_DTYPE, "joint_attention: unsupported dtype combination");
  }
  if (qk_dtype == MMDIT_F32 && v_dtype == MMDIT_F32) {
    AttnArgsF32 a{};
    a.q[0] = static_cast<const float*>(q_cond); a.q[1] = static_cast<const float*>(q_vis);
    a.k[0] = static_cast<const float*>(k_cond); a.k[1] = static_cast<const float*>(k_vis);
    a.v[0] = static_cast<const float*>(v_cond); a.v[1] = static_cast<const float*>(v_vis);
    a.o[0] = o_cond; a.o[1] = o_vis;
    a.lse = lse;
    a.n_cond = n_cond; a.n_vis = n_vis; a.N = N;
    a.in_stride = in_stride; a.out_stride = out_stride;
    a.H = (int)H;
    a.scale = softmax_scale;
    const int64_t blocks = N * H * B;
    if (blocks > 0x7fffffff) return fail(MMDIT_ERR_SHAPE, "joint_attention: grid too large");
    const dim3 grid((unsigned)blocks);
#define ATT_GO(O, L) joint_attn_f32_kernel<O, L><<<grid, 64, 0, stream>>>(a)
    if (out_dtype == MMDIT_F32) { if (has_lse) ATT_GO(MMDIT_F32, true); else ATT_GO(MMDIT_F32, false); }
    else if (out_dtype == MMDIT_BF16) { if (has_lse) ATT_GO(MMDIT_BF16, true); else ATT_GO(MMDIT_BF16, false); }
    else if (out_dtype == MMDIT_F16) { if (has_lse) ATT_GO(MMDIT_F16, true); else ATT_GO(MMDIT_F16, false); }
    else return fail(MMDIT_ERR_DTYPE, "joint_attention: bad out dtype");
#undef ATT_GO
    return check_launch("joint_attention_f32");
  }
  return fail(MMDIT_ERR_DTYPE, "joint_attention: f32 Q/K need an f32 V");
}

}  // namespace mmdit
