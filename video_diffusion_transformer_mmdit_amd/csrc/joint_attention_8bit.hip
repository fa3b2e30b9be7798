// 8-bit joint attention (Wan report, section 4.4.3): S = Q K^T on INT8 codes, O = P V on
// FP8 E4M3 codes, accumulated across key tiles in f32; the same joint, non-causal attention
// over [conditioning | visual] tokens as the 16-bit kernel (Vimoo 1.0 notes, section 2.2).
//
//   logit (log2 units) of query i, key j = acc_ij * c_i,  acc_ij the exact integer dot product
//   of the codes, c_i = s_q[i] * (s_k[tile] * softmax_scale * log2 e);
//   m = an integer reference, at least the ceiling of every logit seen so far;
//   P'_ij = 2^(acc_ij c_i + 8 - m) rounded to E4M3 (P' <= 256);
//   O_i = s_v * sum_j P'_ij V8_j / sum_j P'_ij.
//
// gfx950 design (the structure of the 16-bit kernel, with 8-bit operands):
//   - workgroup = 8 wave64s = 256 queries of one (batch, head), one workgroup per CU; the wave
//     holds its 32 queries' INT8 codes in registers (4 x 16 bytes per lane).
//   - S^T = K Q^T with v_mfma_i32_32x32x32_i8 (8 per 64-key tile instead of 16 f16 MFMAs);
//     every lane owns one query and 16 keys of each 32-key half, as in the 16-bit kernel.
//   - O^T += V^T P'^T with v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales): 4 per tile
//     (one per 32 channels) instead of 16.  V arrives channel-major with the keys of each
//     tile in the order the lane's probability registers hold them, so both MFMA operands
//     are plain 16-byte LDS / register reads and nothing is transposed.
//   - A fifth FP8 MFMA against a constant operand of ones adds up the same rounded P', so
//     the row sums come out of the matrix pipe, consistent with the weights P V used.
//   - The reference m is an integer: each rescale multiplies O and the row sums by an exact
//     power of two (v_ldexp), and the E4M3 rounding of P' does not depend on when m was
//     raised (powers of two commute with it above the subnormal range).
//   - Ping-pong of two wave groups (MFMA-only phases against VALU-only phases), LDS-DMA of
//     K and V tiles (8 KiB each) two stages deep, heads kept per XCD: as in the 16-bit kernel.
//     Each phase covers a pair of 64-key tiles (each with its own K scale), so the pipeline
//     fill and drain around a phase's barrier is paid once per 128 keys.
#include <type_traits>

#include "common.h"

namespace mmdit {

constexpr int A8_BM = 256;          // queries per workgroup
constexpr int A8_BN = 64;           // keys per tile
constexpr int A8_DIM = 128;
constexpr int A8_THREADS = 512;
constexpr int A8_TILE_BYTES = A8_BN * A8_DIM;   // 8 KiB for K (keys x dims) and for V^T (dims x keys)

struct Attn8Args {
  const int8_t* q8[2];      // [0] visual, [1] conditioning
  const float* sq[2];
  const int8_t* k8[2];
  const float* sk[2];
  const uint8_t* v8t[2];
  const float* sv;
  void* o[2];
  float* lse;
  int64_t n_seg[2];
  int64_t N;
  int64_t out_stride;
  int H;
  int nqt;
  float scale_log2;         // softmax_scale * log2(e)
  // Split tail, as in the 16-bit kernel: workgroups [0, full) take items (batch x head, query
  // tile) 0 .. full-1 over all keys; each remaining item is cut into `split` key ranges whose
  // partial results go to `part` for joint_attn_8bit_merge_kernel.  full == nbh * nqt: none.
  int nbh;
  int full;
  int split;
  float* part;
};

// one key range's partial result for one query tile: O (256 x 128 f32, V scale applied) then
// (m, l) per query
constexpr int64_t A8_PART_FLOATS = 256 * 128 + 256 * 2;

// (batch x head, query tile) of work item i; XCD x (i % 8) takes whole heads x, x + 8, ...
// when the (batch, head) count allows
__device__ __forceinline__ void attn8_item(const Attn8Args& a, int i, int& bh, int& qt) {
  if ((a.nbh & 7) == 0) {
    const int j = i >> 3;
    bh = (i & 7) + 8 * (j / a.nqt);
    qt = j % a.nqt;
  } else {
    bh = i / a.nqt;
    qt = i % a.nqt;
  }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ i32x16 mfma_i8(const uint4& a, const uint4& b, const i32x16& c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f8(const uint4& a0, const uint4& a1, const uint4& b0, const uint4& b1,
                                          const f32x16& c) {
  const i32x8 a = __builtin_shufflevector(__builtin_bit_cast(i32x4, a0), __builtin_bit_cast(i32x4, a1), 0, 1, 2, 3, 4, 5, 6, 7);
  const i32x8 b = __builtin_shufflevector(__builtin_bit_cast(i32x4, b0), __builtin_bit_cast(i32x4, b1), 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ int xhalf_max_i(int x) {   // max with the lane 32 apart
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return max((int)r[0], (int)r[1]);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t a8_rsrc(const void* p, int64_t bytes) {
  const uint64_t addr = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  const int num = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, num,
                                           0x00020000);
}

__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <int OUT_DT, bool LSE>
__global__ __launch_bounds__(A8_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void joint_attn_8bit_kernel(Attn8Args a) {
  // two K stages (rows = keys, 128 bytes) and two V^T stages (rows = channels, 64 bytes), each
  // stage a pair of 64-key tiles
  __shared__ __attribute__((aligned(16))) uint8_t lds_k0[2 * A8_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_k1[2 * A8_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v0[2 * A8_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v1[2 * A8_TILE_BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  int qt, bh;
  int slot = -1;   // a split-tail workgroup's partial-result slot
  {
    int item = blockIdx.x;
    if (item >= a.full) {
      slot = item - a.full;
      item = a.full + slot / a.split;
    }
    attn8_item(a, item, bh, qt);
  }
  const int h = bh % a.H;
  const int64_t b = bh / a.H;
  const int64_t N = a.N;
  const int64_t n_vis = a.n_seg[0], n_cond = a.n_seg[1];
  const int64_t HD = (int64_t)a.H * A8_DIM;

  // ---- this lane's query (queries in [cond | vis] order): codes and scale
  const int64_t qi = (int64_t)qt * A8_BM + wave * 32 + l32;
  uint4 qf[4];
  float sq = 0.f;
  if (qi < N) {
    const bool cq = qi < n_cond;
    const int64_t r = cq ? qi : qi - n_cond;
    const int64_t n_s = cq ? n_cond : n_vis;
    const int8_t* qp = (cq ? a.q8[1] : a.q8[0]) + (b * n_s + r) * HD + h * A8_DIM;
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = *reinterpret_cast<const uint4*>(qp + 32 * c + 16 * g);
    sq = (cq ? a.sq[1] : a.sq[0])[((int64_t)b * a.H + h) * n_s + r];
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = make_uint4(0, 0, 0, 0);
  }
  const float kc = a.scale_log2;
  const int t_vis = (int)((n_vis + A8_BN - 1) / A8_BN);
  const int t_cond = (int)((n_cond + A8_BN - 1) / A8_BN);
  const int ntiles = t_vis + t_cond;
  const int npairs = (ntiles + 1) / 2;   // pair p: tiles 2p and 2p + 1 (the latter may not exist)
  // this workgroup's pairs [jbeg, jend): all of them, or one range of a split-tail item
  int jbeg = 0, jend = npairs;
  if (slot >= 0) {
    const int sp = slot % a.split;
    jbeg = (int)((int64_t)npairs * sp / a.split);
    jend = (int)((int64_t)npairs * (sp + 1) / a.split);
  }
  auto tile_seg = [&](int jt, int& sg, int& t) { sg = jt < t_vis ? 0 : 1; t = sg ? jt - t_vis : jt; };
  auto kbuf = [&](auto stage) -> uint8_t* { if constexpr (decltype(stage)::value == 0) return lds_k0; else return lds_k1; };
  auto vbuf = [&](auto stage) -> uint8_t* { if constexpr (decltype(stage)::value == 0) return lds_v0; else return lds_v1; };
  constexpr std::integral_constant<int, 0> S0{};
  constexpr std::integral_constant<int, 1> S1{};

  // ---- per-lane LDS read offsets
  // S^T A operand: key 32 st + l32, dims [32 c + 16 g, +16): logical chunk 2c + g of the
  // 128-byte row, physical chunk ^ (key % 8)
  int k_rd[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) k_rd[c] = l32 * 128 + (((2 * c + g) ^ (l32 & 7)) << 4);
  // O^T A operand: channel 32 dt + l32, the 16-byte chunks g (keys of the first 32-key half)
  // and 2 + g (second half) of the 64-byte row, physical chunk ^ ((row / 4) % 4)
  int v_rd[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) v_rd[hh] = l32 * 64 + (((2 * hh + g) ^ ((l32 >> 2) & 3)) << 4);

  const i32x16 izero = {};
  // S^T of a pair: chains st = 0, 1 (the 32-key halves of the first tile) and 2, 3 (second)
  auto compute_s = [&](const uint8_t* kb, i32x16 (&s)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int st = 0; st < 4; ++st)
        s[st] = mfma_i8(lds16(kb + (st >> 1) * A8_TILE_BYTES + (st & 1) * 4096 + k_rd[c]), qf[c], c == 0 ? izero : s[st]);
  };
  auto phase_barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- ping-pong of two wave groups (see the 16-bit kernel): waves 0-3 load V, waves 4-7
  // load K; group 1 runs one phase behind group 0
  auto run = [&](auto grp_c) {
    constexpr int GRP = decltype(grp_c)::value;
    const int wg = wave & 3;
    // DMA i (0, 1) of this wave fills 1 KiB of the tile.  K: rows of 128 bytes, lane l ->
    // key 8 (2 wg + i) + l / 8, physical chunk l % 8 = logical ^ (key % 8).  V^T: rows of 64
    // bytes, lane l -> channel 16 (2 wg + i) + l / 4, physical chunk l % 4 = logical ^
    // ((channel / 4) % 4).  The immediate offset i * 1024 moves LDS destination and source
    // alike and is taken back out of the per-lane offset.
    const int64_t np_seg[2] = {(int64_t)t_vis * A8_BN, (int64_t)t_cond * A8_BN};
    int off[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ii = 2 * wg + i;
      if constexpr (GRP == 1) {
        const int row = 8 * ii + (lane >> 3);
        off[i] = row * (int)HD + (((lane & 7) ^ (row & 7)) << 4) - i * 1024;
      } else {
        const int row = 16 * ii + (lane >> 2);
        off[i] = (((lane & 3) ^ ((row >> 2) & 3)) << 4) - i * 1024;   // + row * np (per segment)
      }
    }
    int vrow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) vrow[i] = 16 * (2 * wg + i) + (lane >> 2);
    auto dma_tile = [&](int jt, uint8_t* dst) {
      int sg, t;
      tile_seg(jt, sg, t);
      auto* l = (__attribute__((address_space(3))) void*)(dst + wg * 2048);
      if constexpr (GRP == 1) {
        // keys of segment sg from tile t on; rows past the segment's end fail the range check
        const int64_t n_s = a.n_seg[sg];
        const int8_t* base = a.k8[sg] + (b * n_s + (int64_t)t * A8_BN) * HD + h * A8_DIM;
        const int64_t bytes = (n_s - (int64_t)t * A8_BN - 1) * HD + A8_DIM;
        const __amdgpu_buffer_rsrc_t r = a8_rsrc(base, bytes);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, off[0], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, off[1], 0, 1024, 0);
      } else {
        const int64_t np = np_seg[sg];
        const uint8_t* base = a.v8t[sg] + ((int64_t)b * a.H + h) * A8_DIM * np + (int64_t)t * A8_BN;
        const __amdgpu_buffer_rsrc_t r = a8_rsrc(base, (A8_DIM - 1) * np + A8_BN);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, vrow[0] * (int)np + off[0], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l, 16, vrow[1] * (int)np + off[1], 0, 1024, 0);
      }
    };
    // both tiles of pair jp.  A second tile past the last one takes the first tile's codes
    // again: its keys are masked to a zero weight, but the FP8 product of a zero weight with a
    // stale NaN code left in LDS by an earlier kernel would still be NaN, so that half must hold
    // finite codes.
    auto dma_pair = [&](int jp, uint8_t* dst) {
      dma_tile(2 * jp, dst);
      dma_tile(2 * jp + 1 < ntiles ? 2 * jp + 1 : 2 * jp, dst + A8_TILE_BYTES);
    };
    auto k_scale = [&](int jt) {
      if (jt >= ntiles) jt = ntiles - 1;   // the missing second tile of the last pair
      int sg, t;
      tile_seg(jt, sg, t);
      const int nb = sg ? t_cond : t_vis;
      return a.sk[sg][((int64_t)b * a.H + h) * nb + t];
    };

    f32x16 o[4], ol;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) ol[e] = 0.f;
    float m_run = 0.f;     // integer-valued reference (log2 units)
    uint4 pf[4];           // P'_j as E4M3 codes: tile u's bytes 16 hh + 4 i + c in pf[2 u + hh] = its
                           // key 32 hh + 8 i + 4 g + c
    const uint4 ones = make_uint4(0x38383838u, 0x38383838u, 0x38383838u, 0x38383838u);   // E4M3 1.0

    // M(j): S of pair j+1 and O^T += V_j^T P_j'^T (with the row sums) -- MFMA and LDS reads only
    auto phase_m = [&](auto cur_c, int jp, i32x16 (&s)[4]) {
      constexpr int CUR = decltype(cur_c)::value;
      constexpr std::integral_constant<int, CUR> cur{};
      constexpr std::integral_constant<int, CUR ^ 1> oth{};
      if constexpr (GRP == 0) dma_pair(jp + 1 < jend ? jp + 1 : jend - 1, vbuf(oth));
      else dma_pair(jp + 2 < jend ? jp + 2 : jend - 1, kbuf(cur));
      compute_s(kbuf(oth), s);
      const uint8_t* vb = vbuf(cur);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          o[dt] = mfma_f8(lds16(vb + u * A8_TILE_BYTES + dt * 2048 + v_rd[0]),
                          lds16(vb + u * A8_TILE_BYTES + dt * 2048 + v_rd[1]), pf[2 * u], pf[2 * u + 1], o[dt]);
      ol = mfma_f8(ones, ones, pf[0], pf[1], ol);
      ol = mfma_f8(ones, ones, pf[2], pf[3], ol);
      // 16 S MFMAs (one K read each), 8 P V MFMAs (two V reads each), 2 row-sum MFMAs; the
      // reads four ahead of their use, the phase's four DMA loads after its first four MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
      for (int i = 0; i < 26; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        if (i < 14) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        if (i < 4) __builtin_amdgcn_sched_group_barrier(0x010, 1, 1);
      }
      asm volatile("" ::"v"(s[0]), "v"(s[1]), "v"(s[2]), "v"(s[3]));
      asm volatile("" ::"v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(ol));
      if constexpr (GRP == 1) __builtin_amdgcn_s_waitcnt(0xF70);   // this wave's K loads have landed
      phase_barrier();
    };
    // the K scales of the pair the next V phase works on, loaded one phase ahead
    float sk_next[2] = {k_scale(2 * jbeg), k_scale(2 * jbeg + 1)};
    // V(j): integer row maxima, integer reference, P'_j = E4M3(2^(acc c + 8 - m))
    auto phase_v = [&](int jp, i32x16 (&s)[4]) {
      const float skt[2] = {sk_next[0], sk_next[1]};
      const int jn = jp + 1 < jend ? jp + 1 : jp;
      sk_next[0] = k_scale(2 * jn);
      sk_next[1] = k_scale(2 * jn + 1);
      int mxu[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int jt = 2 * jp + u;
        int64_t rows = 0;   // valid keys of tile u (none for a second tile past the last one)
        if (jt < ntiles) {
          int sg, t;
          tile_seg(jt, sg, t);
          rows = a.n_seg[sg] - (int64_t)t * A8_BN;
        }
        if (rows < A8_BN) {   // keys past the end of their stream
          // element e of chain st holds key 32 st + 8 (e / 4) + 4 g + e % 4 of the tile: an
          // arithmetic shift turns (rows - 1 - key) into an all-ones mask for keys past the end
          const int vl = (int)rows - 1 - 4 * g;
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int m = (vl - (st * 32 + 8 * (e >> 2) + (e & 3))) >> 31;
              s[2 * u + st][e] = (INT32_MIN & m) | (s[2 * u + st][e] & ~m);
            }
        }
        int m4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) m4[k] = max(s[2 * u][k], s[2 * u + 1][k]);
#pragma unroll
        for (int e = 4; e < 16; e += 4)
#pragma unroll
          for (int k = 0; k < 4; ++k) m4[k] = max(m4[k], max(s[2 * u][e + k], s[2 * u + 1][e + k]));
        mxu[u] = xhalf_max_i(max(max(m4[0], m4[1]), max(m4[2], m4[3])));
      }
      const float ci[2] = {sq * (skt[0] * kc), sq * (skt[1] * kc)};
      const float mt = fmaxf(ceilf((float)mxu[0] * ci[0]), ceilf((float)mxu[1] * ci[1]));
      if (jp == jbeg || __any(mt > m_run)) {
        const float mnew = jp == jbeg ? mt : fmaxf(m_run, mt);
        if (jp != jbeg) {
          const int sh = (int)(m_run - mnew);   // <= 0: an exact power-of-two rescale
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[dt][e] = __builtin_ldexpf(o[dt][e], sh);
#pragma unroll
          for (int e = 0; e < 16; ++e) ol[e] = __builtin_ldexpf(ol[e], sh);
        }
        m_run = mnew;
      }
      const float bias = 8.f - m_run;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const float c = ci[st >> 1];
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf((float)s[st][4 * i + 0], c, bias));
          const float p1 = __builtin_amdgcn_exp2f(fmaf((float)s[st][4 * i + 1], c, bias));
          const float p2 = __builtin_amdgcn_exp2f(fmaf((float)s[st][4 * i + 2], c, bias));
          const float p3 = __builtin_amdgcn_exp2f(fmaf((float)s[st][4 * i + 3], c, bias));
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
          x = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
          w[i] = (uint32_t)x;
        }
        pf[st] = make_uint4(w[0], w[1], w[2], w[3]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(pf[i].x), "v"(pf[i].y), "v"(pf[i].z), "v"(pf[i].w));
      asm volatile("" ::"v"(m_run));
      if constexpr (GRP == 0) __builtin_amdgcn_s_waitcnt(0xF70);   // this wave's V loads have landed
      phase_barrier();
    };

    if constexpr (GRP == 1) {
      dma_pair(jbeg, lds_k0);
      if (jbeg + 1 < jend) dma_pair(jbeg + 1, lds_k1);
      __builtin_amdgcn_s_waitcnt(0xF70);
    }
    __syncthreads();
    if constexpr (GRP == 1) phase_barrier();
    if constexpr (GRP == 0) dma_pair(jbeg, lds_v0);
    i32x16 s[4];
    compute_s(lds_k0, s);
    asm volatile("" ::"v"(s[0]), "v"(s[1]), "v"(s[2]), "v"(s[3]));
    phase_barrier();
    int jp = jbeg;
    for (; jp + 1 < jend; jp += 2) {
      phase_v(jp, s);
      phase_m(S0, jp, s);
      phase_v(jp + 1, s);
      phase_m(S1, jp + 1, s);
    }
    if (jp < jend) {
      phase_v(jp, s);
      phase_m(S0, jp, s);
    }
    if constexpr (GRP == 0) {
      __builtin_amdgcn_s_waitcnt(0xF70);
      phase_barrier();
    }

    // ---- finish: O = s_v * acc / ell; every row of the ones product holds the row sum
    const float* svp = a.sv + ((int64_t)b * a.H + h) * A8_DIM;
    if (slot >= 0) {   // a key range of a split-tail item: s_v * acc, running max and sum
      float* pb = a.part + (int64_t)slot * A8_PART_FLOATS;
      const int ql = wave * 32 + l32;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int d0 = dt * 32 + 8 * e4 + 4 * g;
          const float4 sv = *reinterpret_cast<const float4*>(svp + d0);
          *reinterpret_cast<float4*>(pb + ql * 128 + d0) =
              make_float4(o[dt][4 * e4] * sv.x, o[dt][4 * e4 + 1] * sv.y, o[dt][4 * e4 + 2] * sv.z,
                          o[dt][4 * e4 + 3] * sv.w);
        }
      if (g == 0) *reinterpret_cast<float2*>(pb + 256 * 128 + 2 * ql) = make_float2(m_run, ol[0]);
      return;
    }
    if (qi >= N) return;
    const float ell = ol[0];
    const float inv = 1.0f / ell;
    const bool is_cond = qi < n_cond;
    const int64_t row = is_cond ? b * n_cond + qi : b * n_vis + (qi - n_cond);
    void* obase = is_cond ? a.o[1] : a.o[0];
    const int64_t ooff = row * a.out_stride + (int64_t)h * A8_DIM;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d0 = dt * 32 + 8 * e4 + 4 * g;
        const float4 sv = *reinterpret_cast<const float4*>(svp + d0);
        const float v0 = o[dt][4 * e4 + 0] * sv.x * inv, v1 = o[dt][4 * e4 + 1] * sv.y * inv;
        const float v2 = o[dt][4 * e4 + 2] * sv.z * inv, v3 = o[dt][4 * e4 + 3] * sv.w * inv;
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
      if (g == 0) a.lse[((int64_t)b * a.H + h) * N + qi] = (m_run - 8.f + log2f(ell)) * 0.69314718055994530942f;
    }
  };
  if (wave >= 4) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 0>{});
}

// Split-tail items: per query, the `split` key ranges' results (s_v * acc_s relative to 2^(m_s
// - 8), sums l_s; the m_s are integers) combine as O = sum_s 2^(m_s - M) O_s / L, M = max_s
// m_s, L = sum_s 2^(m_s - M) l_s: every weight is an exact power of two, as in the rescale.
// One thread per query and four dims; 32 workgroups of 256 threads per item.  Calls that
// ask for the LSE are not split.
template <int OUT_DT>
__global__ __launch_bounds__(256) void joint_attn_8bit_merge_kernel(Attn8Args a) {
  const int r = blockIdx.x >> 5;
  const int t = (blockIdx.x & 31) * 256 + threadIdx.x;
  const int ql = t >> 5, d0 = (t & 31) * 4;
  int bh, qt;
  attn8_item(a, a.full + r, bh, qt);
  const int64_t qi = (int64_t)qt * A8_BM + ql;
  if (qi >= a.N) return;
  const float* pb = a.part + (int64_t)r * a.split * A8_PART_FLOATS;
  float mmax = -INFINITY;
  for (int sp = 0; sp < a.split; ++sp) mmax = fmaxf(mmax, pb[sp * A8_PART_FLOATS + 256 * 128 + 2 * ql]);
  float l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < a.split; ++sp) {
    const float* ps = pb + sp * A8_PART_FLOATS;
    const float w = __builtin_ldexpf(1.0f, (int)(ps[256 * 128 + 2 * ql] - mmax));
    l = fmaf(w, ps[256 * 128 + 2 * ql + 1], l);
    const float4 o = *reinterpret_cast<const float4*>(ps + ql * 128 + d0);
    acc[0] = fmaf(w, o.x, acc[0]); acc[1] = fmaf(w, o.y, acc[1]);
    acc[2] = fmaf(w, o.z, acc[2]); acc[3] = fmaf(w, o.w, acc[3]);
  }
  const float inv = 1.0f / l;
  const int h = bh % a.H;
  const int64_t b = bh / a.H;
  const int64_t n_cond = a.n_seg[1], n_vis = a.n_seg[0];
  const bool is_cond = qi < n_cond;
  const int64_t row = is_cond ? b * n_cond + qi : b * n_vis + (qi - n_cond);
  void* obase = is_cond ? a.o[1] : a.o[0];
  const int64_t off = row * a.out_stride + (int64_t)h * A8_DIM + d0;
  const float v0 = acc[0] * inv, v1 = acc[1] * inv, v2 = acc[2] * inv, v3 = acc[3] * inv;
  if constexpr (OUT_DT == MMDIT_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(obase) + off) = make_float4(v0, v1, v2, v3);
  } else if constexpr (OUT_DT == MMDIT_BF16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(obase) + off) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(obase) + off) = make_uint2(pack_f16x2(v0, v1), pack_f16x2(v2, v3));
  }
}

int launch_joint_attention_8bit(const mmdit_attn8_stream* const* seg, const int64_t* n, const float* v_scale,
                                int64_t B, int64_t H, float softmax_scale, void* o_vis, void* o_cond, int out_dtype,
                                int64_t out_stride, float* lse, hipStream_t stream, float* split_ws,
                                size_t split_ws_bytes) {
  const int64_t N = n[0] + n[1];
  if (B == 0 || H == 0 || N == 0) return MMDIT_OK;
  Attn8Args a{};
  for (int s = 0; s < 2; ++s) {
    if (n[s] == 0) continue;
    a.q8[s] = static_cast<const int8_t*>(seg[s]->q8);
    a.sq[s] = seg[s]->q_scale;
    a.k8[s] = static_cast<const int8_t*>(seg[s]->k8);
    a.sk[s] = seg[s]->k_scale;
    a.v8t[s] = static_cast<const uint8_t*>(seg[s]->v8t);
  }
  a.sv = v_scale;
  a.o[0] = o_vis; a.o[1] = o_cond;
  a.lse = lse;
  a.n_seg[0] = n[0]; a.n_seg[1] = n[1]; a.N = N;
  a.out_stride = out_stride;
  a.H = (int)H;
  a.nqt = (int)((N + A8_BM - 1) / A8_BM);
  a.scale_log2 = softmax_scale * 1.44269504088896340736f;
  const int64_t items = (int64_t)a.nqt * H * B;
  if (items > 0x7fffffff) return fail(MMDIT_ERR_SHAPE, "joint_attention_8bit: grid too large");
  const bool L = lse != nullptr;
  a.nbh = (int)(H * B);
  a.full = (int)items;
  a.split = 1;
  // Split tail (with a workspace and no LSE): when the items fill R < P workgroup slots of
  // the last round (P = the CU count, one workgroup per CU), cut each of those R items into
  // S = P / R key ranges (at most one per key tile), merged afterwards
  // key ranges are whole pairs of 64-key tiles (the kernel's phase)
  const int64_t npairs = ((n[0] + A8_BN - 1) / A8_BN + (n[1] + A8_BN - 1) / A8_BN + 1) / 2;
  const int64_t round = device_cu_count();
  if (split_ws && !L && items > round) {
    const int64_t R = items % round;
    int64_t S = R ? round / R : 0;
    if (S > npairs) S = npairs;
    if (R > 0 && S > (int64_t)(split_ws_bytes / ((size_t)R * A8_PART_FLOATS * 4))) S = (int64_t)(split_ws_bytes / ((size_t)R * A8_PART_FLOATS * 4));
    if (R > 0 && S >= 2 && (size_t)(R * S * A8_PART_FLOATS) * 4 <= split_ws_bytes) {
      a.full = (int)(items - R);
      a.split = (int)S;
      a.part = split_ws;
    }
  }
  const int tail = (int)(items - a.full);
  const dim3 grid((unsigned)(a.full + (int64_t)tail * a.split));
  const dim3 mgrid((unsigned)(tail * 32));
#define A8_GO(O, LS)                                                                            \
  do {                                                                                          \
    joint_attn_8bit_kernel<O, LS><<<grid, A8_THREADS, 0, stream>>>(a);                         \
    if constexpr (!LS) if (tail > 0) joint_attn_8bit_merge_kernel<O><<<mgrid, 256, 0, stream>>>(a); \
  } while (0)
  if (out_dtype == MMDIT_F32) { if (L) A8_GO(MMDIT_F32, true); else A8_GO(MMDIT_F32, false); }
  else if (out_dtype == MMDIT_BF16) { if (L) A8_GO(MMDIT_BF16, true); else A8_GO(MMDIT_BF16, false); }
  else if (out_dtype == MMDIT_F16) { if (L) A8_GO(MMDIT_F16, true); else A8_GO(MMDIT_F16, false); }
  else return fail(MMDIT_ERR_DTYPE, "joint_attention_8bit: bad out dtype");
#undef A8_GO
  return check_launch("joint_attention_8bit");
}

}  // namespace mmdit
