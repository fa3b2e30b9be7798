// Joint non-causal attention over [conditioning | visual] tokens, split back per stream.
//
// Vimoo 1.0 notes, section 2.2: the two streams' projected sequences are concatenated for
// one attention and the result is split back; the DiT attention is non-causal (Wan report
// reading guide).  Its cost is 4*N^2*D per head (Wan report, section 4.3.1), the dominant
// term of the block.  The concatenation is never materialised: key / query index j < n_cond
// reads the conditioning tensors, j >= n_cond the visual ones.
//
// 16-bit MFMA flash kernel (gfx950):
//   - workgroup = 8 wave64s = 256 queries of one (batch, head); each wave owns 32 queries and
//     the workgroup fills one CU (two waves per SIMD).
//   - The wave computes S^T = K Q^T with v_mfma_f32_32x32x16_{f16,bf16} (A = 32 keys x 16 dims
//     from LDS, B = the wave's Q held in registers for the whole kernel).  In the S^T
//     accumulator layout every lane holds one query (lane % 32) and 16 keys, so the online
//     softmax statistics are per-lane scalars and only a row max needs an exchange between
//     the two half-waves; the row sum is combined once at the end.
//   - P^T comes straight from those accumulators (rounded to f16) as the B operand of
//     O^T = V^T P^T; O^T accumulates 128 dims x 32 queries per wave in registers.  The V^T
//     operand is read from row-major V tiles with ds_read_b64_tr_b16.
//   - K and V tiles of 128 keys reach LDS by LDS-DMA (buffer loads straight into LDS, two
//     stages each, 128 KiB in all, XOR-swizzled chunks for conflict-free reads), issued in the
//     softmax phases so that the MFMA phases hold only MFMAs and their LDS operand reads.
//   - Two wave groups ping-pong: a wave alternates an MFMA-only phase (S of the next tile,
//     P V of this one: 64 MFMAs) and a VALU-only phase (exp2, row sums), one group
//     a phase behind the other, so on every SIMD the matrix pipe and the VALU work
//     concurrently; each phase ends with a workgroup barrier, whose pipeline fill and drain
//     a 128-key tile pays half as often as a 64-key one.
//   - exp2 with log2(e) * softmax_scale folded into Q; the S^T accumulators start from minus
//     the running max (a constant C operand of each chain's first MFMA).  The first tile of
//     a key range sets the running max exactly; after that a tile is weighed against the max
//     as it stands, and only when a lane's sum of the tile's weights passes 2^14 (which
//     bounds each weight) is the max raised to the tile's row max and the tile weighed again
//     (its S recomputed from the K tile still in LDS).  No row max is taken per tile: the
//     softmax phase is exponentials, packing and sums.
//   - Precision: S = Q K^T runs on the operand type of Q and K (f16 or bf16); P is rounded
//     to f16 (P lies in [0, 2^14], where f16 keeps 3 more mantissa bits than bf16) and PV
//     runs on f16 MFMA, so a bf16 V is converted to f16 after it is read from LDS.
//
// fp32 path: a plain wave-per-query VALU kernel with the same online softmax, used for the
// fp32 workload (small sizes).
#include <type_traits>

#include "common.h"

namespace mmdit {

constexpr int ATT_D = 128;
constexpr int ATT_BM = 256;                       // queries per workgroup (8 waves x 32)
constexpr int ATT_BN = 128;                       // keys per tile
constexpr int ATT_THREADS = 512;
constexpr int ATT_K_BYTES = ATT_BN * ATT_D * 2;   // 32 KiB
// A tile's weights are taken against the running max as it stands; only when one lane's sum
// of its weights in the tile (which bounds each of them, all being >= 0) passes this limit is
// the max raised to the tile's and the tile's weights taken again, so every f16 weight that
// reaches the P V product is at most 2^14.
constexpr float ATT_WEIGHT_SUM_LIMIT = 16384.0f;
#ifndef ATT_LDS_AHEAD
#define ATT_LDS_AHEAD 4                           // MFMAs between an LDS operand read and its use
#endif

struct AttnArgs {
  const uint16_t* q[2];   // [0] visual, [1] conditioning (segment order of the key loop)
  const uint16_t* k[2];
  const uint16_t* v[2];
  void* o[2];
  float* lse;
  int64_t n_seg[2];       // n_vis, n_cond
  int64_t N;
  int64_t in_stride, out_stride;
  int H;
  int nqt;
  float scale_log2;       // softmax_scale * log2(e)
  // Work items are (batch item x head, query tile) pairs, nbh * nqt of them.  Split tail:
  // workgroups [0, full) take items 0 .. full-1 over all keys; each of the remaining items
  // (fewer than one round of the chip) is cut into `split` key ranges taken by workgroups
  // full + ..., which leave f32 partial results in `part` for joint_attn_merge_kernel.
  // full == nbh * nqt: none.
  int nbh;
  int full;
  int split;
  float* part;
};

// one key range's partial result for one query tile: O (256 x 128 f32) then (m, l) per query
constexpr int64_t ATT_PART_FLOATS = 256 * 128 + 256 * 2;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

template <int DT>
__device__ __forceinline__ f32x16 mfma16(const uint4& a, const uint4& b, const f32x16& c) {
  if constexpr (DT == MMDIT_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Round two floats to f16 (nearest even); a single v_cvt_pk_f16_f32 on gfx950.
__device__ __forceinline__ uint32_t cvt_pk_f16(float lo, float hi) {
  const float2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, half2_t));
}


// Buffer descriptor over one (segment, batch item, head): rows of `stride` elements, 128
// valid elements in the last row.  Every read stays inside it: the partial last tile of a
// segment clamps its rows to the segment's last row.  The descriptor is built from
// readfirstlane'd words so it provably lives in SGPRs (a descriptor the compiler believes
// divergent costs a waterfall loop per load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seg_rsrc(const uint16_t* base, int64_t rows, int64_t stride) {
  const int64_t bytes = rows > 0 ? ((rows - 1) * stride + ATT_D) * 2 : 0;
  const uint64_t addr = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  const int num = __builtin_amdgcn_readfirstlane((int)bytes);
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, num, 0x00020000);
}

__device__ __forceinline__ float xhalf_max(float x) {   // max with the lane 32 apart
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint4 lds_read16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element (i % 4) of the
// 8-byte reads of lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ uint2 lds_read_tr(const uint8_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(const_cast<uint8_t*>(p)));
  return __builtin_bit_cast(uint2, r);
}

// (batch item x head, query tile) of work item i.  Items are dispatched round-robin over the
// 8 XCDs (i % 8), each with its own L2; when the (batch, head) count allows, XCD x takes whole
// heads x, x + 8, ... so that the 32 workgroups it runs at a time stream the same K and V
// through one L2.
__device__ __forceinline__ void attn_item(const AttnArgs& a, int i, int& bh, int& qt) {
  if ((a.nbh & 7) == 0) {
    const int j = i >> 3;
    bh = (i & 7) + 8 * (j / a.nqt);
    qt = j % a.nqt;
  } else {
    bh = i / a.nqt;
    qt = i % a.nqt;
  }
}

// Offset of an LDS object in the LDS aperture.  A DS instruction reaches 64 KiB past its
// address register through its immediate offset; the kernel's four 32 KiB stage buffers
// span 128 KiB, so reads of a buffer above the first 64 KiB take lane offsets biased by
// 64 KiB (kept opaque, so that the compiler folds only the buffer's remainder and the
// compile-time part of each read into the immediate).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Instruction order of an MFMA phase: 32 MFMAs of S^T (one K fragment read each), then 32 of
// O^T (two V^T fragment reads each), every LDS operand read ATT_LDS_AHEAD MFMAs ahead of its
// use.
constexpr int att_reads(int n) { return n < 32 ? 1 : n < 64 ? 2 : 0; }
constexpr int att_first_reads(int n = 0) { return n < ATT_LDS_AHEAD ? att_reads(n) + att_first_reads(n + 1) : 0; }

template <int I = 0>
__device__ __forceinline__ void m_phase_schedule() {
  if constexpr (I == 0) __builtin_amdgcn_sched_group_barrier(0x100, att_first_reads(), 1);
  if constexpr (I < 64) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    if constexpr (att_reads(I + ATT_LDS_AHEAD) > 0)
      __builtin_amdgcn_sched_group_barrier(0x100, att_reads(I + ATT_LDS_AHEAD), 1);
    m_phase_schedule<I + 1>();
  }
}

template <int QK_DT, int V_DT, int OUT_DT, bool LSE>
__global__ __launch_bounds__(ATT_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void joint_attn_mfma_kernel(AttnArgs a) {
  // LDS: two K stages and two V stages, 32 KiB each (128 keys of 256-byte rows).  Four
  // distinct objects, always addressed with a compile-time stage index, so the wait-count
  // pass can tell an LDS-DMA into one stage from reads of another and does not stall the
  // reads on the prefetch in flight.
  __shared__ __attribute__((aligned(16))) uint8_t lds_k0[ATT_K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_k1[ATT_K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v0[ATT_K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v1[ATT_K_BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;   // wave index in an SGPR
  const int l32 = lane & 31, g = lane >> 5;
  int qt, bh;
  int slot = -1;   // a split-tail workgroup's partial-result slot
  {
    int item = blockIdx.x;
    if (item >= a.full) {
      slot = item - a.full;
      item = a.full + slot / a.split;
    }
    attn_item(a, item, bh, qt);
  }
  const int h = bh % a.H;
  const int64_t b = bh / a.H;
  const int64_t N = a.N;
  const int64_t n_vis = a.n_seg[0], n_cond = a.n_seg[1];
  const int stride = (int)a.in_stride;
  const float c = a.scale_log2;

  // ---- this lane's query row (queries in [cond | vis] order): the B operand of S^T
  const int64_t qi = (int64_t)qt * ATT_BM + wave * 32 + l32;
  uint4 qf[8];
  if (qi < N) {
    const uint16_t* qp = qi < n_cond ? a.q[1] + (b * n_cond + qi) * a.in_stride + h * ATT_D
                                     : a.q[0] + (b * n_vis + (qi - n_cond)) * a.in_stride + h * ATT_D;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const uint4*>(qp + ks * 16 + g * 8);
  } else {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = make_uint4(0, 0, 0, 0);
  }
  // f16 Q is scaled once by softmax_scale * log2(e) (rounded to f16 again), so S comes out of
  // the MFMA in log2 units and the exponential needs no multiply; a bf16 Q would lose 3 more
  // bits in that rounding, so there the accumulator is scaled at the exponential instead.
  constexpr bool PRESCALE = QK_DT == MMDIT_F16;
  const float ce = PRESCALE ? 1.0f : c;          // log2 units per accumulator unit
  const float inv_ce = PRESCALE ? 1.0f : 1.0f / c;
  if constexpr (PRESCALE) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint32_t* w = reinterpret_cast<uint32_t*>(&qf[ks]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half2_t hq = __builtin_bit_cast(half2_t, w[i]);
        w[i] = cvt_pk_f16((float)hq[0] * c, (float)hq[1] * c);
      }
    }
  }
  const int t_vis = (int)((n_vis + ATT_BN - 1) / ATT_BN);
  const int ntiles = t_vis + (int)((n_cond + ATT_BN - 1) / ATT_BN);
  // this workgroup's key tiles [jbeg, jend): all of them, or one range of a split-tail item
  int jbeg = 0, jend = ntiles;
  if (slot >= 0) {
    const int sp = slot % a.split;
    jbeg = (int)((int64_t)ntiles * sp / a.split);
    jend = (int)((int64_t)ntiles * (sp + 1) / a.split);
  }
  auto tile_seg = [&](int jt, int& sg, int& t) { sg = jt < t_vis ? 0 : 1; t = sg ? jt - t_vis : jt; };
  auto tile_rows = [&](int sg, int t) {
    const int64_t r = a.n_seg[sg] - (int64_t)t * ATT_BN;
    return r < ATT_BN ? (int)r : ATT_BN;
  };
  auto kbuf = [&](auto stage) -> uint8_t* { if constexpr (decltype(stage)::value == 0) return lds_k0; else return lds_k1; };
  auto vbuf = [&](auto stage) -> uint8_t* { if constexpr (decltype(stage)::value == 0) return lds_v0; else return lds_v1; };
  constexpr std::integral_constant<int, 0> S0{};
  constexpr std::integral_constant<int, 1> S1{};

  // ---- per-lane LDS read offsets (each biased by 64 KiB for a stage buffer above 64 KiB)
  // S^T A operand: key = 32*st + l32, logical chunk 2*ks + g, physical chunk ^ (key % 16)
  int k_rd[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) k_rd[ks] = l32 * 256 + (((2 * ks + g) ^ (l32 & 15)) << 4);
  // O^T A operand (dims x keys) through transposed reads: 16-lane group G = lane / 16 with
  // k-group g = G / 2 and dim half = G % 2; lane j of the group reads key 4*g + j/4 (+16 s
  // + 8 r) at dims 32*dt + 16*half + 4*(j % 4), and receives 4 consecutive keys of dim
  // 32*dt + 16*half + j.  Physical chunk = logical chunk ^ 4*(key % 4), key % 4 = j / 4.
  int v_rd[4];
  {
    const int G = lane >> 4, j = lane & 15;
    const int gg = G >> 1, half = G & 1;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int chunk = (4 * dt + 2 * half + ((j & 3) >> 1)) ^ ((j >> 2) << 2);
      v_rd[dt] = (4 * gg + (j >> 2)) * 256 + chunk * 16 + (j & 1) * 8;
    }
  }
  // (the same bias serves both stages of K and of V: a stage placed elsewhere still reads the
  // right bytes, its reads just do not fold the whole offset into the immediate)
  const uint32_t khi = lds_offset(lds_k0) & 0xFFFF0000u, vhi = lds_offset(lds_v0) & 0xFFFF0000u;
  if (khi) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) { k_rd[ks] += (int)khi; asm volatile("" : "+v"(k_rd[ks])); }
  }
  if (vhi) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) { v_rd[dt] += (int)vhi; asm volatile("" : "+v"(v_rd[dt])); }
  }

  // S^T of one tile: four independent 32-key accumulator chains, interleaved so that
  // consecutive MFMAs never wait on each other's result; the first MFMA of each chain takes
  // `base` (minus the running max in accumulator units, in every element) as its C operand,
  // so the product comes out relative to the running max with no per-tile initialisation
  auto compute_s = [&](const uint8_t* kb, f32x16 (&s)[4], const f32x16& base) {
    kb -= khi;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int st = 0; st < 4; ++st)
        s[st] = mfma16<QK_DT>(lds_read16(kb + st * 8192 + k_rd[ks]), qf[ks], ks == 0 ? base : s[st]);
  };
  auto row_max = [&](const f32x16 (&s)[4]) {   // max over this query's 128 keys (both half-waves)
    float m4[4];                                 // four independent chains, then a short tree
#pragma unroll
    for (int k = 0; k < 4; ++k) m4[k] = fmaxf(fmaxf(s[0][k], s[1][k]), fmaxf(s[2][k], s[3][k]));
#pragma unroll
    for (int e = 4; e < 16; e += 4)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        m4[k] = fmaxf(fmaxf(m4[k], fmaxf(s[0][e + k], s[1][e + k])), fmaxf(s[2][e + k], s[3][e + k]));
    return xhalf_max(fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3])));
  };
  auto v_frag = [&](const uint8_t* vb, int dt, int ks) {
    const uint8_t* p = vb - vhi + v_rd[dt] + ks * 4096;
    const uint2 lo = lds_read_tr(p), hi = lds_read_tr(p + 2048);
    uint4 f = make_uint4(lo.x, lo.y, hi.x, hi.y);
    if constexpr (V_DT == MMDIT_BF16) {
      f.x = cvt_pk_f16(lo_bf16(f.x), hi_bf16(f.x)); f.y = cvt_pk_f16(lo_bf16(f.y), hi_bf16(f.y));
      f.z = cvt_pk_f16(lo_bf16(f.z), hi_bf16(f.z)); f.w = cvt_pk_f16(lo_bf16(f.w), hi_bf16(f.w));
    }
    return f;
  };
  // Phase barrier: only orders LDS use between the waves; no memory-fence waits.  Every LDS
  // read before it has been consumed (waited for) by an MFMA of the same phase.
  auto phase_barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // ---- Ping-pong of two wave groups.  Waves 0-3 (group 0) and 4-7 (group 1) each hold one
  // wave on every SIMD.  Each wave alternates two phases per 128-key tile:
  //   M(j): S_{j+1} = K_{j+1} Q^T and O^T += V_j^T P_j^T -- MFMA and LDS reads only;
  //   V(j): mask and P_j = exp2(S_j - m), with the running max raised only when a weight
  //         would pass 2^14 -- VALU only.
  // One S accumulator set serves every tile: V(j) consumes S_j before M(j) writes S_{j+1}.
  // Group 1 runs one phase behind group 0 and every phase ends with a workgroup barrier, so
  // on each SIMD one wave keeps the matrix pipe busy while the other runs the softmax.  A
  // tile of 128 keys gives each barrier 64 MFMAs: the pipeline fill and drain around a
  // barrier is paid once per 128 keys.
  // Tiles move by LDS-DMA, issued in the softmax phases (the MFMA phases, which set the pace,
  // then issue no vector-memory instructions: 1.5 % faster than loads among their first
  // MFMAs): group 0 loads V_j at the start of its V(j) and waits for it at that phase's end;
  // group 1 loads K_{j+2} at the end of its V(j) and waits at the end of its M(j).
  auto run = [&](auto grp_c) {
    constexpr int GRP = decltype(grp_c)::value;
    const int wg = wave & 3;   // this wave's index inside its group
    // this group's tensor, one (batch item, head) slice per segment: base and byte extent
    const uint16_t* seg_base[2];
    int64_t seg_bytes[2];
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      const uint16_t* base = GRP ? a.k[sg] : a.v[sg];
      seg_base[sg] = base ? base + (b * a.n_seg[sg]) * a.in_stride + h * ATT_D : (GRP ? a.k[0] : a.v[0]);
      seg_bytes[sg] = a.n_seg[sg] > 0 ? ((a.n_seg[sg] - 1) * a.in_stride + ATT_D) * 2 : 0;
    }
    // DMA i of this wave fills tile rows 32*wg + 4*i .. +3 and, 16 rows further on (scalar
    // offset 16 rows, LDS 4 KiB further), 32*wg + 16 + 4*i .. +3, in lane order (lane l -> row
    // + l/16, physical 16-byte chunk l % 16).  K chunks are XOR-swizzled by (row % 16) for the
    // column reads of S^T, V chunks by 4*(row % 4) for the transposed reads of O^T (rows 16
    // apart share the swizzle); each lane loads the logical chunk that belongs at its
    // physical slot.  The descriptor starts at the tile and ends with the segment, so rows
    // past the segment's end fail its range check and arrive as zeros.  Each half's four
    // loads share one LDS base (M0): the immediate offset i * 1024 moves both the LDS
    // destination and the source, and is taken back out of the per-lane offset, which is
    // therefore fixed for the whole loop.
    int off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 32 * wg + 4 * i + (lane >> 4);
      const int chunk = GRP ? ((lane & 15) ^ (row & 15)) : ((lane & 15) ^ ((row & 3) << 2));
      off[i] = row * stride * 2 + chunk * 16 - i * 1024;
    }
    const int half_soff = 16 * stride * 2;
    auto dma_tile = [&](int jt, uint8_t* dst) {
      int sg, t;
      tile_seg(jt, sg, t);
      const int64_t tile_elems = (int64_t)t * ATT_BN * stride;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>((sg ? seg_base[1] : seg_base[0]) + tile_elems), (short)0,
          (int)((sg ? seg_bytes[1] : seg_bytes[0]) - tile_elems * 2), 0x00020000);
      auto* l0 = (__attribute__((address_space(3))) void*)(dst + wg * 8192);
      auto* l1 = (__attribute__((address_space(3))) void*)(dst + wg * 8192 + 4096);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l0, 16, off[0], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l0, 16, off[1], 0, 1024, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l0, 16, off[2], 0, 2048, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l0, 16, off[3], 0, 3072, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l1, 16, off[0], half_soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l1, 16, off[1], half_soff, 1024, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l1, 16, off[2], half_soff, 2048, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, l1, 16, off[3], half_soff, 3072, 0);
    };

    f32x16 o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[dt][e] = 0.f;
    float m_run = 0.f;         // running max of the logits (log2 units), possibly stale by < 14;
                               // S accumulators hold logit - m_run in accumulator units
    float l_run = 0.f;         // this lane's partial sum of the probabilities
    uint4 pf[8];               // P_j rounded to f16, the B operand of O^T
    f32x16 mneg;               // -m_run in accumulator units: the C operand that starts S^T
#pragma unroll
    for (int e = 0; e < 16; ++e) mneg[e] = 0.f;
    asm volatile("" : "+v"(mneg));   // kept in registers, not rematerialised at each use

    // M(j): S_{j+1} (past the last tile from a stale stage; never used) and O^T += V_j^T P_j^T
    auto phase_m = [&](auto cur_c, int jt, f32x16 (&s)[4]) {
      constexpr int CUR = decltype(cur_c)::value;   // jt % 2
      constexpr std::integral_constant<int, CUR> cur{};
      constexpr std::integral_constant<int, CUR ^ 1> oth{};
      compute_s(kbuf(oth), s, mneg);
      const uint8_t* vb = vbuf(cur);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] = mfma16<MMDIT_F16>(v_frag(vb, dt, ks), pf[ks], o[dt]);
      m_phase_schedule();
      // the products must issue in this phase: pin their results ahead of the barrier (the
      // compiler would otherwise sink MFMAs into the softmax phase that first reads them)
      asm volatile("" ::"v"(s[0]), "v"(s[1]), "v"(s[2]), "v"(s[3]));
      asm volatile("" ::"v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]));
      if constexpr (GRP == 1) __builtin_amdgcn_s_waitcnt(0xF70);   // this wave's K loads have landed
      phase_barrier();
    };
    // V(j): softmax of S_j into P_j.  K_j is still in its stage here: group 1 refills that stage
    // with K_{j+2} only at the end of its own V(j), after every reader of K_j (S_j in both
    // groups' M(j-1), its recompute in group 0's V(j) and in this phase).  Group 0 loads V_j
    // into the stage that held V_{j-2}, last read in both groups' M(j-2).
    auto phase_v = [&](auto cur_c, int jt, f32x16 (&s)[4]) {
      constexpr std::integral_constant<int, decltype(cur_c)::value> cur{};
      if constexpr (GRP == 0) dma_tile(jt, vbuf(cur));
      auto mask_tail = [&]() {  // keys past the end of their segment (a segment's partial last tile)
        int sg, t;
        tile_seg(jt, sg, t);
        const int valid = tile_rows(sg, t);
        if (valid < ATT_BN) {
          // element e of chain st holds key 32 st + 8 (e / 4) + 4 g + e % 4: an arithmetic
          // shift turns (valid - 1 - key) into an all-ones mask for keys past the end, and a
          // bitfield insert puts -inf there (no per-element compare results to hold)
          const int vl = valid - 1 - 4 * g;
#pragma unroll
          for (int st = 0; st < 4; ++st)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const uint32_t m = (uint32_t)((vl - (st * 32 + 8 * (e >> 2) + (e & 3))) >> 31);
              s[st][e] = __uint_as_float((0xFF800000u & m) | (__float_as_uint(s[st][e]) & ~m));
            }
        }
      };
      mask_tail();
      // S holds logit - m_run.  raise_max moves the running max up to this tile's row max (the
      // first tile of a range sets it exactly), rescaling O and l by an exact 2^-delta.
      auto raise_max = [&](bool first) {
        const float dl = row_max(s) * ce;
        const float delta = first ? dl : fmaxf(dl, 0.f);
        if (!first) {
          const float alpha = __builtin_amdgcn_exp2f(-delta);
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[dt][e] *= alpha;
        }
        m_run += delta;
        const float d = delta * inv_ce;
#pragma unroll
        for (int st = 0; st < 4; ++st)
#pragma unroll
          for (int e = 0; e < 16; ++e) s[st][e] -= d;
        const float mb = -m_run * inv_ce;
#pragma unroll
        for (int e = 0; e < 16; ++e) mneg[e] = mb;
        asm volatile("" : "+v"(mneg));
      };
      // P = 2^S into the f16 B operands of the P V product; returns this lane's sum of P
      auto weights = [&]() {
        float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float p0 = __builtin_amdgcn_exp2f(PRESCALE ? s[st][8 * hh + 2 * i] : s[st][8 * hh + 2 * i] * ce);
              const float p1 = __builtin_amdgcn_exp2f(PRESCALE ? s[st][8 * hh + 2 * i + 1] : s[st][8 * hh + 2 * i + 1] * ce);
              w[i] = cvt_pk_f16(p0, p1);
              // plain f32 adds in four chains: the dot-product path (v_dot2) shares the matrix
              // pipe and stalls behind the other wave's MFMAs
              ls[(i & 1) * 2] += p0;
              ls[(i & 1) * 2 + 1] += p1;
            }
            pf[st * 2 + hh] = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
        return (ls[0] + ls[1]) + (ls[2] + ls[3]);
      };
      if (jt == jbeg) raise_max(true);
      float lt = weights();
      if (jt != jbeg && __any(lt > ATT_WEIGHT_SUM_LIMIT)) {
        // rare (a logit far above the running max): S_j again from K_j with the same C operand,
        // so bit-identical, rather than holding S beside P through the exponentials
        compute_s(kbuf(cur), s, mneg);
        mask_tail();
        raise_max(false);
        lt = weights();
      }
      l_run += lt;
      // pin P, l and m: this VALU work belongs to this phase, not the next M phase
#pragma unroll
      for (int i = 0; i < 8; ++i) asm volatile("" ::"v"(pf[i].x), "v"(pf[i].y), "v"(pf[i].z), "v"(pf[i].w));
      asm volatile("" ::"v"(l_run), "v"(m_run), "v"(mneg));
      // past the last tile: a reload of the last one into a stage nobody reads again
      if constexpr (GRP == 1) dma_tile(jt + 2 < jend ? jt + 2 : jend - 1, kbuf(cur));
      if constexpr (GRP == 0) __builtin_amdgcn_s_waitcnt(0xF70);   // this wave's V loads have landed
      phase_barrier();
    };

    // prologue: group 1 loads K_0 and K_1; S_0 is an M phase of its own
    if constexpr (GRP == 1) {
      dma_tile(jbeg, lds_k0);
      if (jbeg + 1 < jend) dma_tile(jbeg + 1, lds_k1);
      __builtin_amdgcn_s_waitcnt(0xF70);
    }
    __syncthreads();
    if constexpr (GRP == 1) phase_barrier();   // group 1 runs one phase behind
    f32x16 s[4];
    compute_s(lds_k0, s, mneg);
    asm volatile("" ::"v"(s[0]), "v"(s[1]), "v"(s[2]), "v"(s[3]));
    phase_barrier();
    int jt = jbeg;
    for (; jt + 1 < jend; jt += 2) {
      phase_v(S0, jt, s);
      phase_m(S0, jt, s);
      phase_v(S1, jt + 1, s);
      phase_m(S1, jt + 1, s);
    }
    if (jt < jend) {
      phase_v(S0, jt, s);
      phase_m(S0, jt, s);
    }
    if constexpr (GRP == 0) phase_barrier();   // match group 1's extra barrier of the prologue

    // ---- finish: combine the two half-wave partial sums, normalise, store
    const float l_tot = xhalf_sum(l_run);
    if (slot >= 0) {   // a key range of a split-tail item: unnormalised O, running max and sum
      float* pb = a.part + (int64_t)slot * ATT_PART_FLOATS;
      const int ql = wave * 32 + l32;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          *reinterpret_cast<float4*>(pb + ql * 128 + dt * 32 + 8 * e4 + 4 * g) =
              make_float4(o[dt][4 * e4], o[dt][4 * e4 + 1], o[dt][4 * e4 + 2], o[dt][4 * e4 + 3]);
      if (g == 0) *reinterpret_cast<float2*>(pb + 256 * 128 + 2 * ql) = make_float2(m_run, l_tot);
      return;
    }
    if (qi >= N) return;
    const float inv = 1.0f / l_tot;
    const bool is_cond = qi < n_cond;
    const int64_t row = is_cond ? b * n_cond + qi : b * n_vis + (qi - n_cond);
    void* obase = is_cond ? a.o[1] : a.o[0];
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
              make_uint2(cvt_pk_f16(v0, v1), cvt_pk_f16(v2, v3));
        }
      }
    if constexpr (LSE) {
      if (g == 0) a.lse[(b * a.H + h) * N + qi] = (m_run + log2f(l_tot)) * 0.69314718055994530942f;
    }
  };
  if (wave >= 4) run(std::integral_constant<int, 1>{});
  else run(std::integral_constant<int, 0>{});
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

// Split-tail items: per query, the `split` key ranges' results (O_s relative to their own
// running max m_s, sums l_s, log2 units) combine as O = sum_s 2^(m_s - M) O_s / L with
// M = max_s m_s and L = sum_s 2^(m_s - M) l_s (calls that ask for the LSE are not split).
// One thread per query and four dims; 32 workgroups of 256 threads per item.
template <int OUT_DT>
__global__ __launch_bounds__(256) void joint_attn_merge_kernel(AttnArgs a) {
  const int r = blockIdx.x >> 5;                       // tail item
  const int t = (blockIdx.x & 31) * 256 + threadIdx.x;
  const int ql = t >> 5, d0 = (t & 31) * 4;            // query in the tile, first dim
  int bh, qt;
  attn_item(a, a.full + r, bh, qt);
  const int64_t qi = (int64_t)qt * ATT_BM + ql;
  if (qi >= a.N) return;
  const float* pb = a.part + (int64_t)r * a.split * ATT_PART_FLOATS;
  float mmax = -INFINITY;
  for (int sp = 0; sp < a.split; ++sp) mmax = fmaxf(mmax, pb[sp * ATT_PART_FLOATS + 256 * 128 + 2 * ql]);
  float l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < a.split; ++sp) {
    const float* ps = pb + sp * ATT_PART_FLOATS;
    const float w = exp2f(ps[256 * 128 + 2 * ql] - mmax);
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
  const int64_t off = row * a.out_stride + (int64_t)h * ATT_D + d0;
  const float v0 = acc[0] * inv, v1 = acc[1] * inv, v2 = acc[2] * inv, v3 = acc[3] * inv;
  if constexpr (OUT_DT == MMDIT_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(obase) + off) = make_float4(v0, v1, v2, v3);
  } else if constexpr (OUT_DT == MMDIT_BF16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(obase) + off) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
  } else {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(obase) + off) = make_uint2(cvt_pk_f16(v0, v1), cvt_pk_f16(v2, v3));
  }
}

template <int QK, int V>
static int attn_go(const AttnArgs& a, dim3 grid, int out_dtype, bool has_lse, hipStream_t stream) {
  const int tail = a.nbh * a.nqt - a.full;   // split-tail items
  const dim3 mgrid((unsigned)(tail * 32));
#define ATT_GO(O, L)                                                                        \
  do {                                                                                      \
    joint_attn_mfma_kernel<QK, V, O, L><<<grid, ATT_THREADS, 0, stream>>>(a);              \
    if constexpr (!L) if (tail > 0) joint_attn_merge_kernel<O><<<mgrid, 256, 0, stream>>>(a);  \
  } while (0)
  if (out_dtype == MMDIT_F32) { if (has_lse) ATT_GO(MMDIT_F32, true); else ATT_GO(MMDIT_F32, false); }
  else if (out_dtype == MMDIT_BF16) { if (has_lse) ATT_GO(MMDIT_BF16, true); else ATT_GO(MMDIT_BF16, false); }
  else if (out_dtype == MMDIT_F16) { if (has_lse) ATT_GO(MMDIT_F16, true); else ATT_GO(MMDIT_F16, false); }
  else return fail(MMDIT_ERR_DTYPE, "joint_attention: bad out dtype");
#undef ATT_GO
  return check_launch("joint_attention");
}

size_t joint_attention_split_bytes(int64_t n_vis, int64_t n_cond, int64_t B, int64_t H, int qk_dtype, bool has_lse) {
  const int64_t N = n_vis + n_cond;
  if (qk_dtype == MMDIT_F32 || has_lse || B < 1 || H < 1 || n_vis < 0 || n_cond < 0 || N < 1) return 0;
  const int64_t items = ((N + ATT_BM - 1) / ATT_BM) * H * B;
  const int64_t round = device_cu_count();
  if (items <= round) return 0;
  const int64_t R = items % round;
  if (R == 0) return 0;
  const int64_t ntiles = (n_vis + ATT_BN - 1) / ATT_BN + (n_cond + ATT_BN - 1) / ATT_BN;
  int64_t S = round / R;
  if (S > ntiles) S = ntiles;
  return S >= 2 ? (size_t)(R * S * ATT_PART_FLOATS) * 4 : 0;
}

int launch_joint_attention(const void* q_vis, const void* k_vis, const void* v_vis, int64_t n_vis,
                           const void* q_cond, const void* k_cond, const void* v_cond,
                           int64_t n_cond, int qk_dtype, int v_dtype, int64_t in_stride, int64_t B, int64_t H,
                           float softmax_scale, void* o_vis, void* o_cond, int out_dtype,
                           int64_t out_stride, float* lse, hipStream_t stream, float* split_ws,
                           size_t split_ws_bytes) {
  const int64_t N = n_vis + n_cond;
  if (B == 0 || H == 0 || N == 0) return MMDIT_OK;
  const bool has_lse = lse != nullptr;
  if (qk_dtype != MMDIT_F32) {
    // the kernel addresses each (segment, batch item, head) through a 32-bit buffer range
    if (((n_vis > 0 ? n_vis - 1 : 0) * in_stride + 128) * 2 >= (int64_t)1 << 31 ||
        ((n_cond > 0 ? n_cond - 1 : 0) * in_stride + 128) * 2 >= (int64_t)1 << 31)
      return fail(MMDIT_ERR_SHAPE, "joint_attention: one stream spans 2 GiB or more per batch item");
    AttnArgs a{};
    a.q[0] = static_cast<const uint16_t*>(q_vis); a.q[1] = static_cast<const uint16_t*>(q_cond);
    a.k[0] = static_cast<const uint16_t*>(k_vis); a.k[1] = static_cast<const uint16_t*>(k_cond);
    a.v[0] = static_cast<const uint16_t*>(v_vis); a.v[1] = static_cast<const uint16_t*>(v_cond);
    a.o[0] = o_vis; a.o[1] = o_cond;
    a.lse = lse;
    a.n_seg[0] = n_vis; a.n_seg[1] = n_cond; a.N = N;
    a.in_stride = in_stride; a.out_stride = out_stride;
    a.H = (int)H;
    a.nqt = (int)((N + ATT_BM - 1) / ATT_BM);
    a.scale_log2 = softmax_scale * 1.44269504088896340736f;
    const int64_t items = (int64_t)a.nqt * H * B;
    if (items > 0x7fffffff) return fail(MMDIT_ERR_SHAPE, "joint_attention: grid too large");
    a.nbh = (int)(H * B);
    a.full = (int)items;
    a.split = 1;
    // Split tail: when the items fill R < P workgroup slots of the last round (P = the CU
    // count, one workgroup per CU), cut each of those R items into S = P / R key ranges (at
    // most one per key tile) so that the last round runs on (nearly) every CU instead of R of
    // them; a merge kernel combines them.
    const int64_t ntiles = (n_vis + ATT_BN - 1) / ATT_BN + (n_cond + ATT_BN - 1) / ATT_BN;
    const int64_t round = device_cu_count();
    if (split_ws && !has_lse && items > round) {
      const int64_t R = items % round;
      int64_t S = R ? round / R : 0;
      if (S > ntiles) S = ntiles;
      if (R > 0 && S > (int64_t)(split_ws_bytes / ((size_t)R * ATT_PART_FLOATS * 4))) S = (int64_t)(split_ws_bytes / ((size_t)R * ATT_PART_FLOATS * 4));
      if (R > 0 && S >= 2 && (size_t)(R * S * ATT_PART_FLOATS) * 4 <= split_ws_bytes) {
        a.full = (int)(items - R);
        a.split = (int)S;
        a.part = split_ws;
      }
    }
    const int64_t blocks = a.full + (items - a.full) * a.split;
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
