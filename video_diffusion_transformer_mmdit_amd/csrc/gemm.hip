// y = epilogue(x W^T + bias): the per-stream projections of the MMDiT block (QKV, output,
// FFN up with GELU, FFN down with the gated residual), Vimoo 1.0 notes section 2.2; their
// cost is the linear term of the Wan report's workload model (section 4.3.1).  The same
// kernel runs the Lite model's 2x2 hidden-space merge and unpatchify (section 2.4), with the
// neighbour gather folded into the x loads and the scatter back to the grid into the stores.
//
// gfx950 design (two kernels share the tile, fragment layout, tile order and epilogue:
// gemm_k64_kernel for 16-bit operands in every layout, gemm_fp8_kernel for FP8 operands):
//   - 256 x 256 output tile per workgroup of 8 wave64s, two per SIMD, arranged 2 (M) x 4
//     (N), each owning 128 x 64 outputs = 4 x 2 tiles of 32 x 32 MFMAs (128 accumulator
//     registers, so two waves fit a SIMD and cover each other's fragment-read waits).  The
//     MFMA computes C^T (A operand = W rows, B operand = x rows), so every lane ends up
//     holding four consecutive output columns of one row, 32 rows apart from its neighbours'.
//   - x and W tiles are K-contiguous in LDS, so both MFMA operands are plain 16-byte LDS
//     reads, and move by LDS-DMA (buffer loads straight into LDS) issued between the MFMAs.
//     16-bit: two stages of K = 64 (rows of 128 bytes), one barrier per stage, the next
//     stage's loads in two fenced groups.  FP8: four stages of 64 bytes per row, the DMA
//     three stages ahead.  Stage buffers are distinct LDS objects addressed with compile-time
//     indices, and the DMA destinations pass through an opaque register copy, so the
//     compiler's wait-count pass leaves every wait to the explicit per-stage ones.
//   - 16-byte LDS chunks are XOR-swizzled by row so that the 16 rows a 16-lane group of a
//     fragment read touches fall on distinct bank groups; a DMA writes 16 bytes per lane in
//     lane order, so each lane loads the logical chunk that belongs at its physical slot.
//     Rows past the end of x or W fail the buffer descriptor's range check and arrive as
//     zeros.
//   - Tiles are renumbered so that each XCD (workgroups go round-robin over the 8 XCDs) owns
//     a contiguous run of tiles, and runs are rastered in bands of 4 M-tiles (2 at K >= 8192),
//     keeping the x and W panels that concurrent workgroups of one XCD share inside its L2.
//   - The epilogue restages each wave's block through LDS (free after the last stage) and
//     applies the FP8 scales, bias, GELU or the gated residual along rows, before the only
//     store of y.
//   - A launch whose last round would leave CUs idle cuts that round's tiles into K ranges
//     (split tail) and sums them in a small elementwise kernel that applies the epilogue.
#include <type_traits>

#include "common.h"

namespace mmdit {

constexpr int GBM = 256, GBN = 256, GBK = 32;
constexpr int GTHREADS = 256;
constexpr int G_TILE_BYTES = 256 * GBK * 2;   // one operand tile of one stage: 16 KiB
constexpr size_t G_PART_BYTES = 256 * 256 * 4;   // f32 partial sums of one tile

struct GemmArgs {
  GemmProblem p[2];
  int64_t tiles0;    // tiles of problem 0
  int64_t tiles;     // total tiles
  // Split tail: workgroups [0, full) take one whole tile each; the remaining tiles (fewer than
  // one round of the chip) are each cut into `split` K ranges taken by workgroups full + ...,
  // which leave f32 partial sums in `part` for gemm_split_finish_kernel.  full == tiles: none.
  int64_t full;
  int split;
  float* part;
  int64_t N, K;
  // M-tiles per raster band: 4 (measured ~1 % faster than 2, 8 or 16 at K = 3072), 2 at
  // K >= 8192 (FFN down 1.7 %, its FP8 form in the 8-bit block 3 %, the Lite merge 3 % faster
  // than with 4)
  int group_m;
  // 2x2 spatial regrouping (GEMM_GATHER_X / GEMM_SCATTER_Y): hidden width C, full grid
  // width W, merged grid width W/2 and merged tokens per frame (H/2)(W/2)
  int c, w, w2, hw2;
};

// Row of the full (T, H, W) token grid holding the top-left neighbour of merged token m
// (frames of all batch items follow one another, so batch and time fold into one index).
__device__ __forceinline__ int merged_row0(int m, const GemmArgs& a) {
  const int f = m / a.hw2, rem = m - f * a.hw2;
  const int i = rem / a.w2, j = rem - i * a.w2;
  return f * 4 * a.hw2 + 2 * i * a.w + 2 * j;
}

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// FP8 E4M3 x E4M3, 32 x 32 x 64, unit block scales (the E8M0 exponent 127 is 2^0); each
// operand is 32 bytes per lane, passed as two 16-byte halves.
__device__ __forceinline__ f32x16 mfma_fp8(const uint4& a0, const uint4& a1, const uint4& b0, const uint4& b1,
                                           const f32x16& c) {
  const i32x8 a = __builtin_shufflevector(__builtin_bit_cast(i32x4, a0), __builtin_bit_cast(i32x4, a1), 0, 1, 2, 3, 4, 5, 6, 7);
  const i32x8 b = __builtin_shufflevector(__builtin_bit_cast(i32x4, b0), __builtin_bit_cast(i32x4, b1), 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int IN_DT>
__device__ __forceinline__ f32x16 mfma32(const uint4& a, const uint4& b, const f32x16& c) {
  if constexpr (IN_DT == MMDIT_BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                 __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// erf by the rational approximation of Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (absolute error at most 1.5e-7):
//   erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),  t = 1 / (1 + p x),
// for x >= 0, extended to x < 0 by symmetry.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
  float q = fmaf(1.061405429f, t, -1.453152027f);
  q = fmaf(q, t, 1.421413741f);
  q = fmaf(q, t, -0.284496736f);
  q = fmaf(q, t, 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(-(ax * ax) * 1.44269504088896340736f);
  return copysignf(fmaf(-(q * t), e, 1.0f), x);
}

__device__ __forceinline__ float gelu_erf(float v) {
  return 0.5f * v * (1.0f + erf_as(v * 0.70710678118654752440f));
}

// Four consecutive elements of dtype DT (0 f32, 1 bf16, 2 f16) as floats, and back.
template <int DT>
__device__ __forceinline__ void load4(const void* base, int64_t idx, float (&v)[4]) {
  if constexpr (DT == MMDIT_F32) {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    if constexpr (DT == MMDIT_BF16) {
      v[0] = lo_bf16(w.x); v[1] = hi_bf16(w.x); v[2] = lo_bf16(w.y); v[3] = hi_bf16(w.y);
    } else {
      v[0] = lo_f16(w.x); v[1] = hi_f16(w.x); v[2] = lo_f16(w.y); v[3] = hi_f16(w.y);
    }
  }
}
// Output stores are non-temporal: no workgroup of the launch reads y, and lines allocated for it
// in L2 would evict the x and W panels that the concurrent workgroups of an XCD share (QKV and
// FFN up 1.5-3 % faster, measured interleaved on one box).
template <int DT>
__device__ __forceinline__ void store4(void* base, int64_t idx, const float (&v)[4]) {
  if constexpr (DT == MMDIT_F32) {
    const f32x4 x = {v[0], v[1], v[2], v[3]};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx));
  } else if constexpr (DT == MMDIT_BF16) {
    const u32x2 x = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx));
  } else {   // f16 outputs are intermediates of the block: range-guarded
    const u32x2 x = {pack_f16x2(sat_f16(v[0]), sat_f16(v[1])), pack_f16x2(sat_f16(v[2]), sat_f16(v[3]))};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx));
  }
}

// Buffer descriptor over `bytes` bytes at `p`, built from readfirstlane'd words so that it
// provably lives in SGPRs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* p, int64_t bytes) {
  const uint64_t addr = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  const int num = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, num,
                                           0x00020000);
}

// An LDS-DMA destination passed through an opaque SGPR copy: the compiler then cannot tell
// which LDS object the load writes and leaves every wait for it to the explicit per-stage
// waits of the kernel (otherwise it drains all stages in flight at each loop iteration).
__device__ __forceinline__ __attribute__((address_space(3))) void* opaque_lds(__attribute__((address_space(3))) void* p) {
  uint32_t a = (uint32_t)(uintptr_t)p;
  asm volatile("" : "+s"(a));
  return (__attribute__((address_space(3))) void*)(uintptr_t)a;
}

// Tile of virtual index t: tiles are renumbered so that each XCD (workgroups go round-robin
// over the 8 XCDs) owns a contiguous run of the whole-tile range, and rastered in bands of
// args.group_m M-tiles inside a problem.
__device__ __forceinline__ void gemm_tile_of(const GemmArgs& args, int64_t t, int& pi, int& m0, int& n0) {
  if (t < args.full && (args.full & 7) == 0) t = (t & 7) * (args.full >> 3) + (t >> 3);
  pi = t < args.tiles0 ? 0 : 1;
  if (pi) t -= args.tiles0;
  const int64_t M = args.p[pi].M, N = args.N;
  const int64_t nTm = (M + GBM - 1) / GBM, nTn = (N + GBN - 1) / GBN;
  const int64_t per_group = (int64_t)args.group_m * nTn;
  const int64_t grp = t / per_group;
  const int64_t first_m = grp * args.group_m;
  const int64_t gm = (nTm - first_m) < args.group_m ? (nTm - first_m) : args.group_m;
  const int64_t in_grp = t - grp * per_group;
  m0 = (int)((first_m + in_grp % gm) * GBM);
  n0 = (int)((in_grp / gm) * GBN);
}

// This workgroup's tile and its range [kb, ke) of K stages (nk stages in all); part_idx >= 0
// for a split-tail workgroup (the index of its partial-sum slot).
__device__ __forceinline__ void gemm_tile(const GemmArgs& args, int nk, int& pi, int& m0, int& n0, int& kb, int& ke,
                                          int64_t& part_idx) {
  const int64_t bid = blockIdx.x;
  if (bid < args.full) {
    gemm_tile_of(args, bid, pi, m0, n0);
    kb = 0;
    ke = nk;
    part_idx = -1;
  } else {
    const int64_t r = (bid - args.full) / args.split;
    const int sp = (int)((bid - args.full) - r * args.split);
    gemm_tile_of(args, args.full + r, pi, m0, n0);
    kb = (int)((int64_t)nk * sp / args.split);
    ke = (int)((int64_t)nk * (sp + 1) / args.split);
    part_idx = bid - args.full;
  }
}

// Partial sums of one split workgroup: wave w's accumulator (j, i) (j < 2), element e, lane l
// at part[((idx * 8 + w) * 8 + 4 j + i) * 16 + e) * 64 + l]: 64 consecutive floats per store
// (stores straight from the accumulator registers; a float4 layout costs register spills).
__device__ __forceinline__ void gemm_store_part8(const GemmArgs& args, int64_t idx, int wave, int lane,
                                                 const f32x16 (&acc)[2][4]) {
  float* base = args.part + ((idx * 8 + wave) * 8) * 16 * 64 + lane;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) base[((4 * j + i) * 16 + e) * 64] = acc[j][i][e];
}

// GELU or gated residual on four consecutive outputs (row m, columns n .. n + 3) that already
// hold x W^T + b.
template <int EPI, int RES_DT>
__device__ __forceinline__ void gemm_epi_tail(const GemmProblem& P, int64_t N, int64_t m, int64_t n, float (&v)[4]) {
  if constexpr (EPI == MMDIT_EPI_GELU) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = gelu_erf(v[q]);
  }
  if constexpr (EPI == MMDIT_EPI_GATED_RES) {
    // rows and rows per batch item are below 2^31 (the launch checks (M + 256) K < 2^31)
    const int64_t b = (uint32_t)m / (uint32_t)P.rows_per_batch;
    float r[4], gt[4];
    load4<RES_DT>(P.res, m * N + n, r);
    load4<MMDIT_F32>(P.gate, b * P.gate_stride + n, gt);
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = fmaf(gt[q], v[q], r[q]);
  }
}

// Raw residual values of one lane's four consecutive outputs (f32: 16 bytes, bf16: 8 bytes),
// loaded ahead of the rows that use them.
template <int RES_DT> struct ResRaw;
template <> struct ResRaw<MMDIT_F32> { float4 v; };
template <> struct ResRaw<MMDIT_BF16> { uint2 v; };
// (non-temporal: each residual element is read once)
template <int RES_DT>
__device__ __forceinline__ void res_load(const void* base, int64_t idx, ResRaw<RES_DT>& r) {
  if constexpr (RES_DT == MMDIT_F32) {
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx));
    r.v = make_float4(x[0], x[1], x[2], x[3]);
  } else {
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + idx));
    r.v = make_uint2(x[0], x[1]);
  }
}
template <int RES_DT>
__device__ __forceinline__ void res_unpack(const ResRaw<RES_DT>& r, float (&v)[4]) {
  if constexpr (RES_DT == MMDIT_F32) { v[0] = r.v.x; v[1] = r.v.y; v[2] = r.v.z; v[3] = r.v.w; }
  else { v[0] = lo_bf16(r.v.x); v[1] = hi_bf16(r.v.x); v[2] = lo_bf16(r.v.y); v[3] = hi_bf16(r.v.y); }
}

// Orders one wave's LDS writes before its own later reads (and reads before later writes):
// a wave's LDS instructions execute in order, so a wavefront-scope fence suffices.
__device__ __forceinline__ void epi_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Epilogue of a 256 x 256 tile through LDS, so that the residual loads and the output stores
// run along rows: wave w restages its 128 x 64 block a quarter (32 rows, accumulators i = q)
// at a time as f32 in its own LDS region, rows 68 floats apart (the 4-float pad spreads the
// rows one 16-lane group touches over distinct bank groups), then reads it back four rows per
// instruction, 16 lanes x 4 columns per row, and applies the FP8 scales, bias, GELU or the
// gated residual to four consecutive outputs per lane.  GEMM_SCATTER_Y: logical output row
// m, column n goes to column n % C of the full-grid token merged_row0(m) + (s / 2) W + s % 2,
// s = n / C (a 64-wide block lies inside one s, as C is a multiple of 256).  `region` holds
// 32 x 68 floats; the caller has made every wave's reads of the K stages complete.
// Gated residual: the residual of a group of four rows is loaded while the previous group is
// computed (the quarter's first group before its restaging), so the loads of consecutive
// groups overlap instead of each group waiting a full memory round trip (all CUs finish their
// K loops together, and the row-by-row epilogue was bound by the load latency of that burst).
// Each wave restages in its own region, so only the wave's own LDS order matters between
// quarters; the gated-residual epilogues still step all waves together with workgroup
// barriers, which measured faster for them (their residual loads then go out together),
// while the others let the waves drift apart.
constexpr int G8_THREADS = 512;                         // the 8-wave kernels' workgroup
constexpr int G8_EPI_STRIDE = 68;                       // floats per restaged row
constexpr int G8_EPI_BYTES = 32 * G8_EPI_STRIDE * 4;    // one wave's quarter block: 8.5 KiB
template <int BIAS_DT, int Y_DT, int EPI, int RES_DT, int LAYOUT, bool FP8 = false>
__device__ __forceinline__ void gemm_epilogue_rows8(const GemmArgs& args, const GemmProblem& Pk,
                                                    const f32x16 (&acc)[2][4], int m0, int n0, int wm, int wn,
                                                    int lane, float* region) {
  // a private copy of the problem: read through the reference, its pointers were reloaded
  // from the kernel arguments after every output store (one scalar load and wait per row)
  const GemmProblem P = Pk;
  const int64_t M = P.M, N = args.N;
  const int l32 = lane & 31, g = lane >> 5;
  const int c16 = lane & 15, r4 = lane >> 4;
  const int64_t n = n0 + wn * 64 + 4 * c16;
  float bias[4] = {0.f, 0.f, 0.f, 0.f};
  if (P.bias && n < N) load4<BIAS_DT>(P.bias, n, bias);
  float sw = 1.f;
  if constexpr (FP8) sw = *P.w_scale;
  int sg = 0;
  if constexpr (LAYOUT == GEMM_SCATTER_Y) sg = (n0 + wn * 64) / args.c;
  constexpr bool GRES = EPI == MMDIT_EPI_GATED_RES;
  // Gates of the batch items this wave's 128 rows belong to: with at least 128 rows per item
  // they span at most two (b0 below row `bnd`, b0 + 1 from it on), loaded once here instead of
  // a division and a gate load per row; shorter items take the per-row form.
  float g0[4] = {0.f, 0.f, 0.f, 0.f}, g1[4] = {0.f, 0.f, 0.f, 0.f};
  int64_t bnd = 0;
  bool gate_rows = false;
  if constexpr (GRES) {
    const uint32_t rpb = (uint32_t)P.rows_per_batch;
    const int64_t mw = m0 + wm * 128;
    gate_rows = rpb < 128;
    if (!gate_rows && mw < M && n < N) {
      const uint32_t b0 = (uint32_t)mw / rpb;
      bnd = (int64_t)(b0 + 1) * rpb;
      load4<MMDIT_F32>(P.gate, (int64_t)b0 * P.gate_stride + n, g0);
      if (bnd < M && bnd < mw + 128) load4<MMDIT_F32>(P.gate, (int64_t)(b0 + 1) * P.gate_stride + n, g1);
    }
  }
  // residual of rows r0 + 4 k + r4 (k = 0..3) of quarter q
  auto res_group = [&](int q, int r0, ResRaw<RES_DT> (&rr)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t m = m0 + wm * 128 + q * 32 + r0 + 4 * k + r4;
      if (m < M && n < N) res_load<RES_DT>(P.res, m * N + n, rr[k]);
    }
  };
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ResRaw<RES_DT> rc[4], rn[4];
    if constexpr (GRES) res_group(q, 0, rc);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) region[l32 * G8_EPI_STRIDE + j * 32 + 8 * (e >> 2) + 4 * g + (e & 3)] = acc[j][q][e];
    if constexpr (GRES) __syncthreads(); else epi_wave_sync();
#pragma unroll
    for (int r0 = 0; r0 < 32; r0 += 16) {
      if constexpr (GRES) {
        if (r0 + 16 < 32) res_group(q, r0 + 16, rn);
      }
      float4 a4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        a4[k] = *reinterpret_cast<const float4*>(region + (r0 + 4 * k + r4) * G8_EPI_STRIDE + 4 * c16);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 a = a4[k];
        const int64_t m = m0 + wm * 128 + q * 32 + r0 + 4 * k + r4;
        if (m >= M || n >= N) continue;
        float v[4];
        if constexpr (FP8) {
          const float rs = P.x_scale[m] * sw;
          v[0] = fmaf(a.x, rs, bias[0]); v[1] = fmaf(a.y, rs, bias[1]);
          v[2] = fmaf(a.z, rs, bias[2]); v[3] = fmaf(a.w, rs, bias[3]);
        } else {
          v[0] = a.x + bias[0]; v[1] = a.y + bias[1]; v[2] = a.z + bias[2]; v[3] = a.w + bias[3];
        }
        if constexpr (GRES) {
          float r[4], gt[4];
          res_unpack<RES_DT>(rc[k], r);
          if (gate_rows) {
            const int64_t b = (uint32_t)m / (uint32_t)P.rows_per_batch;
            load4<MMDIT_F32>(P.gate, b * P.gate_stride + n, gt);
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) gt[c] = m < bnd ? g0[c] : g1[c];
          }
#pragma unroll
          for (int c = 0; c < 4; ++c) v[c] = fmaf(gt[c], v[c], r[c]);
        } else {
          gemm_epi_tail<EPI, RES_DT>(P, N, m, n, v);
        }
        if constexpr (LAYOUT == GEMM_SCATTER_Y) {
          const int64_t yr = (int64_t)merged_row0((int)m, args) + (sg >> 1) * args.w + (sg & 1);
          store4<Y_DT>(P.y, yr * args.c + (n - (int64_t)sg * args.c), v);
        } else {
          store4<Y_DT>(P.y, m * N + n, v);
        }
      }
      if constexpr (GRES) {
#pragma unroll
        for (int k = 0; k < 4; ++k) rc[k] = rn[k];
      }
    }
    if constexpr (GRES) __syncthreads(); else epi_wave_sync();
  }
}

// FP8 operands (E4M3 codes, one byte per element): four LDS stages of K = 64, rows of 64
// bytes; each 32 x 32 output tile takes one 32 x 32 x 64 MFMA per stage.
template <int BIAS_DT, int Y_DT, int EPI, int RES_DT>
__global__ __launch_bounds__(G8_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_fp8_kernel(GemmArgs args) {
  constexpr int KSTEP = 64;   // K values per stage (64 bytes per row)
  // one LDS object per stage: x tile, then W tile
  __shared__ __attribute__((aligned(16))) uint8_t lds_s0[2 * G_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_s1[2 * G_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_s2[2 * G_TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t lds_s3[2 * G_TILE_BYTES];

  int pi, m0, n0, kb, ke;
  int64_t part_idx;
  gemm_tile(args, (int)(args.K / KSTEP), pi, m0, n0, kb, ke, part_idx);
  const GemmProblem& P = args.p[pi];
  const int64_t M = P.M, N = args.N, K = args.K;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;

  // ---- LDS-DMA: wave w fills rows 32w .. 32w+31 of the x tile and of the W tile with two
  // 1 KiB loads each (lane l -> row 32w + 16i + l/4, physical chunk l % 4).  The immediate
  // offset i * 1024 moves the LDS destination and the source alike and is taken back out of
  // the per-lane offset, so both loads of a tile share one LDS base; the K position goes in
  // the scalar offset, which the range check ignores.  Rows past M or N load zeros.
  const __amdgpu_buffer_rsrc_t rx = gemm_rsrc(P.x, M * K);
  const __amdgpu_buffer_rsrc_t rw = gemm_rsrc(P.w, N * K);
  int xo[2], wo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 32 * wave + 16 * i + (lane >> 2);
    const int lc = (lane & 3) ^ swz(row);
    xo[i] = (m0 + row) * (int)K + lc * 16 - i * 1024;
    wo[i] = (n0 + row) * (int)K + lc * 16 - i * 1024;
  }
  auto dma = [&](uint8_t* xs, uint8_t* ws, int k0) {
    const int so = k0 + kb * KSTEP;
    auto* lx = opaque_lds((__attribute__((address_space(3))) void*)(xs + wave * 2048));
    auto* lw = opaque_lds((__attribute__((address_space(3))) void*)(ws + wave * 2048));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, lx, 16, xo[0], so, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, lx, 16, xo[1], so, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, lw, 16, wo[0], so, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, lw, 16, wo[1], so, 1024, 0);
  };
  auto xbuf = [&](auto s) -> uint8_t* {
    constexpr int v = decltype(s)::value;
    if constexpr (v == 0) return lds_s0; else if constexpr (v == 1) return lds_s1;
    else if constexpr (v == 2) return lds_s2; else return lds_s3;
  };
  auto wbuf = [&](auto s) -> uint8_t* { return xbuf(s) + G_TILE_BYTES; };
  constexpr std::integral_constant<int, 0> S0{};
  constexpr std::integral_constant<int, 1> S1{};
  constexpr std::integral_constant<int, 2> S2{};
  constexpr std::integral_constant<int, 3> S3{};

  // ---- fragment reads: row base + l32 of a tile, 16-byte half h = chunk 2 h + g; the swizzle
  // of row base + l32 (base a multiple of 32) depends on l32 only
  int cofs[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) cofs[h] = l32 * 64 + (((2 * h + g) ^ swz(l32)) << 4);

  f32x16 acc[2][4];   // [n tile][m tile] of C^T
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;

  const int nk = ke - kb;   // stages of this workgroup
  auto gbarrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // The whole 32-byte fragments of a stage (both 16-byte halves) are read one stage ahead into
  // one of two register sets (stage parity), while the 8 MFMAs of the current stage run on
  // the other.
  uint4 fw8[2][2][2], fx8[2][4][2];
  auto read8 = [&](const uint8_t* xs, const uint8_t* ws, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < 2; ++j) fw8[BUF][j][h] = *reinterpret_cast<const uint4*>(ws + (wn * 64 + j * 32) * 64 + cofs[h]);
#pragma unroll
      for (int i = 0; i < 4; ++i) fx8[BUF][i][h] = *reinterpret_cast<const uint4*>(xs + (wm * 128 + i * 32) * 64 + cofs[h]);
    }
  };
  // One K stage.  At its start stages kt and kt+1 are in LDS for every wave.  MAIN: stage
  // kt+3 exists (load it; at the end wait with its loads in flight); otherwise the tail
  // decides at run time.  Stage kt+3 goes into the buffers stage kt-1 used (every wave has
  // passed the barrier that ended stage kt-1).
  auto step = [&](auto cur_c, auto main_c, int kt) {
    constexpr int CUR = decltype(cur_c)::value;
    constexpr bool MAIN = decltype(main_c)::value;
    constexpr std::integral_constant<int, (CUR + 1) & 3> next{};
    constexpr std::integral_constant<int, (CUR + 3) & 3> ahead{};
    constexpr std::integral_constant<int, CUR & 1> buf{};
    constexpr std::integral_constant<int, (CUR + 1) & 1> nbuf{};
    if (MAIN || kt + 3 < nk) dma(xbuf(ahead), wbuf(ahead), (kt + 3) * KSTEP);
    if (MAIN || kt + 1 < nk) read8(xbuf(next), wbuf(next), nbuf);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[j][i] = mfma_fp8(fw8[buf][j][0], fw8[buf][j][1], fx8[buf][i][0], fx8[buf][i][1], acc[j][i]);
    // the twelve fragment reads among the eight MFMAs, the four DMA loads among MFMAs 1-4
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
      if (MAIN) __builtin_amdgcn_sched_group_barrier(0x010, 1, 2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
    }
    // the MFMAs only touch registers: keep the scheduler from moving them past the barrier
    __builtin_amdgcn_sched_barrier(0);
    // this wave's loads of stage kt+2 have landed once at most the four loads of stage kt+3
    // are outstanding; after the barrier stage kt+2 is in LDS for everyone
    if (MAIN || kt + 3 < nk) __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0)
    gbarrier();
  };
  constexpr std::true_type MAIN{};
  constexpr std::false_type TAIL{};

  dma(xbuf(S0), wbuf(S0), 0);
  if (1 < nk) dma(xbuf(S1), wbuf(S1), KSTEP);
  if (2 < nk) dma(xbuf(S2), wbuf(S2), 2 * KSTEP);
  // stages 0 and 1 must be in LDS; stage 2 may still be in flight
  if (nk > 2) __builtin_amdgcn_s_waitcnt(0x0F74);   // vmcnt(4)
  else __builtin_amdgcn_s_waitcnt(0x0F70);
  gbarrier();
  read8(xbuf(S0), wbuf(S0), std::integral_constant<int, 0>{});
  int kt = 0;
  for (; kt + 6 < nk; kt += 4) {   // every step of the group has its stage kt+3
    step(S0, MAIN, kt);
    step(S1, MAIN, kt + 1);
    step(S2, MAIN, kt + 2);
    step(S3, MAIN, kt + 3);
  }
  // at most six stages remain (kt % 4 == 0)
  if (kt < nk) step(S0, TAIL, kt);
  if (kt + 1 < nk) step(S1, TAIL, kt + 1);
  if (kt + 2 < nk) step(S2, TAIL, kt + 2);
  if (kt + 3 < nk) step(S3, TAIL, kt + 3);
  if (kt + 4 < nk) step(S0, TAIL, kt + 4);
  if (kt + 5 < nk) step(S1, TAIL, kt + 5);

  if (part_idx >= 0) {
    gemm_store_part8(args, part_idx, wave, lane, acc);
  } else {
    // every wave's fragment reads of the last stage are done after this barrier; waves
    // 3s .. 3s+2 restage in stage buffer s (three 8.5 KiB regions per 32 KiB buffer)
    __syncthreads();
    uint8_t* rb = wave < 3 ? lds_s0 : wave < 6 ? lds_s1 : lds_s2;
    gemm_epilogue_rows8<BIAS_DT, Y_DT, EPI, RES_DT, GEMM_PLAIN, true>(
        args, P, acc, m0, n0, wm, wn, lane, reinterpret_cast<float*>(rb + (wave % 3) * G8_EPI_BYTES));
  }
}

// 16-bit operands, any layout: 8 wave64s, two per SIMD, arranged 2 (M) x 4 (N), each owning
// 128 x 64 outputs = 4 x 2 tiles of 32 x 32 MFMAs (128 accumulator registers, so two waves fit
// a SIMD).  While one wave of a SIMD waits for its fragment reads, the other issues MFMAs;
// the 4-wave form (one wave per SIMD, 128 x 128 each) kept the matrix pipe busy only 50-56 %
// of the time, stalling on its own reads.  Two LDS stages of K = 64 (64 KiB each, rows of 128
// bytes, chunks XOR-swizzled by (row / 2) % 8).  The next stage's eight DMA loads per wave
// go out in two fenced groups during the first quarter of the current stage; before the last
// quarter every wave waits for them and for its own reads of the current stage, and one
// barrier per 64 K follows, after which the next stage's first fragments are read under the
// last quarter's MFMAs.
// GEMM_GATHER_X: x row m, K position k reads channel k % C of the full-grid token
// merged_row0(m) + (s / 2) W + s % 2, s = k / C (a 64-wide K stage never straddles two
// neighbours, as C is a multiple of 256): the per-row part is per lane, the neighbour part
// scalar.  GEMM_SCATTER_Y is the epilogue's.
template <int IN_DT, int BIAS_DT, int Y_DT, int EPI, int RES_DT, int LAYOUT = GEMM_PLAIN>
__global__ __launch_bounds__(G8_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_k64_kernel(GemmArgs args) {
  constexpr int T64 = GBM * 128;   // one operand tile of one stage: 32 KiB
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * T64];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2 * T64];
  int pi, m0, n0, kb, ke;
  int64_t part_idx;
  gemm_tile(args, (int)(args.K / 64), pi, m0, n0, kb, ke, part_idx);
  const GemmProblem& P = args.p[pi];
  const int64_t M = P.M, N = args.N, K = args.K;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = wave >> 2, wn = wave & 3;
  // DMA i (0..3) of a wave fills rows 32 wave + 8 i .. +7 of the x tile, and of the W tile
  // (lane l -> row + l / 8, physical chunk l % 8 = logical ^ ((row / 2) % 8)); the four loads
  // of a tile share one LDS base, the immediate offset i * 1024 moving destination and source
  // alike.  A 128-byte row spans half of the 64 LDS banks, so the 16 rows one 16-lane group
  // of a 16-byte read touches fall in two bank halves by row parity; swizzling by row / 2
  // gives the 8 rows of each parity 8 distinct chunks.
  const __amdgpu_buffer_rsrc_t rx = gemm_rsrc(P.x, M * K * 2);
  const __amdgpu_buffer_rsrc_t rw = gemm_rsrc(P.w, N * K * 2);
  int xo[4], wo[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 32 * wave + 8 * i + (lane >> 3);
    const int lc = (lane & 7) ^ ((row >> 1) & 7);
    // rows past M: an offset past the end of x, so they load zeros
    if constexpr (LAYOUT == GEMM_GATHER_X)
      xo[i] = (m0 + row < M ? merged_row0(m0 + row, args) * args.c * 2 + lc * 16 : 0x7FFF0000) - i * 1024;
    else
      xo[i] = (m0 + row) * (int)K * 2 + lc * 16 - i * 1024;
    wo[i] = (n0 + row) * (int)K * 2 + lc * 16 - i * 1024;
  }
  // scalar byte offset of K position k0 in x (the neighbour's token, then the channel)
  auto x_soff = [&](int k0) {
    if constexpr (LAYOUT == GEMM_GATHER_X) {
      const int sg = __builtin_amdgcn_readfirstlane(k0 / args.c);
      return (((sg >> 1) * args.w + (sg & 1)) * args.c + (k0 - sg * args.c)) * 2;
    } else {
      return k0 * 2;
    }
  };
  auto dma_x = [&](uint8_t* xs, int k0) {
    const int so = x_soff(k0 + kb * 64);
    auto* l = opaque_lds((__attribute__((address_space(3))) void*)(xs + wave * 4096));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, l, 16, xo[0], so, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, l, 16, xo[1], so, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, l, 16, xo[2], so, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, l, 16, xo[3], so, 3072, 0);
  };
  auto dma_w = [&](uint8_t* ws, int k0) {
    const int so = (k0 + kb * 64) * 2;
    auto* l = opaque_lds((__attribute__((address_space(3))) void*)(ws + wave * 4096));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, l, 16, wo[0], so, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, l, 16, wo[1], so, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, l, 16, wo[2], so, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, l, 16, wo[3], so, 3072, 0);
  };
  auto xbuf = [&](auto st) -> uint8_t* { if constexpr (decltype(st)::value == 0) return lds_a; else return lds_b; };
  auto wbuf = [&](auto st) -> uint8_t* { return xbuf(st) + T64; };
  constexpr std::integral_constant<int, 0> S0{};
  constexpr std::integral_constant<int, 1> S1{};
  int cofs[4];   // slice ks: logical chunk 2 ks + g of row l32 (+ a multiple of 32)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) cofs[ks] = l32 * 128 + (((2 * ks + g) ^ ((l32 >> 1) & 7)) << 4);
  f32x16 acc[2][4];   // [n tile][m tile] of C^T
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;
  const int nk = ke - kb;
  auto gbarrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  uint4 wfa[2], xfa[4], wfb[2], xfb[4];
  auto read_slice = [&](const uint8_t* xs, const uint8_t* ws, int ks, uint4 (&wf)[2], uint4 (&xf)[4]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) wf[j] = *reinterpret_cast<const uint4*>(ws + (wn * 64 + j * 32) * 128 + cofs[ks]);
#pragma unroll
    for (int i = 0; i < 4; ++i) xf[i] = *reinterpret_cast<const uint4*>(xs + (wm * 128 + i * 32) * 128 + cofs[ks]);
  };
  auto mma = [&](const uint4 (&wf)[2], const uint4 (&xf)[4]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = mfma32<IN_DT>(wf[j], xf[i], acc[j][i]);
  };
  // 8 MFMAs with the next slice's 6 fragment reads among them
  auto sched = [&]() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      if (i < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
  };
  // stage kt in buffer cur, its slice 0 in wfa / xfa
  auto step = [&](auto cur_c, int kt) {
    constexpr int CUR = decltype(cur_c)::value;
    constexpr std::integral_constant<int, CUR> cur{};
    constexpr std::integral_constant<int, CUR ^ 1> oth{};
    const bool more = kt + 1 < nk;
    read_slice(xbuf(cur), wbuf(cur), 1, wfb, xfb);
    __builtin_amdgcn_sched_barrier(0);
    // slice 0: the next stage's DMA (its buffer's last readers passed the previous barrier) in
    // two fenced groups of four loads, one before each half of the slice's MFMAs (left to the
    // scheduler the loads issue in one burst that holds back the MFMAs behind them)
    if (more) dma_x(xbuf(oth), (kt + 1) * 64);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[0][i] = mfma32<IN_DT>(wfa[0], xfa[i], acc[0][i]);
    __builtin_amdgcn_sched_barrier(0);
    if (more) dma_w(wbuf(oth), (kt + 1) * 64);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[1][i] = mfma32<IN_DT>(wfa[1], xfa[i], acc[1][i]);
    __builtin_amdgcn_sched_barrier(0);
    read_slice(xbuf(cur), wbuf(cur), 2, wfa, xfa);
    mma(wfb, xfb);
    sched();
    __builtin_amdgcn_sched_barrier(0);
    read_slice(xbuf(cur), wbuf(cur), 3, wfb, xfb);
    mma(wfa, xfa);
    sched();
    __builtin_amdgcn_sched_barrier(0);
    // this wave's loads of stage kt+1 have landed and its reads of stage kt are done; after
    // the barrier both hold for every wave
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    gbarrier();
    if (more) read_slice(xbuf(oth), wbuf(oth), 0, wfa, xfa);
    mma(wfb, xfb);
    sched();
    __builtin_amdgcn_sched_barrier(0);
  };
  dma_x(xbuf(S0), 0);
  dma_w(wbuf(S0), 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  gbarrier();
  read_slice(xbuf(S0), wbuf(S0), 0, wfa, xfa);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(S0, kt);
    step(S1, kt + 1);
  }
  if (kt < nk) step(S0, kt);
  if (part_idx >= 0) {
    gemm_store_part8(args, part_idx, wave, lane, acc);
  } else {
    // every wave's fragment reads of the last stage are done after this barrier; waves 0-3
    // restage in the first stage buffer, waves 4-7 in the second
    __syncthreads();
    float* region = reinterpret_cast<float*>((wave < 4 ? lds_a : lds_b) + (wave & 3) * G8_EPI_BYTES);
    gemm_epilogue_rows8<BIAS_DT, Y_DT, EPI, RES_DT, LAYOUT>(args, P, acc, m0, n0, wm, wn, lane, region);
  }
}

// Tail tiles of a split launch (16-bit kernel): each thread sums, in K-range order, the `split`
// partial sums of the four consecutive outputs (row m, columns n .. n + 3) that one GEMM lane
// held as elements 4 e4 .. 4 e4 + 3 of one accumulator, and applies the tile epilogue to
// them; G_SUM_WG workgroups per tail tile cover its 256 x 256 outputs.
constexpr int G_SUM_WG = 64;   // 64 x 256 threads x 4 outputs = 256 x 256
template <int BIAS_DT, int Y_DT, int EPI, int RES_DT>
__global__ __launch_bounds__(GTHREADS) void gemm_split_finish_kernel(GemmArgs args) {
  const int64_t tile = blockIdx.x / G_SUM_WG;
  const int q = (blockIdx.x % G_SUM_WG) * GTHREADS + threadIdx.x;
  const int lane = q & 63, e4 = (q >> 6) & 3, i = (q >> 8) & 3, j = (q >> 10) & 1, wave = q >> 11;
  constexpr int64_t SLOT = G_PART_BYTES / 4;   // floats of one partial-sum slot
  const float* base = args.part + tile * args.split * SLOT + ((wave * 8 + 4 * j + i) * 16 + 4 * e4) * 64 + lane;
  float v[4] = {base[0], base[64], base[128], base[192]};
#pragma unroll 2
  for (int sp = 1; sp < args.split; ++sp) {
    const float* b = base + sp * SLOT;
    v[0] += b[0]; v[1] += b[64]; v[2] += b[128]; v[3] += b[192];
  }
  int pi, m0, n0;
  gemm_tile_of(args, args.full + tile, pi, m0, n0);
  const GemmProblem P = args.p[pi];
  // the accumulator element's place in the tile, as in the GEMM's epilogue
  const int64_t m = m0 + (wave >> 2) * 128 + i * 32 + (lane & 31);
  const int64_t n = n0 + (wave & 3) * 64 + j * 32 + 8 * e4 + 4 * (lane >> 5);
  if (m >= P.M || n >= args.N) return;
  float bias[4] = {0.f, 0.f, 0.f, 0.f};
  if (P.bias) load4<BIAS_DT>(P.bias, n, bias);
#pragma unroll
  for (int c = 0; c < 4; ++c) v[c] += bias[c];
  gemm_epi_tail<EPI, RES_DT>(P, args.N, m, n, v);
  store4<Y_DT>(P.y, m * args.N + n, v);
}

template <int IN_DT, int BIAS_DT, int Y_DT, int EPI, int RES_DT, int LAYOUT = GEMM_PLAIN>
static void gemm_go(const GemmArgs& a, hipStream_t st) {
  // 16-bit operands (K a multiple of 64), plain or Lite layout: the two-stage K = 64 kernel,
  // at every K (with its DMA fenced in groups it also beat a four-stage 16-bit kernel at
  // K = 6144 and 12288); FP8 operands take the four-stage FP8 kernel.
  if constexpr (IN_DT != MMDIT_FP8_E4M3) {
    if constexpr (LAYOUT == GEMM_PLAIN) {
      if (a.full < a.tiles) {   // split tail: whole tiles and K ranges of the tail tiles, then their sums
        const int64_t grid = a.full + (a.tiles - a.full) * a.split;
        gemm_k64_kernel<IN_DT, BIAS_DT, Y_DT, EPI, RES_DT><<<dim3((unsigned)grid), G8_THREADS, 0, st>>>(a);
        gemm_split_finish_kernel<BIAS_DT, Y_DT, EPI, RES_DT><<<dim3((unsigned)((a.tiles - a.full) * G_SUM_WG)), GTHREADS, 0, st>>>(a);
        return;
      }
    }
    gemm_k64_kernel<IN_DT, BIAS_DT, Y_DT, EPI, RES_DT, LAYOUT><<<dim3((unsigned)a.tiles), G8_THREADS, 0, st>>>(a);
  } else {
    static_assert(LAYOUT == GEMM_PLAIN, "FP8 operands use the plain layout");
    gemm_fp8_kernel<BIAS_DT, Y_DT, EPI, RES_DT><<<dim3((unsigned)a.tiles), G8_THREADS, 0, st>>>(a);
  }
}

// Lite merge (GEMM_GATHER_X: y [B*T*(H/2)*(W/2), C] = gather4(x) W^T + b, W [C, 4C]) and
// unpatchify (GEMM_SCATTER_Y: y [B*T*H*W, C] = scatter4(x W^T + b), W [4C, C]).
int launch_lite_regroup(int layout, const void* x, const void* w, const void* bias, int bias_dtype, void* y,
                        int in_dtype, int y_dtype, int64_t B, int64_t T, int64_t H, int64_t W, int64_t C,
                        hipStream_t stream) {
  GemmArgs a{};
  const int64_t M = B * T * (H / 2) * (W / 2);
  const int64_t N = layout == GEMM_GATHER_X ? C : 4 * C;
  const int64_t K = layout == GEMM_GATHER_X ? 4 * C : C;
  if ((M + GBM) * K * 2 >= ((int64_t)1 << 31) || (N + GBN) * K * 2 >= ((int64_t)1 << 31))
    return fail(MMDIT_ERR_SHAPE, "lite: tensors too large for 32-bit buffer offsets");
  a.p[0].x = x; a.p[0].w = w; a.p[0].bias = bias; a.p[0].y = y; a.p[0].M = M; a.p[0].rows_per_batch = M;
  a.tiles0 = a.tiles = ((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN);
  a.full = a.tiles;
  a.split = 1;
  a.group_m = K >= 8192 ? 2 : 4;
  a.N = N; a.K = K;
  a.c = (int)C; a.w = (int)W; a.w2 = (int)(W / 2); a.hw2 = (int)((H / 2) * (W / 2));
  if (a.tiles == 0) return MMDIT_OK;
  const bool bf = bias_dtype == MMDIT_F32;
#define LITE_CASE(L, IN, Y)                                                                   \
  if (layout == L && in_dtype == IN && y_dtype == Y) {                                        \
    if (bf) gemm_go<IN, MMDIT_F32, Y, MMDIT_EPI_NONE, MMDIT_F32, L>(a, stream);                \
    else gemm_go<IN, MMDIT_BF16, Y, MMDIT_EPI_NONE, MMDIT_F32, L>(a, stream);                  \
    return check_launch(L == GEMM_GATHER_X ? "lite_merge" : "lite_unpatchify");               \
  }
#define LITE_IN(L, IN) LITE_CASE(L, IN, MMDIT_F32) LITE_CASE(L, IN, MMDIT_BF16) LITE_CASE(L, IN, MMDIT_F16)
  LITE_IN(GEMM_GATHER_X, MMDIT_BF16) LITE_IN(GEMM_GATHER_X, MMDIT_F16)
  LITE_IN(GEMM_SCATTER_Y, MMDIT_BF16) LITE_IN(GEMM_SCATTER_Y, MMDIT_F16)
#undef LITE_IN
#undef LITE_CASE
  return fail(MMDIT_ERR_DTYPE, "lite: unsupported dtype combination");
}

int launch_linear(const GemmProblem* probs, int nprobs, int x_dtype, int bias_dtype, int y_dtype,
                  int64_t N, int64_t K, int epilogue, int res_dtype, hipStream_t stream, float* split_ws,
                  size_t split_ws_bytes) {
  GemmArgs a{};
  const int64_t nTn = (N + GBN - 1) / GBN;
  int64_t tiles[2] = {0, 0};
  // x and W are addressed through 32-bit buffer offsets, a tile's rows may run 256 past M
  const int64_t es = dtype_size(x_dtype);
  if (N % 4 || (N + GBN) * K * es >= ((int64_t)1 << 31))
    return fail(MMDIT_ERR_SHAPE, "linear: need N a multiple of 4 and (N + 256) * K * elem < 2^31");
  for (int i = 0; i < nprobs; ++i) {
    if ((probs[i].M + GBM) * K * es >= ((int64_t)1 << 31))
      return fail(MMDIT_ERR_SHAPE, "linear: need (M + 256) * K * 2 < 2^31");
    a.p[i] = probs[i];
    tiles[i] = ((probs[i].M + GBM - 1) / GBM) * nTn;
  }
  a.tiles0 = tiles[0];
  a.tiles = tiles[0] + tiles[1];
  a.N = N;
  a.K = K;
  a.full = a.tiles;
  a.split = 1;
  a.group_m = K >= 8192 ? 2 : 4;
  if (a.tiles == 0) return MMDIT_OK;
  // Split tail: when the tiles fill R < P workgroup slots of the last round (P = the CU
  // count, one workgroup per CU), cut each of those R tiles into S = P / R K ranges (at
  // least 2, each of at least 2 stages) so that the last round runs on (nearly) every CU
  // instead of R of them.
  const int64_t round = device_cu_count();
  if (split_ws && x_dtype != MMDIT_FP8_E4M3 && a.tiles > round) {
    const int64_t R = a.tiles % round;
    const int64_t stages = K / 64;   // K = 64 stages of the two-stage kernel
    int64_t S = R ? round / R : 0;
    if (S > stages / 2) S = stages / 2;
    if (R > 0 && S > (int64_t)(split_ws_bytes / ((size_t)R * G_PART_BYTES))) S = (int64_t)(split_ws_bytes / ((size_t)R * G_PART_BYTES));
    if (R > 0 && S >= 2 && (size_t)(R * S) * G_PART_BYTES <= split_ws_bytes) {
      a.full = a.tiles - R;
      a.split = (int)S;
      a.part = split_ws;
    }
  }
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
  GEMM_IN(MMDIT_FP8_E4M3)
#undef GEMM_IN
#undef GEMM_CASE
  return fail(MMDIT_ERR_DTYPE, "linear: unsupported dtype / epilogue combination");
}

}  // namespace mmdit
