/*
 * mmdit.h -- C ABI of the MI355X (gfx950) dual-stream MMDiT block core.
 *
 * The block is the one described in "Vimoo 1.0: Video Generation for Compact,
 * Lightweight, and High-Speed", section 2.2 (Dual-Stream MMDiT Backbone): visual and
 * conditioning tokens keep separate projections and FFNs, are concatenated for one joint
 * non-causal attention, and are modulated by shift / scale / gate vectors produced from a
 * shared timestep bottleneck.  The fusion of QK-Norm with RoPE and of the other
 * memory-bound steps follows "Seaweed-7B: Cost-Effective Training of Video Generation
 * Foundation Model", section 3.4 (kernel fusion).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers.  Every tensor argument is a DEVICE pointer owned by the caller.  The library
 *   never allocates, frees or synchronizes; scratch memory of mmdit_block_fwd comes from
 *   the caller's workspace.  Host-side structs (mmdit_rope3d, mmdit_block_dims,
 *   mmdit_stream_weights) are read during the call only.
 * - Streams.  Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *   null stream) and runs in stream order.  Calls return after enqueueing.
 * - Errors.  Every call returns an mmdit_status.  Arguments are validated before anything
 *   is enqueued; on a validation error nothing runs.  A failed launch returns
 *   MMDIT_ERR_HIP.  mmdit_last_error() returns a thread-local text for the last failure of
 *   the calling thread.  Device faults surface at the caller's next synchronization.
 * - Layouts.  Row-major; tokens are [B, N, ...] with a token row stride given in elements
 *   (batch items are N rows apart).  Heads split channels head-major: channel c of a row
 *   is head c / D, dim c % D.  Weights use the nn.Linear layout [out, in], rows contiguous.
 * - Dtypes.  MMDIT_F32, MMDIT_BF16, MMDIT_F16.  Conversions to 16-bit round to nearest
 *   even.  Accumulation is fp32 everywhere.
 * - Alignment.  Every pointer must be 16-byte aligned and every row stride a multiple of
 *   8 elements (16 bytes for 16-bit types).
 * - Thread safety.  No global mutable state besides the thread-local error text.
 */
#ifndef MMDIT_H_
#define MMDIT_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* MMDIT_FP8_E4M3: the OCP 8-bit float (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * largest finite value 448, no infinities), accepted only where a call says so. */
enum mmdit_dtype { MMDIT_F32 = 0, MMDIT_BF16 = 1, MMDIT_F16 = 2, MMDIT_FP8_E4M3 = 3 };

enum mmdit_status {
  MMDIT_OK = 0,
  MMDIT_ERR_NULL = 1,        /* a required pointer is NULL                               */
  MMDIT_ERR_ALIGN = 2,       /* a pointer or a row stride is not 16-byte aligned         */
  MMDIT_ERR_SHAPE = 3,       /* sizes are inconsistent or out of the supported range     */
  MMDIT_ERR_DTYPE = 4,       /* unsupported dtype or dtype combination                   */
  MMDIT_ERR_WORKSPACE = 5,   /* workspace smaller than mmdit_block_workspace_bytes()     */
  MMDIT_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed               */
  MMDIT_ERR_ALIAS = 7        /* an output overlaps an input where that is not allowed    */
};

/* 3D rotary embedding of visual tokens (Vimoo 1.0 notes, section 2.2): the D head dims
 * are cut into bands of d_t, d_h, d_w dims (16/56/56 for D = 128) rotated by the token's
 * temporal, vertical and horizontal position.  Visual token n of a batch item sits at
 * t = n / (H*W), h = (n / W) % H, w = n % W (w fastest).  Pair j of a band of width d
 * (dims 2j, 2j+1 counted from the band's start) turns by pos * base^(-2j/d).
 * Requirements: T, H, W >= 1; d_t, d_h, d_w even, >= 0, summing to D; base > 0. */
typedef struct {
  int64_t T, H, W;
  int32_t d_t, d_h, d_w;
  float base;
} mmdit_rope3d;

/* ---------------------------------------------------------------------------------
 * mmdit_modulate_ln -- LayerNorm with timestep shift/scale, optionally after a gated
 * residual (Vimoo 1.0 notes, section 2.2: LayerNorm precedes attention and FFN, shift and
 * scale come from the timestep path, gates weight each branch's residual update).
 *
 *   x'  = x + gate * branch          (branch given)   or   x' = x   (branch NULL)
 *   y   = LN(x') * (1 + scale) + shift
 *   LN(v) = (v - mean(v)) / sqrt(var(v) + eps), biased variance over C, no affine.
 *
 * x       [B, N, C]  x_dtype F32 | BF16, rows contiguous (row stride C).
 * branch  [B, N, C]  branch_dtype F32 | BF16, or NULL.
 * gate, shift, scale: f32, [B, C] each; item b's vector starts at ptr + b * mod_stride
 *         (mod_stride in elements, >= C; pass 6*C to read straight from an mmdit
 *         modulation buffer).  gate is required iff branch is given.
 * x_out   [B, N, C] f32 receives x' (may be NULL).
 * y       [B, N, C] y_dtype F32 | BF16 | F16; an f16 y saturates at +-65504 (NaN stays NaN).
 * C must be a multiple of 8 and at most 8192.  N may be 0.  Outputs must not overlap
 * inputs.
 * ------------------------------------------------------------------------------- */
int mmdit_modulate_ln(const void* x, int x_dtype,
                      const void* branch, int branch_dtype, const float* gate,
                      float* x_out,
                      const float* shift, const float* scale, int64_t mod_stride,
                      void* y, int y_dtype,
                      int64_t B, int64_t N, int64_t C, float eps, void* stream);

/* ---------------------------------------------------------------------------------
 * mmdit_qk_norm_rope -- per-head RMSNorm of Q and K with their own learned scales, then
 * (visual stream, rope != NULL) 3D RoPE; the conditioning stream passes rope = NULL and
 * gets no rotation (Vimoo 1.0 notes, section 2.2).  Norm first, rotation second, fused in
 * one pass over HBM (Seaweed-7B, section 3.4).
 *
 *   q^ = RoPE(q / sqrt(mean_d(q^2) + eps) * g_q),  likewise k with g_k.
 *
 * q, k       [B, N, H, D] in_dtype F32 | BF16 | F16; token row stride in_row_stride (>= H*D).
 * q_scale, k_scale  scale_dtype F32 | BF16: [D] shared by all heads (scale_head_stride 0)
 *            or [H, D] (scale_head_stride = D).
 * q_out, k_out  [B, N, H, D] out_dtype F32 | BF16 | F16, row stride out_row_stride.
 *            In place is allowed (q_out == q and k_out == k with equal strides and dtypes);
 *            partial overlap is not.
 * D must be 128.  N may be 0.  With rope, N must equal rope->T * rope->H * rope->W.
 * ------------------------------------------------------------------------------- */
int mmdit_qk_norm_rope(const void* q, const void* k, int in_dtype, int64_t in_row_stride,
                       const void* q_scale, const void* k_scale, int scale_dtype,
                       int64_t scale_head_stride,
                       void* q_out, void* k_out, int out_dtype, int64_t out_row_stride,
                       int64_t B, int64_t N, int64_t H, int64_t D, float eps,
                       const mmdit_rope3d* rope, void* stream);

/* ---------------------------------------------------------------------------------
 * mmdit_joint_attention -- one non-causal softmax attention over the concatenation of
 * the conditioning and visual tokens, split back into the two streams (Vimoo 1.0 notes,
 * section 2.2; non-causal per the Wan report).  For every batch item and head:
 *
 *   O = softmax(Q_all K_all^T * softmax_scale) V_all,  Q/K/V_all = [cond rows | vis rows]
 *
 * (The order of the concatenation does not change any output.)  No mask.
 *
 * q/k/v_vis   [B, n_vis, H, D], q/k/v_cond [B, n_cond, H, D]; one token row stride
 *             in_row_stride for all six.  Q and K are used as given: normalise / rotate
 *             them first.
 * qk_dtype, v_dtype  F16 or BF16 each (MFMA path), or both F32 (fp32 VALU path).  On the
 *             MFMA path Q K^T runs on qk_dtype operands; the probabilities P are rounded to
 *             f16 and P V runs on f16 operands, a bf16 V being converted to f16 on the way
 *             into LDS (V values must lie within the f16 range).
 * o_vis, o_cond  [B, n_s, H, D] out_dtype F32 | BF16 | F16, row stride out_row_stride.
 * lse         optional f32 [B, H, n_cond + n_vis], cond rows first: the natural-log
 *             sum of exp(scaled logits) of each query row, or NULL.
 * workspace   optional device memory (256-byte aligned, caller-owned, contents scratch):
 *             with 16-bit operands, no lse and a last round of 256 workgroups that the
 *             (batch x head, 256-query tile) items fill only partly, those items are split
 *             over key ranges whose results go there (up to 256 x 33280 floats = 34 MB) and
 *             are merged (O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s).  NULL or too
 *             small: no split.  Calls that share a workspace must not overlap.  The
 *             workspace must not overlap any input, output or lse (MMDIT_ERR_ALIAS).
 * D must be 128; n_vis + n_cond >= 1; a stream with n_s = 0 may pass NULL pointers.
 * ------------------------------------------------------------------------------- */
int mmdit_joint_attention(const void* q_vis, const void* k_vis, const void* v_vis, int64_t n_vis,
                          const void* q_cond, const void* k_cond, const void* v_cond, int64_t n_cond,
                          int qk_dtype, int v_dtype, int64_t in_row_stride,
                          int64_t B, int64_t H, int64_t D, float softmax_scale,
                          void* o_vis, void* o_cond, int out_dtype, int64_t out_row_stride,
                          float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * mmdit_joint_attention_noalloc -- mmdit_joint_attention for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments and results as mmdit_joint_attention without the workspace: the split tail's
 * key-range results go to a static scratch array inside the library, MMDIT_NOALLOC_SCRATCH_BYTES
 * (34,078,720 bytes: 256 slots of one 256-query tile) on each GPU the library runs on, held
 * until the process ends.  The GPU is the one that runs `stream` (the current device for the
 * null stream); the first call on a GPU takes the scratch's address there, making that device
 * current for the lookup and restoring the caller's.  No call allocates or frees memory.  The scratch is shared by every call on
 * a GPU and keeps the last call's contents (nothing in it needs to start at zero): calls that
 * overlap in time on one GPU (different streams, or threads without ordering) race and must be
 * serialised by the caller.  A call whose split tail would need more than the scratch holds
 * (possible only on a device with more than 256 compute units) returns MMDIT_ERR_WORKSPACE
 * before anything is enqueued.
 * ------------------------------------------------------------------------------- */
#define MMDIT_NOALLOC_SCRATCH_BYTES ((size_t)34078720)
int mmdit_joint_attention_noalloc(const void* q_vis, const void* k_vis, const void* v_vis, int64_t n_vis,
                                  const void* q_cond, const void* k_cond, const void* v_cond, int64_t n_cond,
                                  int qk_dtype, int v_dtype, int64_t in_row_stride,
                                  int64_t B, int64_t H, int64_t D, float softmax_scale,
                                  void* o_vis, void* o_cond, int out_dtype, int64_t out_row_stride,
                                  float* lse, void* stream);

/* ---------------------------------------------------------------------------------
 * mmdit_cast -- elementwise dtype change, y[i] = x[i] rounded to y_dtype (nearest even).
 * Not a step of the pages' method: it lets bf16 inputs reach the 16-bit attention kernel as
 * f16 operands (a bf16 V converted inside the kernel costs its MFMA-only phase 16
 * conversions per key tile), the same conversion the block applies to its weights.
 *
 * x [n] x_dtype, y [n] y_dtype: F32 | BF16 | F16, two different types; both 16-byte aligned.
 * y may be x itself when both types are 16-bit (in place); any other overlap is refused
 * (MMDIT_ERR_ALIAS).  n may be 0.
 * ------------------------------------------------------------------------------- */
int mmdit_cast(const void* x, int x_dtype, void* y, int y_dtype, int64_t n, void* stream);

/* ---------------------------------------------------------------------------------
 * mmdit_linear -- y = epilogue(x W^T + bias) on bf16 / f16 MFMA, fp32 accumulate.  The
 * per-stream projections of the block (QKV, output, FFN) all run through this GEMM.
 *
 * x  [M, K] x_dtype BF16 | F16 (row stride K);  w [N, K] same dtype as x;  bias [N] f32 |
 *    bf16 (bias_dtype) or NULL.
 * epilogue:
 *   MMDIT_EPI_NONE      y = acc + bias
 *   MMDIT_EPI_GELU      y = GELU(acc + bias), erf form (erf to 1.5e-7 absolute,
 *                       Abramowitz & Stegun 7.1.26)
 *   MMDIT_EPI_GATED_RES y = res + gate[b] * (acc + bias), b = row / rows_per_batch;
 *                       res [M, N] res_dtype F32 | BF16; gate f32, item b at
 *                       gate + b * gate_stride (gate_stride a multiple of 4).
 * y  [M, N] y_dtype F32 | BF16 | F16; an f16 y saturates at +-65504 (NaN stays NaN).
 * K must be a multiple of 64, N a multiple of 4, M, N >= 0; x and w are addressed with 32-bit offsets: (M + 256) * K and (N + 256) * K
 * elements must stay below 2^30.  Pointers 16-byte aligned.
 * ------------------------------------------------------------------------------- */
enum mmdit_epilogue { MMDIT_EPI_NONE = 0, MMDIT_EPI_GELU = 1, MMDIT_EPI_GATED_RES = 2 };

int mmdit_linear(const void* x, const void* w, int x_dtype,
                 const void* bias, int bias_dtype,
                 void* y, int y_dtype,
                 int64_t M, int64_t N, int64_t K,
                 int epilogue, const void* res, int res_dtype,
                 const float* gate, int64_t gate_stride, int64_t rows_per_batch,
                 void* stream);

/* ---------------------------------------------------------------------------------
 * 8-bit joint attention (Wan report, section 4.4.3: INT8 for S = Q K^T, FP8 E4M3 for O = P V,
 * f32 accumulation across key blocks), the same joint non-causal attention as
 * mmdit_joint_attention (Vimoo 1.0 notes, section 2.2) on quantized operands.  The page
 * does not fix the scale granularity; this library uses:
 *   Q^: one INT8 scale per (token, head);  K^: one per (head, block of 64 consecutive keys
 *   of one stream);  V: one E4M3 scale per (head, channel) over the keys of both streams.
 * Each scale is amax / qmax in f32 (127 for INT8, 448 for E4M3; an all-zero group gets 1);
 * codes are rint(x * (1/s)) clamped to +-127 (INT8) or E4M3(clamp(x * (1/s), +-448)).
 *
 * mmdit_attn8_stream: the quantized operands of one stream of n tokens, caller-owned:
 *   q8       [B, n, H, D] INT8 codes (row stride H*D bytes)     q_scale [B, H, n] f32
 *   k8       [B, n, H, D] INT8 codes                            k_scale [B, H, ceil(n/64)] f32
 *   v8t      [B, H, D, np] E4M3 codes, np = 64 * ceil(n/64): channel-major; within each
 *            64-key tile, key k = 32h + 8i + 4g + c (h, g in {0,1}; i, c in 0..3) sits at byte
 *            16(2h + g) + 4i + c, the order in which the attention kernel holds its weights;
 *            keys past n are zero codes.
 * ------------------------------------------------------------------------------- */
typedef struct {
  void* q8;
  float* q_scale;
  void* k8;
  float* k_scale;
  void* v8t;
} mmdit_attn8_stream;

/* mmdit_attn8_quantize -- the operands above from 16-bit (or f32) Q^, K^, V of both streams
 * (the same inputs as mmdit_joint_attention: [B, n, H, D] views with one token row stride
 * in_row_stride, Q^/K^ already normalised and rotated); v_scale [B, H, D] f32 receives the
 * V scales (it is also the kernel's amax accumulator).  D = 128.  A stream with n = 0 is
 * skipped (its struct may be NULL).  Outputs must not overlap the inputs. */
int mmdit_attn8_quantize(const void* q_vis, const void* k_vis, const void* v_vis, int64_t n_vis,
                         const void* q_cond, const void* k_cond, const void* v_cond, int64_t n_cond,
                         int in_dtype, int64_t in_row_stride, int64_t B, int64_t H, int64_t D,
                         const mmdit_attn8_stream* vis, const mmdit_attn8_stream* cond,
                         float* v_scale, void* stream);

/* mmdit_joint_attention_8bit -- for every batch item and head, with the codes and scales of
 * mmdit_attn8_quantize, per query i and key j (keys of both streams):
 *   y_ij = acc_ij * c_ij in log2 units, acc_ij the exact integer dot product of the codes,
 *          c_ij = s_q[i] * (s_k[block of j] * (softmax_scale * log2 e)), all f32;
 *   m_i  = an integer reference, at least ceil(y_ij) for every key seen (kept exact: raising
 *          it rescales the accumulators by a power of two);
 *   P'_ij = E4M3(2^(acc_ij c_ij + 8 - m_i)) (so P' <= 256), summed by the FP8 MFMA;
 *   O_i  = s_v * (sum_j P'_ij V8_j) / (sum_j P'_ij).
 * o_vis, o_cond, out_dtype, out_row_stride, lse as for mmdit_joint_attention (lse is
 * ln(sum_j P'_ij) + (m_i - 8) ln 2).  D = 128.
 * workspace (optional, device memory, 256-byte aligned, caller-owned, contents scratch):
 * when the (batch x head, 256-query tile) items leave the GPU's last round of 256
 * workgroups partly empty and no lse is asked for, those items are split over key ranges
 * whose results go there (up to 256 x 33280 floats = 34 MB) and are merged: the ranges' sums
 * combine with exact power-of-two weights 2^(m_s - max m), so O changes only by the f32
 * summation order.  NULL or too small: no split.  Calls that share a workspace must not
 * overlap.  Outputs, lse and workspace must be disjoint from every operand (codes, scales,
 * v_scale) and from one another (MMDIT_ERR_ALIAS). */
int mmdit_joint_attention_8bit(const mmdit_attn8_stream* vis, int64_t n_vis,
                               const mmdit_attn8_stream* cond, int64_t n_cond,
                               const float* v_scale, int64_t B, int64_t H, int64_t D,
                               float softmax_scale,
                               void* o_vis, void* o_cond, int out_dtype, int64_t out_row_stride,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * mmdit_quantize_fp8 -- symmetric FP8 E4M3 quantization, with one scale per row (per_row
 * != 0: per-token activations) or one for the whole tensor (per_row == 0: weights), the
 * scaling of the Wan report's FP8 GEMMs (section 4.4.3).
 *
 *   s = amax / 448 in f32 (amax over the row or the tensor; an all-zero group gets s = 1)
 *   q = E4M3(clamp(x * (1/s), -448, 448)), rounded to nearest, ties to even
 *
 * x [rows, cols] x_dtype F32 | BF16 | F16, contiguous; q [rows, cols] E4M3 codes (bytes);
 * scales [rows] (per_row) or [1] f32.  cols a multiple of 8.  The per-tensor form runs four
 * kernels (clear, amax, quantize, scale) and uses scales[0] as its accumulator.  Outputs
 * must not overlap x or each other.
 * ------------------------------------------------------------------------------- */
int mmdit_quantize_fp8(const void* x, int x_dtype, int64_t rows, int64_t cols, int per_row,
                       void* q, float* scales, void* stream);

/* ---------------------------------------------------------------------------------
 * mmdit_linear_fp8 -- mmdit_linear on FP8 operands (Wan report, section 4.4.3: FP8 GEMM with
 * per-tensor weight and per-token activation scales):
 *
 *   y = epilogue((xq wq^T) * x_scale[m] * w_scale[0] + bias)
 *
 * xq [M, K], wq [N, K] E4M3 codes (from mmdit_quantize_fp8); x_scale [M], w_scale [1] f32.
 * The products of the codes are summed by the gfx950 8-bit MFMA (32 x 32 x 64) into f32;
 * the hardware does not sum the 64 products of one instruction exactly (it deviates from the
 * exact sum by up to ~4e-5 of the result's rms).  Everything else (bias, epilogues, res,
 * gate, rows_per_batch, dtypes of bias / y / res, the 2^31-byte limit with one byte per
 * element, alignment, aliasing) is as for mmdit_linear.  K a multiple of 64.
 * ------------------------------------------------------------------------------- */
int mmdit_linear_fp8(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                     const void* bias, int bias_dtype, void* y, int y_dtype,
                     int64_t M, int64_t N, int64_t K,
                     int epilogue, const void* res, int res_dtype,
                     const float* gate, int64_t gate_stride, int64_t rows_per_batch,
                     void* stream);

/* ---------------------------------------------------------------------------------
 * mmdit_modulation -- the per-(block, stream) modulation Linear: the shared timestep
 * bottleneck tvec is mapped directly to six C-vectors (Vimoo 1.0 notes, sections 2.2 and
 * 2.4), in the order shift_attn, scale_attn, gate_attn, shift_ffn, scale_ffn, gate_ffn.
 *
 *   mod[b] = W_mod tvec[b] + b_mod
 *
 * w_mod [6C, Dt] BF16;  b_mod [6C] BF16 or NULL;  tvec [B, Dt] t_dtype F32 | BF16;
 * mod   [B, 6C] f32.  Dt must be a multiple of 8 and at most 16384 (1536 in the full
 * model, 16 in Lite).
 * ------------------------------------------------------------------------------- */
int mmdit_modulation(const void* w_mod, const void* b_mod, const void* tvec, int t_dtype,
                     float* mod, int64_t B, int64_t C6, int64_t Dt, void* stream);

/* ---------------------------------------------------------------------------------
 * mmdit_timestep_embed -- timestep conditioning up to the shared bottleneck (Vimoo 1.0
 * notes, section 2.2; the 16-wide Lite bottleneck, section 2.4).  Per batch item b:
 *
 *   e[b]      = [cos(t[b] f_0) .. cos(t[b] f_{h-1}), sin(t[b] f_0) .. sin(t[b] f_{h-1})],
 *               h = freq_dim / 2, f_j = max_period^(-j / h)      (the pages fix only the
 *               width, 256; the cosine-first layout and max_period 10000 are a reading)
 *   hidden[b] = W1 e[b] + b1                     (the MLP's first layer, before its SiLU)
 *   temb[b]   = W2 SiLU(hidden[b]) + b2          (the 3072-d timestep representation)
 *   tvec[b]   = W3 SiLU(temb[b]) + b3            (the bottleneck shared by every block)
 *
 * SiLU(x) = x / (1 + exp(-x)).  t [B] f32 (timestep values as given, e.g. in [0, 1000]);
 * w1 [Dh, freq_dim], w2 [Dh, Dh], w3 [Dt, Dh] and biases b1 [Dh], b2 [Dh], b3 [Dt] of
 * w_dtype F32 | BF16 (biases may be NULL); outputs hidden, temb [B, Dh] and tvec [B, Dt]
 * f32, all three caller-owned (hidden doubles as the scratch between the layers).
 * freq_dim a multiple of 16 and Dh a multiple of 8, both <= 16384; Dt >= 1; max_period > 1.
 * The angles t f_j are formed in double, so large timesteps keep full f32 accuracy.
 * Outputs must not overlap each other or any input (MMDIT_ERR_ALIAS).
 * ------------------------------------------------------------------------------- */
int mmdit_timestep_embed(const float* t, int64_t B,
                         const void* w1, const void* b1, const void* w2, const void* b2,
                         const void* w3, const void* b3, int w_dtype,
                         int64_t freq_dim, int64_t hidden_dim, int64_t Dt, float max_period,
                         float* hidden, float* temb, float* tvec, void* stream);

/* ---------------------------------------------------------------------------------
 * mmdit_lite_merge / mmdit_lite_unpatchify -- the Lite model's hidden-space 2x2 spatial
 * merge before the backbone and its inverse after it (Vimoo 1.0 notes, section 2.4: four
 * neighbouring hidden vectors of each 2x2 region are concatenated and mapped 4C -> C; the
 * unpatchify projection expands each vector C -> 4C into four position-specific outputs;
 * time is not merged).  The neighbour order is (dh, dw) = (0,0), (0,1), (1,0), (1,1), each
 * neighbour's C channels contiguous (the pages fix only that the four are concatenated).
 *
 * Tokens of a batch item are the (t, h, w) grid flattened with w fastest; merged token
 * (t, i, j) covers full-grid tokens (t, 2i+dh, 2j+dw).
 *
 *   merge:       y[b, (t,i,j)]  = W [x(t,2i,2j) | x(t,2i,2j+1) | x(t,2i+1,2j) | x(t,2i+1,2j+1)] + bias
 *                x [B, T*H*W, C], w [C, 4C], bias [C] or NULL, y [B, T*(H/2)*(W/2), C]
 *   unpatchify:  z = W x[b, (t,i,j)] + bias (4C values); y(t, 2i+dh, 2j+dw) = z[(2dh+dw)C .. +C]
 *                x [B, T*(H/2)*(W/2), C], w [4C, C], bias [4C] or NULL, y [B, T*H*W, C]
 *
 * x and w BF16 | F16 (the same dtype; MFMA operands, fp32 accumulation), bias F32 | BF16,
 * y F32 | BF16 | F16.  H and W even (odd grids, such as the 45-row 720p latent, are not
 * defined by the pages and are rejected), C a multiple of 256, x and w below 2^31 bytes.
 * The gather of the four neighbours happens inside the GEMM's loads and the scatter inside
 * its stores: no regrouped copy of x or y is made.  y must not overlap x, w or bias.
 * ------------------------------------------------------------------------------- */
int mmdit_lite_merge(const void* x, int x_dtype, const void* w, const void* bias, int bias_dtype,
                     void* y, int y_dtype, int64_t B, int64_t T, int64_t H, int64_t W, int64_t C,
                     void* stream);
int mmdit_lite_unpatchify(const void* x, int x_dtype, const void* w, const void* bias, int bias_dtype,
                          void* y, int y_dtype, int64_t B, int64_t T, int64_t H, int64_t W, int64_t C,
                          void* stream);

/* ---------------------------------------------------------------------------------
 * mmdit_block_fwd -- one dual-stream MMDiT block forward (Vimoo 1.0 notes, section 2.2).
 * Per stream s (vis, cond):
 *   mod_s = W_mod,s tvec + b_mod,s  -> shift_a, scale_a, gate_a, shift_f, scale_f, gate_f
 *   h     = LN(x_s) (1 + scale_a) + shift_a
 *   q,k,v = split(h W_qkv^T + b_qkv);  q,k <- RMSNorm (scales q_norm, k_norm), RoPE on vis
 *   O_vis, O_cond = joint attention over [cond | vis]
 *   x1    = x_s + gate_a (O_s W_o^T + b_o)                       (fp32)
 *   h2    = LN(x1) (1 + scale_f) + shift_f
 *   out_s = x1 + gate_f (GELU(h2 W_fc1^T + b_fc1) W_fc2^T + b_fc2)   (out_dtype)
 *
 * dims: C = H*D, D = 128, F and C multiples of 256, Dt a multiple of 8.
 * w_dtype: MMDIT_BF16 (every weight bf16), or MMDIT_F16 with act_dtype F16: the four GEMM
 * matrices w_qkv, w_o, w_fc1, w_fc2 are given in f16 (converted once, e.g. with mmdit_cast,
 * as a deployment stores them) and every other weight stays bf16.
 * w_dtype MMDIT_FP8_E4M3 with act_dtype F16 selects the 8-bit block of the Wan report's
 * inference setup (section 4.4.3): the four GEMM matrices are E4M3 codes with one f32 scale
 * each (s_qkv, s_o, s_fc1, s_fc2, device pointers; mmdit_quantize_fp8 per tensor makes
 * them), every GEMM quantizes its f16 input per token (mmdit_quantize_fp8's rule) and runs
 * as mmdit_linear_fp8, and the attention quantizes the f16 q^ | k^ | v rows as
 * mmdit_attn8_quantize and runs mmdit_joint_attention_8bit; everything else is as in the
 * 16-bit block.  The scale pointers are ignored for the other w_dtypes.
 * Weights (per stream, nn.Linear layout): w_mod [6C, Dt], b_mod [6C],
 * w_qkv [3C, C], b_qkv [3C] (rows: q, then k, then v), q_norm, k_norm [D] (or [H, D] with
 * qk_scale_head_stride = D), w_o [C, C], b_o [C], w_fc1 [F, C], b_fc1 [F], w_fc2 [C, F],
 * b_fc2 [C].  Bias pointers may be NULL (no bias).
 * x_vis [B, n_vis, C], x_cond [B, n_cond, C] x_dtype BF16 | F32; tvec [B, Dt] t_dtype
 * BF16 | F32; rope describes the visual grid (n_vis = T*H*W); out_vis, out_cond
 * [B, n_s, C] out_dtype F32 | BF16.
 * act_dtype selects the type of every 16-bit intermediate (h, q|k|v, O, h2, GELU output)
 * and hence of every MFMA operand: MMDIT_BF16 (weights used as given) or MMDIT_F16 (with
 * bf16 matrices, the four weight matrices of each stream are converted to f16 in the
 * workspace on every call; f16 keeps 3 more mantissa bits, which the block's range-bounded
 * intermediates can use).
 * The modulation vectors, LayerNorm statistics, softmax state and the residual stream x1
 * are f32 in both cases.
 * workspace: >= mmdit_block_workspace_bytes(dims, B, n_vis, n_cond), 256-byte aligned;
 * its contents after the call are the intermediates listed by mmdit_block_workspace_offsets.
 * ------------------------------------------------------------------------------- */
typedef struct {
  const void *w_mod, *b_mod, *w_qkv, *b_qkv, *q_norm, *k_norm,
             *w_o, *b_o, *w_fc1, *b_fc1, *w_fc2, *b_fc2;
  const float *s_qkv, *s_o, *s_fc1, *s_fc2;   /* E4M3 matrices only: [1] f32 scale each */
} mmdit_stream_weights;

typedef struct {
  int64_t C, H, D, F, Dt;
  float ln_eps, qk_eps;
  int64_t qk_scale_head_stride;
  int w_dtype;
  int act_dtype;
} mmdit_block_dims;

/* Workspace regions (byte offsets from the workspace start), per stream s = 0 (vis), 1 (cond);
 * "act" is act_dtype:
 *   MMDIT_WS_MOD    f32 [B, 6C]   modulation vectors
 *   MMDIT_WS_H      act [B*n, C]  LN-modulated input of the QKV GEMM; then the attention output O
 *   MMDIT_WS_QKV    act [B*n, 3C] q^ | k^ | v after QK-norm and RoPE; then h2 (first B*n*C)
 *   MMDIT_WS_X1     f32 [B*n, C]  residual after the attention branch
 *   MMDIT_WS_G      act [B*n, F]  GELU(h2 W_fc1^T + b_fc1)
 *   MMDIT_WS_WQKV, MMDIT_WS_WO, MMDIT_WS_W1, MMDIT_WS_W2: f16 copies of w_qkv, w_o, w_fc1,
 *                   w_fc2 (act_dtype F16 with w_dtype BF16 only).
 *   MMDIT_WS_SPLIT  f32 64 MiB, stream 0 only: partial sums of the GEMM tiles of a launch's
 *                   last, partial round, each computed over K ranges by several workgroups,
 *                   and likewise the attention's last-round query tiles computed over key
 *                   ranges (its contents after the call are scratch).
 *   8-bit block (w_dtype MMDIT_FP8_E4M3) only:
 *   MMDIT_WS_XQ     E4M3 [B*n, max(C, F)] codes of the current GEMM input (after the call:
 *                   those of the GELU output g, [B*n, F])
 *   MMDIT_WS_XS     f32 [B*n] their per-token scales
 *   MMDIT_WS_Q8, MMDIT_WS_QS, MMDIT_WS_K8, MMDIT_WS_KS, MMDIT_WS_V8T: the stream's
 *                   mmdit_attn8_stream operands (q8, q_scale, k8, k_scale, v8t)
 *   MMDIT_WS_VS     f32 [B, H, D], stream 0 only: the V scales of both streams */
enum { MMDIT_WS_MOD = 0, MMDIT_WS_H = 1, MMDIT_WS_QKV = 2, MMDIT_WS_X1 = 3, MMDIT_WS_G = 4,
       MMDIT_WS_WQKV = 5, MMDIT_WS_WO = 6, MMDIT_WS_W1 = 7, MMDIT_WS_W2 = 8, MMDIT_WS_SPLIT = 9,
       MMDIT_WS_XQ = 10, MMDIT_WS_XS = 11, MMDIT_WS_Q8 = 12, MMDIT_WS_QS = 13, MMDIT_WS_K8 = 14,
       MMDIT_WS_KS = 15, MMDIT_WS_V8T = 16, MMDIT_WS_VS = 17, MMDIT_WS_COUNT = 18 };

size_t mmdit_block_workspace_bytes(const mmdit_block_dims* dims, int64_t B, int64_t n_vis,
                                   int64_t n_cond);

/* Fills offsets[2][MMDIT_WS_COUNT] (stream-major); unused regions get SIZE_MAX.  Returns a
 * status (dims validated as for mmdit_block_fwd). */
int mmdit_block_workspace_offsets(const mmdit_block_dims* dims, int64_t B, int64_t n_vis,
                                  int64_t n_cond, size_t* offsets);

int mmdit_block_fwd(const mmdit_block_dims* dims,
                    const mmdit_stream_weights* w_vis, const mmdit_stream_weights* w_cond,
                    const void* x_vis, const void* x_cond, int x_dtype,
                    const void* tvec, int t_dtype,
                    const mmdit_rope3d* rope, int64_t n_cond,
                    void* out_vis, void* out_cond, int out_dtype,
                    void* workspace, size_t workspace_bytes, int64_t B, void* stream);

/* mmdit_block_fwd_events -- mmdit_block_fwd that also records caller-owned hipEvents on
 * `stream` around each stage, for per-kernel timing of the same launch sequence.
 * events: array of 2 * MMDIT_STAGE_COUNT hipEvent_t handles (passed as void*), entry
 * 2*i before stage i and 2*i+1 after it; the array or any entry may be NULL (not
 * recorded).  Everything else is exactly mmdit_block_fwd. */
enum { MMDIT_STAGE_MOD_LN1 = 0,       /* modulation GEMV, LN-modulate (+ f16 weight copies)  */
       MMDIT_STAGE_QKV = 1,           /* QKV GEMM (8-bit block: with the quantization of h)  */
       MMDIT_STAGE_QK_NORM_ROPE = 2,  /* QK RMSNorm + 3D RoPE                                */
       MMDIT_STAGE_ATTENTION = 3,     /* joint attention (8-bit block: with its operands'    */
                                      /* quantization)                                       */
       MMDIT_STAGE_OUT_PROJ = 4,      /* output projection + gated residual (8-bit: with O's) */
       MMDIT_STAGE_LN2 = 5,           /* LN-modulate of the FFN branch                       */
       MMDIT_STAGE_FFN_UP = 6,        /* FFN up + GELU (8-bit: with h2's quantization)       */
       MMDIT_STAGE_FFN_DOWN = 7,      /* FFN down + gated residual (8-bit: with g's)         */
       MMDIT_STAGE_COUNT = 8 };

int mmdit_block_fwd_events(const mmdit_block_dims* dims,
                           const mmdit_stream_weights* w_vis, const mmdit_stream_weights* w_cond,
                           const void* x_vis, const void* x_cond, int x_dtype,
                           const void* tvec, int t_dtype,
                           const mmdit_rope3d* rope, int64_t n_cond,
                           void* out_vis, void* out_cond, int out_dtype,
                           void* workspace, size_t workspace_bytes, int64_t B, void* stream,
                           void* const* events);

/* Text of a status code (static storage). */
const char* mmdit_status_str(int status);
/* Thread-local detail of the calling thread's last failed call ("" if none). */
const char* mmdit_last_error(void);
/* ABI version: bumped whenever a signature or a layout above changes. */
int mmdit_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MMDIT_H_ */
