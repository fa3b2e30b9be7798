// One dual-stream MMDiT block forward (Vimoo 1.0 notes, section 2.2), enqueued on one
// stream from the library's kernels.  Both streams share every launch where the shapes
// allow it (the GEMMs run the visual and conditioning problems in one grid), and the
// workspace regions are reused once their contents are dead (h -> O, qkv -> h2).
//
// The 8-bit block (w_dtype E4M3) is the Wan report's inference setup (section 4.4.3): the
// same steps with every GEMM on FP8 operands (the f16 input quantized per token, the
// weights per tensor) and the attention on INT8 Q K^T and FP8 P V.
#include "common.h"

namespace mmdit {

int validate_rope(const mmdit_rope3d* r, int64_t N, int64_t D);

struct WsLayout {
  size_t off[2][MMDIT_WS_COUNT];
  size_t total;
};

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static int validate_dims(const mmdit_block_dims* d, int64_t B, int64_t n_vis, int64_t n_cond) {
  if (!d) return fail(MMDIT_ERR_NULL, "block: dims is NULL");
  if (d->D != 128) return fail(MMDIT_ERR_SHAPE, "block: D must be 128");
  if (d->H < 1 || d->C != d->H * d->D) return fail(MMDIT_ERR_SHAPE, "block: C must equal H * D");
  if (d->C % 256 || d->F < 256 || d->F % 256) return fail(MMDIT_ERR_SHAPE, "block: C and F must be multiples of 256");
  if (d->C > 8192 || d->F > 65536) return fail(MMDIT_ERR_SHAPE, "block: C <= 8192 and F <= 65536");
  if (d->Dt < 8 || d->Dt % 8) return fail(MMDIT_ERR_SHAPE, "block: Dt must be a positive multiple of 8");
  if (B < 1 || n_vis < 1 || n_cond < 0) return fail(MMDIT_ERR_SHAPE, "block: need B >= 1, n_vis >= 1, n_cond >= 0");
  if (!extents_ok({B, n_vis, d->F}) || !extents_ok({B, n_cond, d->F}) || !extents_ok({B, 6, d->C}))
    return fail(MMDIT_ERR_SHAPE, "block: sizes too large");
  if (d->Dt > 16384) return fail(MMDIT_ERR_SHAPE, "block: Dt must be <= 16384");
  if (d->qk_scale_head_stride != 0 && d->qk_scale_head_stride != d->D)
    return fail(MMDIT_ERR_SHAPE, "block: qk_scale_head_stride must be 0 or D");
  if (!(d->ln_eps >= 0.f) || !(d->qk_eps >= 0.f)) return fail(MMDIT_ERR_SHAPE, "block: eps must be >= 0");
  if (d->w_dtype != MMDIT_BF16 && !((d->w_dtype == MMDIT_F16 || d->w_dtype == MMDIT_FP8_E4M3) && d->act_dtype == MMDIT_F16))
    return fail(MMDIT_ERR_DTYPE, "block: w_dtype must be bf16, or f16 or fp8_e4m3 with act_dtype f16");
  if (d->act_dtype != MMDIT_BF16 && d->act_dtype != MMDIT_F16) return fail(MMDIT_ERR_DTYPE, "block: act_dtype must be bf16 or f16");
  return MMDIT_OK;
}

// 256 GEMM tile partial sums (f32), also holding the attention's split-tail key-range results
// (at most 256 x (256 x 128 + 512) floats)
constexpr size_t BLOCK_SPLIT_BYTES = (size_t)256 * 256 * 256 * 4;

static void layout(const mmdit_block_dims* d, int64_t B, int64_t n_vis, int64_t n_cond, WsLayout* L) {
  size_t cur = 0;
  const size_t C = (size_t)d->C, F = (size_t)d->F;
  const int64_t ns[2] = {n_vis, n_cond};
  const size_t H = (size_t)d->H;
  for (int s = 0; s < 2; ++s) {
    const size_t n = (size_t)(B * ns[s]);
    const bool q8 = d->w_dtype == MMDIT_FP8_E4M3;   // the 8-bit block
    const bool cvt = !q8 && d->act_dtype != d->w_dtype;   // bf16 matrices, f16 operands: per-call copies
    const size_t nb = (size_t)((ns[s] + 63) / 64);   // 64-key blocks of the stream (8-bit attention)
    const size_t sz[MMDIT_WS_COUNT] = {(size_t)B * 6 * C * 4, n * C * 2, n * 3 * C * 2, n * C * 4, n * F * 2,
                                       cvt ? 3 * C * C * 2 : 0, cvt ? C * C * 2 : 0,
                                       cvt ? F * C * 2 : 0, cvt ? C * F * 2 : 0,
                                       s == 0 ? BLOCK_SPLIT_BYTES : 0,
                                       q8 ? n * (F > C ? F : C) : 0, q8 ? n * 4 : 0,
                                       q8 ? n * C : 0, q8 ? n * H * 4 : 0, q8 ? n * C : 0,
                                       q8 ? (size_t)B * H * nb * 4 : 0, q8 ? (size_t)B * C * nb * 64 : 0,
                                       q8 && s == 0 ? (size_t)B * C * 4 : 0};
    for (int r = 0; r < MMDIT_WS_COUNT; ++r) {
      if (sz[r] == 0 && r >= MMDIT_WS_WQKV) { L->off[s][r] = SIZE_MAX; continue; }
      L->off[s][r] = cur;
      cur = align256(cur + sz[r]);
    }
  }
  L->total = cur;
}

// The 8-bit block: S1, S2, S4 and S7 as in the 16-bit block; each GEMM quantizes its f16
// input per token into the XQ / XS regions and runs on FP8 operands; the attention
// quantizes q^ | k^ | v into the Q8 ... VS regions and runs the 8-bit kernel (its split tail
// in the split region).  `mark` records the caller's stage events.
template <typename Mark>
static int block_fwd_8bit(const mmdit_block_dims& d, const mmdit_stream_weights* const* ws, const void* const* xs,
                          int x_dtype, const void* tvec, int t_dtype, const mmdit_rope3d* rope, const int64_t* ns,
                          void* const* outs, int out_dtype, uint8_t* wsb, const WsLayout& L, int64_t B,
                          hipStream_t sm, Mark mark) {
  const int64_t C = d.C, F = d.F, H = d.H;
  const int nstreams = ns[1] > 0 ? 2 : 1;
  int st;
  float* mod[2];
  void *hbuf[2], *qkv[2], *g[2];
  float* x1[2];
  uint8_t* xq[2];
  float* xsc[2];
  mmdit_attn8_stream a8[2];
  for (int s = 0; s < 2; ++s) {
    mod[s] = reinterpret_cast<float*>(wsb + L.off[s][MMDIT_WS_MOD]);
    hbuf[s] = wsb + L.off[s][MMDIT_WS_H];
    qkv[s] = wsb + L.off[s][MMDIT_WS_QKV];
    x1[s] = reinterpret_cast<float*>(wsb + L.off[s][MMDIT_WS_X1]);
    g[s] = wsb + L.off[s][MMDIT_WS_G];
    xq[s] = wsb + L.off[s][MMDIT_WS_XQ];
    xsc[s] = reinterpret_cast<float*>(wsb + L.off[s][MMDIT_WS_XS]);
    a8[s] = mmdit_attn8_stream{wsb + L.off[s][MMDIT_WS_Q8], reinterpret_cast<float*>(wsb + L.off[s][MMDIT_WS_QS]),
                               wsb + L.off[s][MMDIT_WS_K8], reinterpret_cast<float*>(wsb + L.off[s][MMDIT_WS_KS]),
                               wsb + L.off[s][MMDIT_WS_V8T]};
  }
  float* vscale = reinterpret_cast<float*>(wsb + L.off[0][MMDIT_WS_VS]);
  float* split = reinterpret_cast<float*>(wsb + L.off[0][MMDIT_WS_SPLIT]);
  // per-token FP8 codes of each stream's f16 GEMM input x_s [B * n_s, K]
  auto quantize_inputs = [&](void* const* x, int64_t K) -> int {
    for (int s = 0; s < nstreams; ++s)
      if (int r = launch_quantize_fp8(x[s], MMDIT_F16, B * ns[s], K, 1, xq[s], xsc[s], sm)) return r;
    return MMDIT_OK;
  };
  GemmProblem p[2];
  auto problems = [&](auto fill) {
    for (int s = 0; s < nstreams; ++s) {
      p[s] = GemmProblem{};
      p[s].M = B * ns[s];
      p[s].rows_per_batch = ns[s];
      p[s].x = xq[s];
      p[s].x_scale = xsc[s];
      fill(s, p[s]);
    }
  };

  // S1 modulation vectors; S2 LN-modulate for the attention branch (f16 h)
  if ((st = mark(MMDIT_STAGE_MOD_LN1, 0))) return st;
  for (int s = 0; s < nstreams; ++s) {
    if ((st = launch_modulation(ws[s]->w_mod, ws[s]->b_mod, tvec, t_dtype, mod[s], B, 6 * C, d.Dt, sm))) return st;
    if ((st = launch_modulate_ln(xs[s], x_dtype, nullptr, MMDIT_BF16, nullptr, nullptr, mod[s] + 0, mod[s] + C,
                                 6 * C, hbuf[s], MMDIT_F16, B, ns[s], C, d.ln_eps, sm))) return st;
  }
  if ((st = mark(MMDIT_STAGE_MOD_LN1, 1))) return st;
  // S3 QKV projection on FP8 operands
  if ((st = mark(MMDIT_STAGE_QKV, 0))) return st;
  if ((st = quantize_inputs(hbuf, C))) return st;
  problems([&](int s, GemmProblem& q) { q.w = ws[s]->w_qkv; q.w_scale = ws[s]->s_qkv; q.bias = ws[s]->b_qkv; q.y = qkv[s]; });
  if ((st = launch_linear(p, nstreams, MMDIT_FP8_E4M3, MMDIT_BF16, MMDIT_F16, 3 * C, C, MMDIT_EPI_NONE, MMDIT_F32, sm))) return st;
  if ((st = mark(MMDIT_STAGE_QKV, 1))) return st;
  // S4 QK RMSNorm (+ RoPE on the visual stream), in place in the packed qkv rows
  if ((st = mark(MMDIT_STAGE_QK_NORM_ROPE, 0))) return st;
  for (int s = 0; s < nstreams; ++s) {
    uint16_t* base = static_cast<uint16_t*>(qkv[s]);
    if ((st = launch_qk_norm_rope(base, base + C, MMDIT_F16, 3 * C, ws[s]->q_norm, ws[s]->k_norm, MMDIT_BF16,
                                  d.qk_scale_head_stride, base, base + C, MMDIT_F16, 3 * C, B, ns[s], H, d.qk_eps,
                                  s == 0 ? rope : nullptr, sm))) return st;
  }
  if ((st = mark(MMDIT_STAGE_QK_NORM_ROPE, 1))) return st;
  // S5 8-bit joint attention -> O (f16) in the h region
  if ((st = mark(MMDIT_STAGE_ATTENTION, 0))) return st;
  {
    const uint16_t* qv = static_cast<const uint16_t*>(qkv[0]);
    const uint16_t* qc = ns[1] > 0 ? static_cast<const uint16_t*>(qkv[1]) : nullptr;
    const void* q[2] = {qv, qc};
    const void* k[2] = {qv + C, qc ? qc + C : nullptr};
    const void* v[2] = {qv + 2 * C, qc ? qc + 2 * C : nullptr};
    const mmdit_attn8_stream* seg[2] = {&a8[0], ns[1] > 0 ? &a8[1] : nullptr};
    if ((st = launch_attn8_quantize(q, k, v, ns, MMDIT_F16, 3 * C, B, H, seg, vscale, sm))) return st;
    if ((st = launch_joint_attention_8bit(seg, ns, vscale, B, H, 1.0f / sqrtf((float)d.D), hbuf[0],
                                          ns[1] > 0 ? hbuf[1] : nullptr, MMDIT_F16, C, nullptr, sm, split,
                                          BLOCK_SPLIT_BYTES))) return st;
  }
  if ((st = mark(MMDIT_STAGE_ATTENTION, 1))) return st;
  // S6 output projection with the attention gate: x1 = x + gate_a (O W_o^T + b_o), f32
  if ((st = mark(MMDIT_STAGE_OUT_PROJ, 0))) return st;
  if ((st = quantize_inputs(hbuf, C))) return st;
  problems([&](int s, GemmProblem& q) {
    q.w = ws[s]->w_o; q.w_scale = ws[s]->s_o; q.bias = ws[s]->b_o; q.y = x1[s]; q.res = xs[s];
    q.gate = mod[s] + 2 * C; q.gate_stride = 6 * C;
  });
  if ((st = launch_linear(p, nstreams, MMDIT_FP8_E4M3, MMDIT_BF16, MMDIT_F32, C, C, MMDIT_EPI_GATED_RES, x_dtype, sm))) return st;
  if ((st = mark(MMDIT_STAGE_OUT_PROJ, 1))) return st;
  // S7 LN-modulate for the FFN branch -> h2 (f16) in the qkv region
  if ((st = mark(MMDIT_STAGE_LN2, 0))) return st;
  for (int s = 0; s < nstreams; ++s)
    if ((st = launch_modulate_ln(x1[s], MMDIT_F32, nullptr, MMDIT_F32, nullptr, nullptr, mod[s] + 3 * C, mod[s] + 4 * C,
                                 6 * C, qkv[s], MMDIT_F16, B, ns[s], C, d.ln_eps, sm))) return st;
  if ((st = mark(MMDIT_STAGE_LN2, 1))) return st;
  // S8 FFN up + GELU -> g (f16)
  if ((st = mark(MMDIT_STAGE_FFN_UP, 0))) return st;
  if ((st = quantize_inputs(qkv, C))) return st;
  problems([&](int s, GemmProblem& q) { q.w = ws[s]->w_fc1; q.w_scale = ws[s]->s_fc1; q.bias = ws[s]->b_fc1; q.y = g[s]; });
  if ((st = launch_linear(p, nstreams, MMDIT_FP8_E4M3, MMDIT_BF16, MMDIT_F16, F, C, MMDIT_EPI_GELU, MMDIT_F32, sm))) return st;
  if ((st = mark(MMDIT_STAGE_FFN_UP, 1))) return st;
  // S9 FFN down with the FFN gate: out = x1 + gate_f (g W_2^T + b_2)
  if ((st = mark(MMDIT_STAGE_FFN_DOWN, 0))) return st;
  if ((st = quantize_inputs(g, F))) return st;
  problems([&](int s, GemmProblem& q) {
    q.w = ws[s]->w_fc2; q.w_scale = ws[s]->s_fc2; q.bias = ws[s]->b_fc2; q.y = outs[s]; q.res = x1[s];
    q.gate = mod[s] + 5 * C; q.gate_stride = 6 * C;
  });
  if ((st = launch_linear(p, nstreams, MMDIT_FP8_E4M3, MMDIT_BF16, out_dtype, C, F, MMDIT_EPI_GATED_RES, MMDIT_F32, sm))) return st;
  return mark(MMDIT_STAGE_FFN_DOWN, 1);
}

}  // namespace mmdit

using namespace mmdit;

extern "C" {

size_t mmdit_block_workspace_bytes(const mmdit_block_dims* dims, int64_t B, int64_t n_vis, int64_t n_cond) {
  if (validate_dims(dims, B, n_vis, n_cond) != MMDIT_OK) return 0;
  WsLayout L;
  layout(dims, B, n_vis, n_cond, &L);
  return L.total;
}

int mmdit_block_workspace_offsets(const mmdit_block_dims* dims, int64_t B, int64_t n_vis, int64_t n_cond,
                                  size_t* offsets) {
  const int r = validate_dims(dims, B, n_vis, n_cond);
  if (r) return r;
  if (!offsets) return fail(MMDIT_ERR_NULL, "block: offsets is NULL");
  WsLayout L;
  layout(dims, B, n_vis, n_cond, &L);
  for (int s = 0; s < 2; ++s)
    for (int i = 0; i < MMDIT_WS_COUNT; ++i) offsets[s * MMDIT_WS_COUNT + i] = L.off[s][i];
  return MMDIT_OK;
}

int mmdit_block_fwd_events(const mmdit_block_dims* dims, const mmdit_stream_weights* w_vis,
                           const mmdit_stream_weights* w_cond, const void* x_vis, const void* x_cond,
                           int x_dtype, const void* tvec, int t_dtype, const mmdit_rope3d* rope,
                           int64_t n_cond, void* out_vis, void* out_cond, int out_dtype, void* workspace,
                           size_t workspace_bytes, int64_t B, void* stream, void* const* events) {
  set_error("");
  if (!rope) return fail(MMDIT_ERR_NULL, "block: rope is required (visual grid)");
  if (rope->T < 1 || rope->H < 1 || rope->W < 1 || !extents_ok({rope->T, rope->H, rope->W}))
    return fail(MMDIT_ERR_SHAPE, "block: the visual grid must be non-empty and of a representable size");
  const int64_t n_vis = rope->T * rope->H * rope->W;
  int st = validate_dims(dims, B, n_vis, n_cond);
  if (st) return st;
  const mmdit_block_dims& d = *dims;
  if ((st = validate_rope(rope, n_vis, d.D))) return st;
  if (x_dtype != MMDIT_BF16 && x_dtype != MMDIT_F32) return fail(MMDIT_ERR_DTYPE, "block: x must be bf16 or f32");
  if (t_dtype != MMDIT_BF16 && t_dtype != MMDIT_F32) return fail(MMDIT_ERR_DTYPE, "block: tvec must be bf16 or f32");
  if (out_dtype != MMDIT_F32 && out_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, "block: out must be f32 or bf16");
  if (!w_vis || !w_cond || !x_vis || !tvec || !out_vis || !workspace) return fail(MMDIT_ERR_NULL, "block: null pointer");
  if (n_cond > 0 && (!x_cond || !out_cond)) return fail(MMDIT_ERR_NULL, "block: conditioning pointers required");
  const mmdit_stream_weights* ws[2] = {w_vis, w_cond};
  for (int s = 0; s < 2; ++s) {
    const mmdit_stream_weights& w = *ws[s];
    if (s == 1 && n_cond == 0) continue;
    if (!w.w_mod || !w.w_qkv || !w.q_norm || !w.k_norm || !w.w_o || !w.w_fc1 || !w.w_fc2)
      return fail(MMDIT_ERR_NULL, "block: weight matrices and QK-norm scales are required");
    const void* ps[12] = {w.w_mod, w.b_mod, w.w_qkv, w.b_qkv, w.q_norm, w.k_norm, w.w_o, w.b_o, w.w_fc1, w.b_fc1, w.w_fc2, w.b_fc2};
    for (const void* p : ps)
      if (p && !aligned16(p)) return fail(MMDIT_ERR_ALIGN, "block: weights must be 16-byte aligned");
    if (dims->w_dtype == MMDIT_FP8_E4M3) {
      const float* sc[4] = {w.s_qkv, w.s_o, w.s_fc1, w.s_fc2};
      for (const float* p : sc) {
        if (!p) return fail(MMDIT_ERR_NULL, "block: E4M3 matrices need their scales s_qkv, s_o, s_fc1, s_fc2");
        if (reinterpret_cast<uintptr_t>(p) & 3) return fail(MMDIT_ERR_ALIGN, "block: weight scales must be 4-byte aligned");
      }
    }
  }
  if (!aligned16(x_vis) || (x_cond && !aligned16(x_cond)) || !aligned16(tvec) || !aligned16(out_vis) ||
      (out_cond && !aligned16(out_cond)) || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(MMDIT_ERR_ALIGN, "block: activations 16-byte aligned, workspace 256-byte aligned");
  WsLayout L;
  layout(dims, B, n_vis, n_cond, &L);
  if (workspace_bytes < L.total) return fail(MMDIT_ERR_WORKSPACE, "block: workspace too small");

  hipStream_t sm = static_cast<hipStream_t>(stream);
  auto mark = [&](int stage, int end) -> int {
    if (!events || !events[2 * stage + end]) return MMDIT_OK;
    const hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[2 * stage + end]), sm);
    return e == hipSuccess ? MMDIT_OK : fail(MMDIT_ERR_HIP, std::string("hipEventRecord: ") + hipGetErrorString(e));
  };
  uint8_t* wsb = static_cast<uint8_t*>(workspace);
  const int64_t C = d.C, F = d.F, H = d.H;
  const int64_t ns[2] = {n_vis, n_cond};
  const void* xs[2] = {x_vis, x_cond};
  void* outs[2] = {out_vis, out_cond};
  float* mod[2];
  void *hbuf[2], *qkv[2], *g[2];
  float* x1[2];
  const void *wqkv[2], *wo[2], *w1[2], *w2[2];
  for (int s = 0; s < 2; ++s) {
    mod[s] = reinterpret_cast<float*>(wsb + L.off[s][MMDIT_WS_MOD]);
    hbuf[s] = wsb + L.off[s][MMDIT_WS_H];
    qkv[s] = wsb + L.off[s][MMDIT_WS_QKV];
    x1[s] = reinterpret_cast<float*>(wsb + L.off[s][MMDIT_WS_X1]);
    g[s] = wsb + L.off[s][MMDIT_WS_G];
    wqkv[s] = ws[s]->w_qkv;
    wo[s] = ws[s]->w_o;
    w1[s] = ws[s]->w_fc1;
    w2[s] = ws[s]->w_fc2;
  }
  const int nstreams = n_cond > 0 ? 2 : 1;
  const int act = d.act_dtype;
  float* split = reinterpret_cast<float*>(wsb + L.off[0][MMDIT_WS_SPLIT]);
  if (d.w_dtype == MMDIT_FP8_E4M3)
    return block_fwd_8bit(d, ws, xs, x_dtype, tvec, t_dtype, rope, ns, outs, out_dtype, wsb, L, B, sm, mark);

  // S1 modulation vectors; S2 LN-modulate for the attention branch
  if ((st = mark(MMDIT_STAGE_MOD_LN1, 0))) return st;
  for (int s = 0; s < nstreams; ++s) {
    if ((st = launch_modulation(ws[s]->w_mod, ws[s]->b_mod, tvec, t_dtype, mod[s], B, 6 * C, d.Dt, sm))) return st;
    if ((st = launch_modulate_ln(xs[s], x_dtype, nullptr, MMDIT_BF16, nullptr, nullptr, mod[s] + 0, mod[s] + C,
                                 6 * C, hbuf[s], act, B, ns[s], C, d.ln_eps, sm))) return st;
    if (act != d.w_dtype) {
      const void* src[4] = {ws[s]->w_qkv, ws[s]->w_o, ws[s]->w_fc1, ws[s]->w_fc2};
      const void** dst[4] = {&wqkv[s], &wo[s], &w1[s], &w2[s]};
      const int region[4] = {MMDIT_WS_WQKV, MMDIT_WS_WO, MMDIT_WS_W1, MMDIT_WS_W2};
      const int64_t count[4] = {3 * C * C, C * C, F * C, C * F};
      for (int i = 0; i < 4; ++i) {
        void* copy = wsb + L.off[s][region[i]];
        if ((st = launch_convert_bf16_to_f16(src[i], copy, count[i], sm))) return st;
        *dst[i] = copy;
      }
    }
  }
  if ((st = mark(MMDIT_STAGE_MOD_LN1, 1))) return st;
  GemmProblem p[2];
  auto problems = [&](auto fill) {
    for (int s = 0; s < nstreams; ++s) { p[s] = GemmProblem{}; p[s].M = B * ns[s]; p[s].rows_per_batch = ns[s]; fill(s, p[s]); }
  };
  // S3 QKV projection
  problems([&](int s, GemmProblem& q) { q.x = hbuf[s]; q.w = wqkv[s]; q.bias = ws[s]->b_qkv; q.y = qkv[s]; });
  if ((st = mark(MMDIT_STAGE_QKV, 0))) return st;
  if ((st = launch_linear(p, nstreams, act, MMDIT_BF16, act, 3 * C, C, MMDIT_EPI_NONE, MMDIT_F32, sm, split, BLOCK_SPLIT_BYTES))) return st;
  if ((st = mark(MMDIT_STAGE_QKV, 1))) return st;
  // S4 QK RMSNorm (+ RoPE on the visual stream), in place in the packed qkv rows
  if ((st = mark(MMDIT_STAGE_QK_NORM_ROPE, 0))) return st;
  for (int s = 0; s < nstreams; ++s) {
    uint16_t* base = static_cast<uint16_t*>(qkv[s]);
    if ((st = launch_qk_norm_rope(base, base + C, act, 3 * C, ws[s]->q_norm, ws[s]->k_norm, MMDIT_BF16,
                                  d.qk_scale_head_stride, base, base + C, act, 3 * C, B, ns[s], H, d.qk_eps,
                                  s == 0 ? rope : nullptr, sm))) return st;
  }
  if ((st = mark(MMDIT_STAGE_QK_NORM_ROPE, 1))) return st;
  // S5 joint attention -> O (bf16) in the h region
  if ((st = mark(MMDIT_STAGE_ATTENTION, 0))) return st;
  {
    const uint16_t* qv = static_cast<const uint16_t*>(qkv[0]);
    const uint16_t* qc = n_cond > 0 ? static_cast<const uint16_t*>(qkv[1]) : nullptr;
    if ((st = launch_joint_attention(qv, qv + C, qv + 2 * C, n_vis, qc, qc ? qc + C : nullptr, qc ? qc + 2 * C : nullptr,
                                     n_cond, act, act, 3 * C, B, H, 1.0f / sqrtf((float)d.D), hbuf[0],
                                     n_cond > 0 ? hbuf[1] : nullptr, act, C, nullptr, sm, split,
                                     BLOCK_SPLIT_BYTES))) return st;
  }
  if ((st = mark(MMDIT_STAGE_ATTENTION, 1))) return st;
  // S6 output projection with the attention gate: x1 = x + gate_a (O W_o^T + b_o), f32
  problems([&](int s, GemmProblem& q) {
    q.x = hbuf[s]; q.w = wo[s]; q.bias = ws[s]->b_o; q.y = x1[s]; q.res = xs[s];
    q.gate = mod[s] + 2 * C; q.gate_stride = 6 * C;
  });
  if ((st = mark(MMDIT_STAGE_OUT_PROJ, 0))) return st;
  if ((st = launch_linear(p, nstreams, act, MMDIT_BF16, MMDIT_F32, C, C, MMDIT_EPI_GATED_RES, x_dtype, sm, split, BLOCK_SPLIT_BYTES))) return st;
  if ((st = mark(MMDIT_STAGE_OUT_PROJ, 1))) return st;
  if ((st = mark(MMDIT_STAGE_LN2, 0))) return st;
  // S7 LN-modulate for the FFN branch -> h2 in the qkv region
  for (int s = 0; s < nstreams; ++s)
    if ((st = launch_modulate_ln(x1[s], MMDIT_F32, nullptr, MMDIT_F32, nullptr, nullptr, mod[s] + 3 * C, mod[s] + 4 * C,
                                 6 * C, qkv[s], act, B, ns[s], C, d.ln_eps, sm))) return st;
  if ((st = mark(MMDIT_STAGE_LN2, 1))) return st;
  // S8 FFN up + GELU
  problems([&](int s, GemmProblem& q) { q.x = qkv[s]; q.w = w1[s]; q.bias = ws[s]->b_fc1; q.y = g[s]; });
  if ((st = mark(MMDIT_STAGE_FFN_UP, 0))) return st;
  if ((st = launch_linear(p, nstreams, act, MMDIT_BF16, act, F, C, MMDIT_EPI_GELU, MMDIT_F32, sm, split, BLOCK_SPLIT_BYTES))) return st;
  if ((st = mark(MMDIT_STAGE_FFN_UP, 1))) return st;
  // S9 FFN down with the FFN gate: out = x1 + gate_f (g W_2^T + b_2)
  problems([&](int s, GemmProblem& q) {
    q.x = g[s]; q.w = w2[s]; q.bias = ws[s]->b_fc2; q.y = outs[s]; q.res = x1[s];
    q.gate = mod[s] + 5 * C; q.gate_stride = 6 * C;
  });
  if ((st = mark(MMDIT_STAGE_FFN_DOWN, 0))) return st;
  if ((st = launch_linear(p, nstreams, act, MMDIT_BF16, out_dtype, C, F, MMDIT_EPI_GATED_RES, MMDIT_F32, sm, split, BLOCK_SPLIT_BYTES))) return st;
  if ((st = mark(MMDIT_STAGE_FFN_DOWN, 1))) return st;
  return MMDIT_OK;
}

int mmdit_block_fwd(const mmdit_block_dims* dims, const mmdit_stream_weights* w_vis,
                    const mmdit_stream_weights* w_cond, const void* x_vis, const void* x_cond,
                    int x_dtype, const void* tvec, int t_dtype, const mmdit_rope3d* rope,
                    int64_t n_cond, void* out_vis, void* out_cond, int out_dtype, void* workspace,
                    size_t workspace_bytes, int64_t B, void* stream) {
  return mmdit_block_fwd_events(dims, w_vis, w_cond, x_vis, x_cond, x_dtype, tvec, t_dtype, rope, n_cond,
                                out_vis, out_cond, out_dtype, workspace, workspace_bytes, B, stream, nullptr);
}

}  // extern "C"
