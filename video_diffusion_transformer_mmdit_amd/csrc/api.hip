// extern "C" entry points of libmmdit: argument validation, then dispatch to the kernels.
// Every check runs before anything is enqueued, so a rejected call touches no HIP state.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "common.h"

namespace mmdit {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
int fail(int status, const std::string& msg) {
  g_last_error = std::string(mmdit_status_str(status)) + ": " + msg;
  return status;
}
int device_cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];   // 0: not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MMDIT_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return MMDIT_OK;
}

static bool valid_dtype(int dt) { return dt == MMDIT_F32 || dt == MMDIT_BF16 || dt == MMDIT_F16; }

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// bytes spanned by `rows` rows of `row_elems` elements at `stride` elements
static size_t span(int64_t rows, int64_t row_elems, int64_t stride, int dt) {
  if (rows <= 0) return 0;
  return (size_t)((rows - 1) * stride + row_elems) * (size_t)dtype_size(dt);
}

int validate_rope(const mmdit_rope3d* r, int64_t N, int64_t D) {
  if (r->T < 1 || r->H < 1 || r->W < 1) return fail(MMDIT_ERR_SHAPE, "rope: T, H, W must be >= 1");
  if (!extents_ok({r->T, r->H, r->W})) return fail(MMDIT_ERR_SHAPE, "rope: T * H * W too large");
  if (r->d_t < 0 || r->d_h < 0 || r->d_w < 0 || (r->d_t & 1) || (r->d_h & 1) || (r->d_w & 1))
    return fail(MMDIT_ERR_SHAPE, "rope: band widths must be even and >= 0");
  if ((int64_t)r->d_t + r->d_h + r->d_w != D) return fail(MMDIT_ERR_SHAPE, "rope: d_t + d_h + d_w != D");
  if (!(r->base > 0.f)) return fail(MMDIT_ERR_SHAPE, "rope: base must be > 0");
  if (r->T * r->H * r->W != N) return fail(MMDIT_ERR_SHAPE, "rope: N != T * H * W");
  return MMDIT_OK;
}

// Scratch of mmdit_joint_attention_noalloc: the key-range results of the attention's split
// tail (at most 256 slots of one 256-query tile's unnormalised O, 256 x 128 f32, and (m, l)
// per query).  Each device holds its own copy for the life of the process; its address is
// taken once per device, with that device current, and only that address reaches the kernels.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)256 * (256 * 128 + 256 * 2) * 4;
static_assert(NOALLOC_SCRATCH_BYTES == MMDIT_NOALLOC_SCRATCH_BYTES, "scratch size and header disagree");
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];
constexpr int NOALLOC_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};

// The scratch address on the device that runs `stream` (the current device for the null
// stream).  The first call on a device makes that device current for the lookup and then
// restores the caller's.
static int noalloc_scratch(void* stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MMDIT_ERR_HIP, std::string("noalloc: device of the stream: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return fail(MMDIT_ERR_HIP, "noalloc: device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess || !p)
      return fail(MMDIT_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MMDIT_OK;
}

}  // namespace mmdit

using namespace mmdit;

extern "C" {

const char* mmdit_status_str(int s) {
  switch (s) {
    case MMDIT_OK: return "MMDIT_OK";
    case MMDIT_ERR_NULL: return "MMDIT_ERR_NULL";
    case MMDIT_ERR_ALIGN: return "MMDIT_ERR_ALIGN";
    case MMDIT_ERR_SHAPE: return "MMDIT_ERR_SHAPE";
    case MMDIT_ERR_DTYPE: return "MMDIT_ERR_DTYPE";
    case MMDIT_ERR_WORKSPACE: return "MMDIT_ERR_WORKSPACE";
    case MMDIT_ERR_HIP: return "MMDIT_ERR_HIP";
    case MMDIT_ERR_ALIAS: return "MMDIT_ERR_ALIAS";
    default: return "MMDIT_ERR_UNKNOWN";
  }
}

const char* mmdit_last_error(void) { return g_last_error.c_str(); }

int mmdit_abi_version(void) { return 8; }

int mmdit_modulate_ln(const void* x, int x_dtype, const void* branch, int branch_dtype,
                      const float* gate, float* x_out, const float* shift, const float* scale,
                      int64_t mod_stride, void* y, int y_dtype, int64_t B, int64_t N, int64_t C,
                      float eps, void* stream) {
  g_last_error.clear();
  if (B < 0 || N < 0 || C < 8 || C % 8 || C > 8192)
    return fail(MMDIT_ERR_SHAPE, "modulate_ln: need B, N >= 0 and C a multiple of 8 in [8, 8192]");
  if (mod_stride < C) return fail(MMDIT_ERR_SHAPE, "modulate_ln: mod_stride < C");
  if (!extents_ok({B, N, C}) || !extents_ok({B, mod_stride})) return fail(MMDIT_ERR_SHAPE, "modulate_ln: sizes too large");
  if (!(eps >= 0.f)) return fail(MMDIT_ERR_SHAPE, "modulate_ln: eps must be >= 0");
  if (x_dtype != MMDIT_F32 && x_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, "modulate_ln: x must be f32 or bf16");
  if (branch && branch_dtype != MMDIT_F32 && branch_dtype != MMDIT_BF16)
    return fail(MMDIT_ERR_DTYPE, "modulate_ln: branch must be f32 or bf16");
  if (!valid_dtype(y_dtype)) return fail(MMDIT_ERR_DTYPE, "modulate_ln: bad y dtype");
  if (B * N == 0) return MMDIT_OK;
  if (!x || !shift || !scale || !y) return fail(MMDIT_ERR_NULL, "modulate_ln: x, shift, scale and y are required");
  if (branch && !gate) return fail(MMDIT_ERR_NULL, "modulate_ln: gate is required with branch");
  if (!aligned16(x) || !aligned16(y) || (branch && !aligned16(branch)) || (x_out && !aligned16(x_out)) ||
      !aligned16(shift) || !aligned16(scale) || (gate && !aligned16(gate)) || (mod_stride % 4))
    return fail(MMDIT_ERR_ALIGN, "modulate_ln: pointers must be 16-byte aligned, mod_stride a multiple of 4");
  const int64_t rows = B * N;
  const size_t ny = span(rows, C, C, y_dtype), nx = span(rows, C, C, x_dtype);
  const size_t nxo = x_out ? span(rows, C, C, MMDIT_F32) : 0;
  const size_t nb = branch ? span(rows, C, C, branch_dtype) : 0;
  if (overlaps(y, ny, x, nx) || overlaps(y, ny, branch, nb) || overlaps(x_out, nxo, x, nx) ||
      overlaps(x_out, nxo, branch, nb) || overlaps(x_out, nxo, y, ny))
    return fail(MMDIT_ERR_ALIAS, "modulate_ln: outputs overlap inputs");
  return launch_modulate_ln(x, x_dtype, branch, branch_dtype, gate, x_out, shift, scale, mod_stride, y,
                            y_dtype, B, N, C, eps, static_cast<hipStream_t>(stream));
}

int mmdit_qk_norm_rope(const void* q, const void* k, int in_dtype, int64_t in_row_stride,
                       const void* q_scale, const void* k_scale, int scale_dtype,
                       int64_t scale_head_stride, void* q_out, void* k_out, int out_dtype,
                       int64_t out_row_stride, int64_t B, int64_t N, int64_t H, int64_t D,
                       float eps, const mmdit_rope3d* rope, void* stream) {
  g_last_error.clear();
  if (D != 128) return fail(MMDIT_ERR_SHAPE, "qk_norm_rope: D must be 128");
  if (B < 0 || N < 0 || H < 1 || H > 4096) return fail(MMDIT_ERR_SHAPE, "qk_norm_rope: need B, N >= 0, 1 <= H <= 4096");
  if (!extents_ok({B, N, in_row_stride}) || !extents_ok({B, N, out_row_stride}))
    return fail(MMDIT_ERR_SHAPE, "qk_norm_rope: sizes too large");
  if (in_row_stride < H * D || out_row_stride < H * D) return fail(MMDIT_ERR_SHAPE, "qk_norm_rope: row stride < H*D");
  if (scale_head_stride != 0 && scale_head_stride != D)
    return fail(MMDIT_ERR_SHAPE, "qk_norm_rope: scale_head_stride must be 0 or D");
  if (!(eps >= 0.f)) return fail(MMDIT_ERR_SHAPE, "qk_norm_rope: eps must be >= 0");
  if (!valid_dtype(in_dtype)) return fail(MMDIT_ERR_DTYPE, "qk_norm_rope: bad in dtype");
  if (scale_dtype != MMDIT_F32 && scale_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, "qk_norm_rope: scale dtype must be f32 or bf16");
  if (!valid_dtype(out_dtype)) return fail(MMDIT_ERR_DTYPE, "qk_norm_rope: bad out dtype");
  if (in_dtype == MMDIT_F32 && out_dtype == MMDIT_F16) return fail(MMDIT_ERR_DTYPE, "qk_norm_rope: f32 -> f16 not supported");
  if (rope) { const int r = validate_rope(rope, N, D); if (r) return r; }
  if (B * N == 0) return MMDIT_OK;
  if (!q || !k || !q_scale || !k_scale || !q_out || !k_out) return fail(MMDIT_ERR_NULL, "qk_norm_rope: null pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_out) || !aligned16(k_out) || !aligned16(q_scale) ||
      !aligned16(k_scale) || (in_row_stride % 8) || (out_row_stride % 8))
    return fail(MMDIT_ERR_ALIGN, "qk_norm_rope: pointers 16-byte aligned, strides multiples of 8 elements");
  const int64_t rows = B * N, hd = H * D;
  const size_t nq = span(rows, hd, in_row_stride, in_dtype), nqo = span(rows, hd, out_row_stride, out_dtype);
  const bool q_inplace = q_out == q, k_inplace = k_out == k;
  if ((q_inplace || k_inplace) && (in_dtype != out_dtype || in_row_stride != out_row_stride))
    return fail(MMDIT_ERR_ALIAS, "qk_norm_rope: in place needs equal dtypes and strides");
  // Outputs may only coincide exactly with their own input.  With a shared packed row
  // (q, k, v of one token in one row) the spans interleave, so check per-row extents.
  auto rows_clash = [&](const void* o, const void* i, int odt, int idt) {
    const uintptr_t po = reinterpret_cast<uintptr_t>(o), pi = reinterpret_cast<uintptr_t>(i);
    const int64_t so = out_row_stride * dtype_size(odt), si = in_row_stride * dtype_size(idt);
    const int64_t lo = hd * dtype_size(odt), li = hd * dtype_size(idt);
    if (so == si) {  // same row pitch: compare the in-row windows
      const int64_t delta = (int64_t)po - (int64_t)pi;
      int64_t r = delta % so;
      if (r < 0) r += so;
      const bool hit = (r < li) || (so - r < lo);
      return hit && overlaps(o, nqo, i, nq);
    }
    return overlaps(o, nqo, i, nq);
  };
  if ((!q_inplace && rows_clash(q_out, q, out_dtype, in_dtype)) || rows_clash(q_out, k, out_dtype, in_dtype) ||
      (!k_inplace && rows_clash(k_out, k, out_dtype, in_dtype)) || rows_clash(k_out, q, out_dtype, in_dtype) ||
      rows_clash(q_out, k_out, out_dtype, out_dtype))
    return fail(MMDIT_ERR_ALIAS, "qk_norm_rope: outputs partially overlap inputs");
  return launch_qk_norm_rope(q, k, in_dtype, in_row_stride, q_scale, k_scale, scale_dtype,
                             scale_head_stride, q_out, k_out, out_dtype, out_row_stride, B, N, H,
                             eps, rope, static_cast<hipStream_t>(stream));
}

int mmdit_joint_attention(const void* q_vis, const void* k_vis, const void* v_vis, int64_t n_vis,
                          const void* q_cond, const void* k_cond, const void* v_cond, int64_t n_cond,
                          int qk_dtype, int v_dtype, int64_t in_row_stride, int64_t B, int64_t H, int64_t D,
                          float softmax_scale, void* o_vis, void* o_cond, int out_dtype,
                          int64_t out_row_stride, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  g_last_error.clear();
  if (D != 128) return fail(MMDIT_ERR_SHAPE, "joint_attention: D must be 128");
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(MMDIT_ERR_ALIGN, "joint_attention: workspace must be 256-byte aligned");
  if (!extents_ok({B}) || !extents_ok({H}) || !extents_ok({n_vis}) || !extents_ok({n_cond}))
    return fail(MMDIT_ERR_SHAPE, "joint_attention: sizes must be >= 0 and below 2^31");
  if (H < 1 || n_vis + n_cond < 1)
    return fail(MMDIT_ERR_SHAPE, "joint_attention: need B >= 0, H >= 1, n_vis + n_cond >= 1");
  if (H > 4096 || !extents_ok({B, n_vis, in_row_stride}) || !extents_ok({B, n_cond, in_row_stride}) ||
      !extents_ok({B, n_vis, out_row_stride}) || !extents_ok({B, n_cond, out_row_stride}) ||
      !extents_ok({B, H, n_vis + n_cond}))
    return fail(MMDIT_ERR_SHAPE, "joint_attention: sizes too large");
  if (in_row_stride < H * D || out_row_stride < H * D) return fail(MMDIT_ERR_SHAPE, "joint_attention: row stride < H*D");
  if (!(softmax_scale > 0.f)) return fail(MMDIT_ERR_SHAPE, "joint_attention: softmax_scale must be > 0");
  if (!valid_dtype(qk_dtype) || !valid_dtype(v_dtype) || ((qk_dtype == MMDIT_F32) != (v_dtype == MMDIT_F32)))
    return fail(MMDIT_ERR_DTYPE, "joint_attention: Q/K and V must be 16-bit (f16 / bf16) or all f32");
  if (!valid_dtype(out_dtype)) return fail(MMDIT_ERR_DTYPE, "joint_attention: bad out dtype");
  if (B == 0) return MMDIT_OK;
  if (n_vis > 0 && (!q_vis || !k_vis || !v_vis || !o_vis)) return fail(MMDIT_ERR_NULL, "joint_attention: visual pointers required");
  if (n_cond > 0 && (!q_cond || !k_cond || !v_cond || !o_cond)) return fail(MMDIT_ERR_NULL, "joint_attention: conditioning pointers required");
  const void* ins[6] = {q_vis, k_vis, v_vis, q_cond, k_cond, v_cond};
  const int64_t nin[6] = {n_vis, n_vis, n_vis, n_cond, n_cond, n_cond};
  for (int i = 0; i < 6; ++i)
    if (nin[i] > 0 && !aligned16(ins[i])) return fail(MMDIT_ERR_ALIGN, "joint_attention: inputs must be 16-byte aligned");
  if ((n_vis > 0 && !aligned16(o_vis)) || (n_cond > 0 && !aligned16(o_cond)) || (lse && !aligned16(lse)) ||
      (in_row_stride % 8) || (out_row_stride % 8))
    return fail(MMDIT_ERR_ALIGN, "joint_attention: outputs 16-byte aligned, strides multiples of 8 elements");
  const int64_t hd = H * D;
  const void* outs[2] = {o_vis, o_cond};
  const int64_t nout[2] = {n_vis, n_cond};
  for (int o = 0; o < 2; ++o) {
    if (nout[o] == 0) continue;
    const size_t no = span(B * nout[o], hd, out_row_stride, out_dtype);
    for (int i = 0; i < 6; ++i)
      if (nin[i] > 0 && overlaps(outs[o], no, ins[i], span(B * nin[i], hd, in_row_stride, i % 3 == 2 ? v_dtype : qk_dtype)))
        return fail(MMDIT_ERR_ALIAS, "joint_attention: outputs overlap inputs");
    if (lse && overlaps(outs[o], no, lse, (size_t)(B * H * (n_vis + n_cond)) * 4))
      return fail(MMDIT_ERR_ALIAS, "joint_attention: lse overlaps an output");
  }
  if (n_vis > 0 && n_cond > 0 &&
      overlaps(o_vis, span(B * n_vis, hd, out_row_stride, out_dtype), o_cond, span(B * n_cond, hd, out_row_stride, out_dtype)))
    return fail(MMDIT_ERR_ALIAS, "joint_attention: o_vis and o_cond overlap");
  // the split tail writes key-range results into the workspace while other workgroups read the
  // inputs and write the outputs: it must be disjoint from all of them
  if (workspace && workspace_bytes > 0) {
    for (int i = 0; i < 6; ++i)
      if (nin[i] > 0 && overlaps(workspace, workspace_bytes, ins[i],
                                 span(B * nin[i], hd, in_row_stride, i % 3 == 2 ? v_dtype : qk_dtype)))
        return fail(MMDIT_ERR_ALIAS, "joint_attention: workspace overlaps an input");
    for (int o = 0; o < 2; ++o)
      if (nout[o] > 0 && overlaps(workspace, workspace_bytes, outs[o], span(B * nout[o], hd, out_row_stride, out_dtype)))
        return fail(MMDIT_ERR_ALIAS, "joint_attention: workspace overlaps an output");
    if (lse && overlaps(workspace, workspace_bytes, lse, (size_t)(B * H * (n_vis + n_cond)) * 4))
      return fail(MMDIT_ERR_ALIAS, "joint_attention: workspace overlaps lse");
  }
  return launch_joint_attention(q_vis, k_vis, v_vis, n_vis, q_cond, k_cond, v_cond, n_cond, qk_dtype, v_dtype,
                                in_row_stride, B, H, softmax_scale, o_vis, o_cond, out_dtype,
                                out_row_stride, lse, static_cast<hipStream_t>(stream), static_cast<float*>(workspace),
                                workspace ? workspace_bytes : 0);
}

int mmdit_joint_attention_noalloc(const void* q_vis, const void* k_vis, const void* v_vis, int64_t n_vis,
                                  const void* q_cond, const void* k_cond, const void* v_cond, int64_t n_cond,
                                  int qk_dtype, int v_dtype, int64_t in_row_stride, int64_t B, int64_t H,
                                  int64_t D, float softmax_scale, void* o_vis, void* o_cond, int out_dtype,
                                  int64_t out_row_stride, float* lse, void* stream) {
  g_last_error.clear();
  if (!extents_ok({B}) || !extents_ok({H}) || !extents_ok({n_vis}) || !extents_ok({n_cond}))
    return fail(MMDIT_ERR_SHAPE, "joint_attention_noalloc: sizes must be >= 0 and below 2^31");
  const size_t need = joint_attention_split_bytes(n_vis, n_cond, B, H, qk_dtype, lse != nullptr);
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(MMDIT_ERR_WORKSPACE, "joint_attention_noalloc: the split tail needs " + std::to_string(need) +
                                         " bytes of scratch; the static scratch holds " +
                                         std::to_string(NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  const int st = noalloc_scratch(stream, &ws);
  if (st) return st;
  return mmdit_joint_attention(q_vis, k_vis, v_vis, n_vis, q_cond, k_cond, v_cond, n_cond, qk_dtype, v_dtype,
                               in_row_stride, B, H, D, softmax_scale, o_vis, o_cond, out_dtype, out_row_stride,
                               lse, ws, NOALLOC_SCRATCH_BYTES, stream);
}

int mmdit_linear(const void* x, const void* w, int x_dtype, const void* bias, int bias_dtype,
                 void* y, int y_dtype, int64_t M, int64_t N, int64_t K, int epilogue,
                 const void* res, int res_dtype, const float* gate, int64_t gate_stride,
                 int64_t rows_per_batch, void* stream) {
  g_last_error.clear();
  if (!extents_ok({M}) || !extents_ok({N}) || !extents_ok({K}) || K < 64 || K % 64 || N % 4)
    return fail(MMDIT_ERR_SHAPE, "linear: need M, N >= 0, N a multiple of 4 and K a positive multiple of 64");
  if (!extents_ok({M + 256, K}) || !extents_ok({N + 256, K}) || !extents_ok({M, N}) || !extents_ok({rows_per_batch}) ||
      !extents_ok({gate_stride}) || (M + 256) * K * 2 >= ((int64_t)1 << 31) || (N + 256) * K * 2 >= ((int64_t)1 << 31))
    return fail(MMDIT_ERR_SHAPE, "linear: x or w too large for 32-bit buffer offsets");
  if (x_dtype != MMDIT_BF16 && x_dtype != MMDIT_F16) return fail(MMDIT_ERR_DTYPE, "linear: x/w must be bf16 or f16");
  if (bias && bias_dtype != MMDIT_F32 && bias_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, "linear: bias must be f32 or bf16");
  if (!valid_dtype(y_dtype)) return fail(MMDIT_ERR_DTYPE, "linear: bad y dtype");
  if (epilogue < MMDIT_EPI_NONE || epilogue > MMDIT_EPI_GATED_RES) return fail(MMDIT_ERR_SHAPE, "linear: bad epilogue");
  if (epilogue == MMDIT_EPI_GATED_RES) {
    if (res_dtype != MMDIT_F32 && res_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, "linear: res must be f32 or bf16");
    if (y_dtype == MMDIT_F16) return fail(MMDIT_ERR_DTYPE, "linear: gated residual output must be f32 or bf16");
    if (rows_per_batch < 1 || gate_stride < N || gate_stride % 4)
      return fail(MMDIT_ERR_SHAPE, "linear: rows_per_batch >= 1 and gate_stride >= N, a multiple of 4");
  }
  if (M == 0 || N == 0) return MMDIT_OK;
  if (!x || !w || !y) return fail(MMDIT_ERR_NULL, "linear: x, w, y required");
  if (epilogue == MMDIT_EPI_GATED_RES && (!res || !gate)) return fail(MMDIT_ERR_NULL, "linear: res and gate required");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (bias && !aligned16(bias)) || (res && !aligned16(res)) ||
      (gate && !aligned16(gate)))
    return fail(MMDIT_ERR_ALIGN, "linear: pointers must be 16-byte aligned");
  const size_t ny = (size_t)(M * N) * dtype_size(y_dtype);
  if (overlaps(y, ny, x, (size_t)(M * K) * dtype_size(x_dtype)) || overlaps(y, ny, w, (size_t)(N * K) * dtype_size(x_dtype)) ||
      (res && res != y && overlaps(y, ny, res, (size_t)(M * N) * dtype_size(res_dtype))))
    return fail(MMDIT_ERR_ALIAS, "linear: y overlaps an input");
  GemmProblem p{};
  p.x = x; p.w = w; p.bias = bias; p.y = y; p.res = res; p.gate = gate; p.M = M;
  p.gate_stride = gate_stride; p.rows_per_batch = rows_per_batch > 0 ? rows_per_batch : M;
  return launch_linear(&p, 1, x_dtype, bias_dtype, y_dtype, N, K, epilogue, res_dtype,
                       static_cast<hipStream_t>(stream));
}

int mmdit_attn8_quantize(const void* q_vis, const void* k_vis, const void* v_vis, int64_t n_vis,
                         const void* q_cond, const void* k_cond, const void* v_cond, int64_t n_cond,
                         int in_dtype, int64_t in_row_stride, int64_t B, int64_t H, int64_t D,
                         const mmdit_attn8_stream* vis, const mmdit_attn8_stream* cond, float* v_scale,
                         void* stream) {
  g_last_error.clear();
  if (!extents_ok({B}) || !extents_ok({H}) || !extents_ok({n_vis}) || !extents_ok({n_cond}) || !extents_ok({in_row_stride}))
    return fail(MMDIT_ERR_SHAPE, "attn8_quantize: sizes must be >= 0 and below 2^31");
  if (D != 128) return fail(MMDIT_ERR_SHAPE, "attn8_quantize: D must be 128");
  if (!valid_dtype(in_dtype)) return fail(MMDIT_ERR_DTYPE, "attn8_quantize: inputs must be f32, bf16 or f16");
  if (H > 4096 || !extents_ok({B, n_vis + 64, in_row_stride}) || !extents_ok({B, n_cond + 64, in_row_stride}) ||
      !extents_ok({B, H, 128, n_vis + 64}) || !extents_ok({B, H, 128, n_cond + 64}))
    return fail(MMDIT_ERR_SHAPE, "attn8_quantize: sizes too large");
  if (in_row_stride < H * D || in_row_stride % 8) return fail(MMDIT_ERR_ALIGN, "attn8_quantize: row stride >= H*D, a multiple of 8");
  if (B == 0 || H == 0 || n_vis + n_cond == 0) return MMDIT_OK;
  if (!v_scale) return fail(MMDIT_ERR_NULL, "attn8_quantize: v_scale required");
  const void* qs[2] = {q_vis, q_cond};
  const void* ks[2] = {k_vis, k_cond};
  const void* vs[2] = {v_vis, v_cond};
  const int64_t n[2] = {n_vis, n_cond};
  const mmdit_attn8_stream* out[2] = {vis, cond};
  const size_t es = dtype_size(in_dtype);
  for (int s = 0; s < 2; ++s) {
    if (n[s] == 0) continue;
    const mmdit_attn8_stream* o = out[s];
    if (!qs[s] || !ks[s] || !vs[s] || !o || !o->q8 || !o->q_scale || !o->k8 || !o->k_scale || !o->v8t)
      return fail(MMDIT_ERR_NULL, "attn8_quantize: inputs and every output of a non-empty stream are required");
    if (!aligned16(qs[s]) || !aligned16(ks[s]) || !aligned16(vs[s]) || !aligned16(o->q8) || !aligned16(o->k8) ||
        !aligned16(o->v8t) || (reinterpret_cast<uintptr_t>(o->q_scale) & 3) || (reinterpret_cast<uintptr_t>(o->k_scale) & 3))
      return fail(MMDIT_ERR_ALIGN, "attn8_quantize: tensors 16-byte aligned, scales 4-byte aligned");
    const int64_t nb = (n[s] + 63) / 64;
    if (B * H * 128 * nb * 64 >= ((int64_t)1 << 40) || (128 * nb * 64) >= ((int64_t)1 << 31))
      return fail(MMDIT_ERR_SHAPE, "attn8_quantize: stream too long");
    const size_t in_bytes = (size_t)((B * n[s] - 1) * in_row_stride + H * D) * es;
    const void* outs[5] = {o->q8, o->q_scale, o->k8, o->k_scale, o->v8t};
    const size_t nout[5] = {(size_t)(B * n[s] * H * D), (size_t)(B * H * n[s]) * 4, (size_t)(B * n[s] * H * D),
                            (size_t)(B * H * nb) * 4, (size_t)(B * H * D * nb * 64)};
    for (int i = 0; i < 5; ++i) {
      for (int t = 0; t < 2; ++t)
        if (n[t] > 0 && (overlaps(outs[i], nout[i], qs[t], (size_t)((B * n[t] - 1) * in_row_stride + H * D) * es) ||
                         overlaps(outs[i], nout[i], ks[t], (size_t)((B * n[t] - 1) * in_row_stride + H * D) * es) ||
                         overlaps(outs[i], nout[i], vs[t], (size_t)((B * n[t] - 1) * in_row_stride + H * D) * es)))
          return fail(MMDIT_ERR_ALIAS, "attn8_quantize: an output overlaps an input");
      if (overlaps(outs[i], nout[i], v_scale, (size_t)(B * H * D) * 4))
        return fail(MMDIT_ERR_ALIAS, "attn8_quantize: an output overlaps v_scale");
    }
    (void)in_bytes;
  }
  if (reinterpret_cast<uintptr_t>(v_scale) & 15) return fail(MMDIT_ERR_ALIGN, "attn8_quantize: v_scale 16-byte aligned");
  return launch_attn8_quantize(qs, ks, vs, n, in_dtype, in_row_stride, B, H, out, v_scale,
                               static_cast<hipStream_t>(stream));
}

int mmdit_joint_attention_8bit(const mmdit_attn8_stream* vis, int64_t n_vis, const mmdit_attn8_stream* cond,
                               int64_t n_cond, const float* v_scale, int64_t B, int64_t H, int64_t D,
                               float softmax_scale, void* o_vis, void* o_cond, int out_dtype,
                               int64_t out_row_stride, float* lse, void* workspace, size_t workspace_bytes,
                               void* stream) {
  g_last_error.clear();
  if (!extents_ok({B}) || !extents_ok({H}) || !extents_ok({n_vis}) || !extents_ok({n_cond}) || !extents_ok({out_row_stride}))
    return fail(MMDIT_ERR_SHAPE, "joint_attention_8bit: sizes must be >= 0 and below 2^31");
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(MMDIT_ERR_ALIGN, "joint_attention_8bit: workspace must be 256-byte aligned");
  if (D != 128) return fail(MMDIT_ERR_SHAPE, "joint_attention_8bit: D must be 128");
  if (H > 4096 || !extents_ok({B, n_vis + 64, H, D}) || !extents_ok({B, n_cond + 64, H, D}) ||
      !extents_ok({B, n_vis, out_row_stride}) || !extents_ok({B, n_cond, out_row_stride}))
    return fail(MMDIT_ERR_SHAPE, "joint_attention_8bit: sizes too large");
  if (!valid_dtype(out_dtype)) return fail(MMDIT_ERR_DTYPE, "joint_attention_8bit: bad out dtype");
  if (out_row_stride < H * D || out_row_stride % 8) return fail(MMDIT_ERR_ALIGN, "joint_attention_8bit: out row stride >= H*D, a multiple of 8");
  if (!(softmax_scale > 0.f) || !(softmax_scale < 3.0e38f)) return fail(MMDIT_ERR_SHAPE, "joint_attention_8bit: softmax_scale must be positive and finite");
  if (B == 0 || H == 0 || n_vis + n_cond == 0) return MMDIT_OK;
  const mmdit_attn8_stream* seg[2] = {vis, cond};
  const int64_t n[2] = {n_vis, n_cond};
  void* outs[2] = {o_vis, o_cond};
  if (!v_scale) return fail(MMDIT_ERR_NULL, "joint_attention_8bit: v_scale required");
  if (reinterpret_cast<uintptr_t>(v_scale) & 15) return fail(MMDIT_ERR_ALIGN, "joint_attention_8bit: v_scale 16-byte aligned");
  for (int s = 0; s < 2; ++s) {
    if (n[s] == 0) continue;
    const mmdit_attn8_stream* o = seg[s];
    if (!o || !o->q8 || !o->q_scale || !o->k8 || !o->k_scale || !o->v8t || !outs[s])
      return fail(MMDIT_ERR_NULL, "joint_attention_8bit: every operand and the output of a non-empty stream are required");
    if (!aligned16(o->q8) || !aligned16(o->k8) || !aligned16(o->v8t) || !aligned16(outs[s]) ||
        (reinterpret_cast<uintptr_t>(o->q_scale) & 3) || (reinterpret_cast<uintptr_t>(o->k_scale) & 3))
      return fail(MMDIT_ERR_ALIGN, "joint_attention_8bit: tensors 16-byte aligned, scales 4-byte aligned");
    const int64_t nb = (n[s] + 63) / 64;
    if ((n[s] + 64) * H * D >= ((int64_t)1 << 31) || 128 * nb * 64 >= ((int64_t)1 << 31))
      return fail(MMDIT_ERR_SHAPE, "joint_attention_8bit: one stream spans 2 GiB or more per batch item");
  }
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return fail(MMDIT_ERR_ALIGN, "joint_attention_8bit: lse 4-byte aligned");
  // outputs (and the split tail's workspace) must be disjoint from every operand and from
  // one another: other workgroups are still reading the operands while they are written
  {
    const size_t nlse = lse ? (size_t)(B * H * (n_vis + n_cond)) * 4 : 0;
    const size_t nvs = (size_t)(B * H * D) * 4;
    size_t nout[2] = {0, 0};
    for (int s = 0; s < 2; ++s) nout[s] = n[s] > 0 ? span(B * n[s], H * D, out_row_stride, out_dtype) : 0;
    struct Span { const void* p; size_t n; };
    Span ops[11];
    int nops = 0;
    for (int s = 0; s < 2; ++s) {
      if (n[s] == 0) continue;
      const mmdit_attn8_stream* o = seg[s];
      const int64_t nb = (n[s] + 63) / 64;
      ops[nops++] = {o->q8, (size_t)(B * n[s] * H * D)};
      ops[nops++] = {o->q_scale, (size_t)(B * H * n[s]) * 4};
      ops[nops++] = {o->k8, (size_t)(B * n[s] * H * D)};
      ops[nops++] = {o->k_scale, (size_t)(B * H * nb) * 4};
      ops[nops++] = {o->v8t, (size_t)(B * H * D * nb * 64)};
    }
    ops[nops++] = {v_scale, nvs};
    const Span wr[4] = {{outs[0], nout[0]}, {outs[1], nout[1]}, {lse, nlse},
                        {workspace, workspace ? workspace_bytes : 0}};
    for (int w = 0; w < 4; ++w) {
      for (int i = 0; i < nops; ++i)
        if (overlaps(wr[w].p, wr[w].n, ops[i].p, ops[i].n))
          return fail(MMDIT_ERR_ALIAS, "joint_attention_8bit: an output or the workspace overlaps an operand");
      for (int v = w + 1; v < 4; ++v)
        if (overlaps(wr[w].p, wr[w].n, wr[v].p, wr[v].n))
          return fail(MMDIT_ERR_ALIAS, "joint_attention_8bit: outputs, lse and workspace must not overlap");
    }
  }
  return launch_joint_attention_8bit(seg, n, v_scale, B, H, softmax_scale, o_vis, o_cond, out_dtype, out_row_stride,
                                     lse, static_cast<hipStream_t>(stream), static_cast<float*>(workspace),
                                     workspace ? workspace_bytes : 0);
}

int mmdit_cast(const void* x, int x_dtype, void* y, int y_dtype, int64_t n, void* stream) {
  g_last_error.clear();
  if (!extents_ok({n})) return fail(MMDIT_ERR_SHAPE, "cast: n must be >= 0 and below 2^31");
  if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype) || x_dtype == y_dtype)
    return fail(MMDIT_ERR_DTYPE, "cast: x and y must be two different dtypes of f32, bf16, f16");
  if (n == 0) return MMDIT_OK;
  if (!x || !y) return fail(MMDIT_ERR_NULL, "cast: x and y required");
  if (!aligned16(x) || !aligned16(y)) return fail(MMDIT_ERR_ALIGN, "cast: x and y must be 16-byte aligned");
  const size_t nx = (size_t)n * dtype_size(x_dtype), ny = (size_t)n * dtype_size(y_dtype);
  const bool in_place = x == y && nx == ny;
  if (!in_place && overlaps(x, nx, y, ny)) return fail(MMDIT_ERR_ALIAS, "cast: y overlaps x (only an exact in-place cast between 16-bit types is allowed)");
  return launch_cast(x, x_dtype, y, y_dtype, n, static_cast<hipStream_t>(stream));
}

int mmdit_quantize_fp8(const void* x, int x_dtype, int64_t rows, int64_t cols, int per_row, void* q,
                       float* scales, void* stream) {
  g_last_error.clear();
  if (rows < 0 || cols < 8 || cols % 8 || cols > ((int64_t)1 << 30))
    return fail(MMDIT_ERR_SHAPE, "quantize_fp8: cols must be a positive multiple of 8");
  if (!valid_dtype(x_dtype)) return fail(MMDIT_ERR_DTYPE, "quantize_fp8: x must be f32, bf16 or f16");
  if (!extents_ok({rows, cols})) return fail(MMDIT_ERR_SHAPE, "quantize_fp8: sizes too large");
  if (rows == 0) return MMDIT_OK;
  if (!x || !q || !scales) return fail(MMDIT_ERR_NULL, "quantize_fp8: x, q, scales required");
  if (!aligned16(x) || !aligned16(q) || (reinterpret_cast<uintptr_t>(scales) & 3))
    return fail(MMDIT_ERR_ALIGN, "quantize_fp8: x and q must be 16-byte aligned, scales 4-byte aligned");
  const size_t n = (size_t)(rows * cols), ns = (size_t)(per_row ? rows : 1) * 4;
  if (overlaps(q, n, x, n * dtype_size(x_dtype)) || overlaps(scales, ns, x, n * dtype_size(x_dtype)) ||
      overlaps(scales, ns, q, n))
    return fail(MMDIT_ERR_ALIAS, "quantize_fp8: outputs overlap x or each other");
  return launch_quantize_fp8(x, x_dtype, rows, cols, per_row ? 1 : 0, static_cast<uint8_t*>(q), scales,
                             static_cast<hipStream_t>(stream));
}

int mmdit_linear_fp8(const void* xq, const float* x_scale, const void* wq, const float* w_scale,
                     const void* bias, int bias_dtype, void* y, int y_dtype, int64_t M, int64_t N, int64_t K,
                     int epilogue, const void* res, int res_dtype, const float* gate, int64_t gate_stride,
                     int64_t rows_per_batch, void* stream) {
  g_last_error.clear();
  if (!extents_ok({M}) || !extents_ok({N}) || !extents_ok({K}) || K < 64 || K % 64 || N % 4)
    return fail(MMDIT_ERR_SHAPE, "linear_fp8: need M, N >= 0, N a multiple of 4 and K a positive multiple of 64");
  if (!extents_ok({M + 256, K}) || !extents_ok({N + 256, K}) || !extents_ok({M, N}) || !extents_ok({rows_per_batch}) ||
      !extents_ok({gate_stride}) || (M + 256) * K >= ((int64_t)1 << 31) || (N + 256) * K >= ((int64_t)1 << 31))
    return fail(MMDIT_ERR_SHAPE, "linear_fp8: x or w too large for 32-bit buffer offsets");
  if (bias && bias_dtype != MMDIT_F32 && bias_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, "linear_fp8: bias must be f32 or bf16");
  if (!valid_dtype(y_dtype)) return fail(MMDIT_ERR_DTYPE, "linear_fp8: bad y dtype");
  if (epilogue < MMDIT_EPI_NONE || epilogue > MMDIT_EPI_GATED_RES) return fail(MMDIT_ERR_SHAPE, "linear_fp8: bad epilogue");
  if (epilogue == MMDIT_EPI_GATED_RES) {
    if (res_dtype != MMDIT_F32 && res_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, "linear_fp8: res must be f32 or bf16");
    if (y_dtype == MMDIT_F16) return fail(MMDIT_ERR_DTYPE, "linear_fp8: gated residual output must be f32 or bf16");
    if (rows_per_batch < 1 || gate_stride < N || gate_stride % 4)
      return fail(MMDIT_ERR_SHAPE, "linear_fp8: rows_per_batch >= 1 and gate_stride >= N, a multiple of 4");
  }
  if (M == 0 || N == 0) return MMDIT_OK;
  if (!xq || !wq || !y || !x_scale || !w_scale) return fail(MMDIT_ERR_NULL, "linear_fp8: xq, x_scale, wq, w_scale, y required");
  if (epilogue == MMDIT_EPI_GATED_RES && (!res || !gate)) return fail(MMDIT_ERR_NULL, "linear_fp8: res and gate required");
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || (bias && !aligned16(bias)) || (res && !aligned16(res)) ||
      (gate && !aligned16(gate)) || (reinterpret_cast<uintptr_t>(x_scale) & 3) || (reinterpret_cast<uintptr_t>(w_scale) & 3))
    return fail(MMDIT_ERR_ALIGN, "linear_fp8: pointers must be 16-byte aligned (scales 4-byte)");
  const size_t ny = (size_t)(M * N) * dtype_size(y_dtype);
  if (overlaps(y, ny, xq, (size_t)(M * K)) || overlaps(y, ny, wq, (size_t)(N * K)) ||
      overlaps(y, ny, x_scale, (size_t)M * 4) || overlaps(y, ny, w_scale, 4) ||
      (res && res != y && overlaps(y, ny, res, (size_t)(M * N) * dtype_size(res_dtype))))
    return fail(MMDIT_ERR_ALIAS, "linear_fp8: y overlaps an input");
  GemmProblem p{};
  p.x = xq; p.w = wq; p.bias = bias; p.y = y; p.res = res; p.gate = gate; p.M = M;
  p.gate_stride = gate_stride; p.rows_per_batch = rows_per_batch > 0 ? rows_per_batch : M;
  p.x_scale = x_scale; p.w_scale = w_scale;
  return launch_linear(&p, 1, MMDIT_FP8_E4M3, bias_dtype, y_dtype, N, K, epilogue, res_dtype,
                       static_cast<hipStream_t>(stream));
}

int mmdit_modulation(const void* w_mod, const void* b_mod, const void* tvec, int t_dtype, float* mod,
                     int64_t B, int64_t C6, int64_t Dt, void* stream) {
  g_last_error.clear();
  if (B < 0 || C6 < 0 || Dt < 8 || Dt % 8) return fail(MMDIT_ERR_SHAPE, "modulation: Dt must be a positive multiple of 8");
  if (Dt > 16384) return fail(MMDIT_ERR_SHAPE, "modulation: Dt must be <= 16384");
  if (!extents_ok({B, C6}) || !extents_ok({C6, Dt})) return fail(MMDIT_ERR_SHAPE, "modulation: sizes too large");
  if (t_dtype != MMDIT_F32 && t_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, "modulation: tvec must be f32 or bf16");
  if (B == 0 || C6 == 0) return MMDIT_OK;
  if (!w_mod || !tvec || !mod) return fail(MMDIT_ERR_NULL, "modulation: w_mod, tvec, mod required");
  if (!aligned16(w_mod) || !aligned16(tvec) || !aligned16(mod)) return fail(MMDIT_ERR_ALIGN, "modulation: pointers must be 16-byte aligned");
  return launch_modulation(w_mod, b_mod, tvec, t_dtype, mod, B, C6, Dt, static_cast<hipStream_t>(stream));
}

static int lite_regroup(int layout, const char* name, const void* x, int x_dtype, const void* w,
                        const void* bias, int bias_dtype, void* y, int y_dtype, int64_t B, int64_t T,
                        int64_t H, int64_t W, int64_t C, void* stream) {
  g_last_error.clear();
  const std::string n(name);
  if (B < 0 || T < 0 || H < 2 || W < 2 || H % 2 || W % 2)
    return fail(MMDIT_ERR_SHAPE, n + ": the grid needs T >= 0 and an even H, W >= 2 (the merge is defined for even grids)");
  if (C < 256 || C % 256) return fail(MMDIT_ERR_SHAPE, n + ": C must be a positive multiple of 256");
  if (!extents_ok({B, T, H, W, C})) return fail(MMDIT_ERR_SHAPE, n + ": sizes too large");
  if (x_dtype != MMDIT_BF16 && x_dtype != MMDIT_F16) return fail(MMDIT_ERR_DTYPE, n + ": x and w must be bf16 or f16");
  if (bias && bias_dtype != MMDIT_F32 && bias_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, n + ": bias must be f32 or bf16");
  if (!valid_dtype(y_dtype)) return fail(MMDIT_ERR_DTYPE, n + ": bad y dtype");
  const int64_t M = B * T * (H / 2) * (W / 2);
  if ((M + 256) * 4 * C * 2 >= ((int64_t)1 << 31) || (4 * C + 256) * C * 2 >= ((int64_t)1 << 31))
    return fail(MMDIT_ERR_SHAPE, n + ": x or w too large for 32-bit buffer offsets");
  if (M == 0) return MMDIT_OK;
  if (!x || !w || !y) return fail(MMDIT_ERR_NULL, n + ": x, w, y required");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (bias && !aligned16(bias)))
    return fail(MMDIT_ERR_ALIGN, n + ": pointers must be 16-byte aligned");
  const size_t nx = (size_t)(4 * M * C) * 2, nw = (size_t)(4 * C * C) * 2;
  const size_t ny = (size_t)(4 * M * C / (layout == GEMM_GATHER_X ? 4 : 1)) * dtype_size(y_dtype);
  if (overlaps(y, ny, x, layout == GEMM_GATHER_X ? nx : nx / 4) || overlaps(y, ny, w, nw) ||
      (bias && overlaps(y, ny, bias, (size_t)(layout == GEMM_GATHER_X ? C : 4 * C) * dtype_size(bias_dtype))))
    return fail(MMDIT_ERR_ALIAS, n + ": y overlaps an input");
  return launch_lite_regroup(layout, x, w, bias, bias_dtype, y, x_dtype, y_dtype, B, T, H, W, C,
                             static_cast<hipStream_t>(stream));
}

int mmdit_lite_merge(const void* x, int x_dtype, const void* w, const void* bias, int bias_dtype, void* y,
                     int y_dtype, int64_t B, int64_t T, int64_t H, int64_t W, int64_t C, void* stream) {
  return lite_regroup(GEMM_GATHER_X, "lite_merge", x, x_dtype, w, bias, bias_dtype, y, y_dtype, B, T, H, W, C, stream);
}

int mmdit_lite_unpatchify(const void* x, int x_dtype, const void* w, const void* bias, int bias_dtype, void* y,
                          int y_dtype, int64_t B, int64_t T, int64_t H, int64_t W, int64_t C, void* stream) {
  return lite_regroup(GEMM_SCATTER_Y, "lite_unpatchify", x, x_dtype, w, bias, bias_dtype, y, y_dtype, B, T, H, W,
                      C, stream);
}

int mmdit_timestep_embed(const float* t, int64_t B, const void* w1, const void* b1, const void* w2,
                         const void* b2, const void* w3, const void* b3, int w_dtype, int64_t freq_dim,
                         int64_t hidden_dim, int64_t Dt, float max_period, float* hidden, float* temb,
                         float* tvec, void* stream) {
  g_last_error.clear();
  if (B < 0 || freq_dim < 16 || freq_dim % 16 || hidden_dim < 8 || hidden_dim % 8 || Dt < 1)
    return fail(MMDIT_ERR_SHAPE, "timestep_embed: freq_dim a positive multiple of 16, hidden_dim of 8, Dt >= 1");
  if (freq_dim > 16384 || hidden_dim > 16384) return fail(MMDIT_ERR_SHAPE, "timestep_embed: freq_dim and hidden_dim must be <= 16384");
  if (!extents_ok({B, hidden_dim}) || !extents_ok({B, Dt}) || !extents_ok({Dt, hidden_dim}))
    return fail(MMDIT_ERR_SHAPE, "timestep_embed: sizes too large");
  if (!(max_period > 1.f) || !(max_period < 3.0e38f)) return fail(MMDIT_ERR_SHAPE, "timestep_embed: max_period must be a finite value > 1");
  if (w_dtype != MMDIT_F32 && w_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, "timestep_embed: weights must be f32 or bf16");
  if (B == 0) return MMDIT_OK;
  if (!t || !w1 || !w2 || !w3 || !hidden || !temb || !tvec) return fail(MMDIT_ERR_NULL, "timestep_embed: t, w1, w2, w3, hidden, temb, tvec required");
  const void* ps[] = {t, w1, w2, w3, b1, b2, b3, hidden, temb, tvec};
  for (const void* p : ps)
    if (p && !aligned16(p)) return fail(MMDIT_ERR_ALIGN, "timestep_embed: pointers must be 16-byte aligned");
  const size_t ws = dtype_size(w_dtype);
  const size_t nh = (size_t)(B * hidden_dim) * 4, nt = (size_t)(B * Dt) * 4;
  const void* outs[] = {hidden, temb, tvec};
  const size_t nout[] = {nh, nh, nt};
  const void* ins[] = {t, w1, w2, w3, b1, b2, b3};
  const size_t nin[] = {(size_t)B * 4, (size_t)(hidden_dim * freq_dim) * ws, (size_t)(hidden_dim * hidden_dim) * ws,
                        (size_t)(Dt * hidden_dim) * ws, (size_t)hidden_dim * ws, (size_t)hidden_dim * ws, (size_t)Dt * ws};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 7; ++i)
      if (ins[i] && overlaps(outs[o], nout[o], ins[i], nin[i])) return fail(MMDIT_ERR_ALIAS, "timestep_embed: an output overlaps an input");
    for (int p = o + 1; p < 3; ++p)
      if (overlaps(outs[o], nout[o], outs[p], nout[p])) return fail(MMDIT_ERR_ALIAS, "timestep_embed: outputs overlap");
  }
  return launch_timestep_embed(t, B, w1, b1, w2, b2, w3, b3, w_dtype, freq_dim, hidden_dim, Dt, max_period,
                               hidden, temb, tvec, static_cast<hipStream_t>(stream));
}

}  // extern "C"
