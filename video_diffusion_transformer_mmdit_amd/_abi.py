"""ctypes binding of libmmdit.so: argument marshalling only.

Torch supplies device memory and the current HIP stream; every function below checks
shapes, takes ``data_ptr()`` and strides, and calls the C entry point of the same name
declared in include/mmdit.h.  A non-zero status raises MmditError with the library's text.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import c_float, c_int, c_int32, c_int64, c_size_t, c_void_p
from typing import Dict, Optional, Sequence, Tuple

import torch

F32, BF16, F16, FP8_E4M3 = 0, 1, 2, 3
EPI_NONE, EPI_GELU, EPI_GATED_RES = 0, 1, 2
(WS_MOD, WS_H, WS_QKV, WS_X1, WS_G, WS_WQKV, WS_WO, WS_W1, WS_W2, WS_SPLIT,
 WS_XQ, WS_XS, WS_Q8, WS_QS, WS_K8, WS_KS, WS_V8T, WS_VS) = range(18)
WS_COUNT = 18
STAGES = ("mod_ln1", "qkv", "qk_norm_rope", "attention", "out_proj", "ln2", "ffn_up", "ffn_down")
STAGE_COUNT = len(STAGES)

_TORCH_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
_DT_TORCH = {v: k for k, v in _TORCH_DT.items()}


class MmditError(RuntimeError):
    pass


class Rope3D(ctypes.Structure):
    """3D RoPE of the visual grid: T x H x W tokens, head dims split d_t/d_h/d_w."""
    _fields_ = [("T", c_int64), ("H", c_int64), ("W", c_int64),
                ("d_t", c_int32), ("d_h", c_int32), ("d_w", c_int32), ("base", c_float)]

    @classmethod
    def make(cls, grid: Sequence[int], split: Sequence[int] = (16, 56, 56), base: float = 10000.0):
        return cls(int(grid[0]), int(grid[1]), int(grid[2]), int(split[0]), int(split[1]),
                   int(split[2]), float(base))


class Attn8Stream(ctypes.Structure):
    """Quantized operands of one stream for the 8-bit joint attention (device pointers)."""
    _fields_ = [("q8", c_void_p), ("q_scale", c_void_p), ("k8", c_void_p), ("k_scale", c_void_p),
                ("v8t", c_void_p)]


class StreamWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("w_mod", "b_mod", "w_qkv", "b_qkv", "q_norm", "k_norm",
                                         "w_o", "b_o", "w_fc1", "b_fc1", "w_fc2", "b_fc2",
                                         "s_qkv", "s_o", "s_fc1", "s_fc2")]


class BlockDims(ctypes.Structure):
    _fields_ = [("C", c_int64), ("H", c_int64), ("D", c_int64), ("F", c_int64), ("Dt", c_int64),
                ("ln_eps", c_float), ("qk_eps", c_float), ("qk_scale_head_stride", c_int64),
                ("w_dtype", c_int), ("act_dtype", c_int)]

    @classmethod
    def make(cls, C, H, F, Dt, ln_eps=1e-6, qk_eps=1e-6, qk_scale_head_stride=0,
             act_dtype=torch.float16, matrix_dtype=torch.bfloat16):
        """matrix_dtype: dtype of the four GEMM weight matrices (w_qkv, w_o, w_fc1, w_fc2);
        float16 (with act_dtype float16) means they were converted once by the caller;
        torch.float8_e4m3fn (with act_dtype float16) selects the 8-bit block, its matrices
        given as E4M3 codes (uint8) with their scales (see fp8_block_weights)."""
        mdt = FP8_E4M3 if matrix_dtype == torch.float8_e4m3fn else _TORCH_DT[matrix_dtype]
        return cls(C, H, C // H, F, Dt, ln_eps, qk_eps, qk_scale_head_stride, mdt, _TORCH_DT[act_dtype])


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmmdit.so")


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libmmdit.so once.  Raises if it has not been built: there is no fallback."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise MmditError(f"{path} is missing; build it with "
                         "`python -m video_diffusion_transformer_mmdit_amd.build`")
    L = ctypes.CDLL(path)
    i64, vp, f, i = c_int64, c_void_p, c_float, c_int
    sig = {
        "mmdit_modulate_ln": [vp, i, vp, i, vp, vp, vp, vp, i64, vp, i, i64, i64, i64, f, vp],
        "mmdit_qk_norm_rope": [vp, vp, i, i64, vp, vp, i, i64, vp, vp, i, i64, i64, i64, i64, i64, f,
                               ctypes.POINTER(Rope3D), vp],
        "mmdit_joint_attention": [vp, vp, vp, i64, vp, vp, vp, i64, i, i, i64, i64, i64, i64, f, vp, vp, i,
                                  i64, vp, vp, ctypes.c_size_t, vp],
        "mmdit_joint_attention_noalloc": [vp, vp, vp, i64, vp, vp, vp, i64, i, i, i64, i64, i64, i64, f, vp, vp, i,
                                          i64, vp, vp],
        "mmdit_linear": [vp, vp, i, vp, i, vp, i, i64, i64, i64, i, vp, i, vp, i64, i64, vp],
        "mmdit_cast": [vp, i, vp, i, i64, vp],
        "mmdit_modulation": [vp, vp, vp, i, vp, i64, i64, i64, vp],
        "mmdit_lite_merge": [vp, i, vp, vp, i, vp, i, i64, i64, i64, i64, i64, vp],
        "mmdit_lite_unpatchify": [vp, i, vp, vp, i, vp, i, i64, i64, i64, i64, i64, vp],
        "mmdit_quantize_fp8": [vp, i, i64, i64, i, vp, vp, vp],
        "mmdit_attn8_quantize": [vp, vp, vp, i64, vp, vp, vp, i64, i, i64, i64, i64, i64,
                                 ctypes.POINTER(Attn8Stream), ctypes.POINTER(Attn8Stream), vp, vp],
        "mmdit_joint_attention_8bit": [ctypes.POINTER(Attn8Stream), i64, ctypes.POINTER(Attn8Stream), i64, vp,
                                       i64, i64, i64, f, vp, vp, i, i64, vp, vp, ctypes.c_size_t, vp],
        "mmdit_linear_fp8": [vp, vp, vp, vp, vp, i, vp, i, i64, i64, i64, i, vp, i, vp, i64, i64, vp],
        "mmdit_timestep_embed": [vp, i64, vp, vp, vp, vp, vp, vp, i, i64, i64, i64, f, vp, vp, vp, vp],
        "mmdit_block_workspace_offsets": [ctypes.POINTER(BlockDims), i64, i64, i64, ctypes.POINTER(c_size_t)],
        "mmdit_block_fwd": [ctypes.POINTER(BlockDims), ctypes.POINTER(StreamWeights),
                            ctypes.POINTER(StreamWeights), vp, vp, i, vp, i, ctypes.POINTER(Rope3D), i64,
                            vp, vp, i, vp, c_size_t, i64, vp],
        "mmdit_block_fwd_events": [ctypes.POINTER(BlockDims), ctypes.POINTER(StreamWeights),
                                   ctypes.POINTER(StreamWeights), vp, vp, i, vp, i, ctypes.POINTER(Rope3D),
                                   i64, vp, vp, i, vp, c_size_t, i64, vp, ctypes.POINTER(c_void_p)],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = c_int
    L.mmdit_block_workspace_bytes.argtypes = [ctypes.POINTER(BlockDims), i64, i64, i64]
    L.mmdit_block_workspace_bytes.restype = c_size_t
    L.mmdit_status_str.argtypes = [c_int]
    L.mmdit_status_str.restype = ctypes.c_char_p
    L.mmdit_last_error.argtypes = []
    L.mmdit_last_error.restype = ctypes.c_char_p
    L.mmdit_abi_version.argtypes = []
    L.mmdit_abi_version.restype = c_int
    _LIB = L
    return L


def abi_version() -> int:
    return lib().mmdit_abi_version()


def _check(status: int, name: str):
    if status != 0:
        msg = lib().mmdit_last_error().decode()
        raise MmditError(f"{name} failed ({lib().mmdit_status_str(status).decode()}): {msg}")


def _dt(t: torch.Tensor) -> int:
    try:
        return _TORCH_DT[t.dtype]
    except KeyError:
        raise MmditError(f"unsupported dtype {t.dtype}") from None


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise MmditError("tensors must live on the GPU")


def _on_device(device: torch.device, **named):
    """Every given tensor must be a GPU tensor on ``device`` (the device the kernels run on):
    a host or other-device pointer handed to a kernel would be written through."""
    for name, t in named.items():
        if t is None:
            continue
        if not t.is_cuda or device.type != "cuda" or t.device != device:
            raise MmditError(f"{name} must be a GPU tensor on {device} (got {t.device})")


def _workspace_bytes(workspace: Optional[torch.Tensor]) -> int:
    if workspace is None:
        return 0
    if not workspace.is_contiguous():
        raise MmditError("workspace must be contiguous")
    return workspace.numel() * workspace.element_size()


def _rows(t: torch.Tensor, name: str) -> Tuple[int, int, int]:
    """[B, N, H, D] view with contiguous (H, D) and batch items N rows apart ->
    (B, N, row_stride)."""
    if t.dim() != 4:
        raise MmditError(f"{name} must be [B, N, H, D]")
    B, N, H, D = t.shape
    if t.stride(3) != 1 or (H > 1 and t.stride(2) != D):
        raise MmditError(f"{name}: heads and dims must be contiguous")
    rs = t.stride(1)
    if B > 1 and N > 0 and t.stride(0) != N * rs:
        raise MmditError(f"{name}: batch items must be N rows apart")
    return B, N, rs


# --------------------------------------------------------------------------- calls
def modulate_ln(x: torch.Tensor, shift: torch.Tensor, scale: torch.Tensor, *,
                branch: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None,
                x_out: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                y_dtype=torch.bfloat16, eps: float = 1e-6) -> torch.Tensor:
    """y = LN(x + gate*branch) * (1 + scale) + shift.  x [B, N, C]; shift/scale/gate f32
    [B, C] (rows may be strided, e.g. slices of a [B, 6C] modulation buffer)."""
    _need_gpu(x, shift, scale, branch, gate, x_out, y)
    B, N, C = x.shape
    if not x.is_contiguous():
        raise MmditError("x must be contiguous")
    mods = [m for m in (shift, scale, gate) if m is not None]
    for m in mods:
        if m.dtype != torch.float32 or m.dim() != 2 or m.stride(1) != 1 or m.shape != (B, C):
            raise MmditError("shift / scale / gate must be f32 [B, C] with unit inner stride")
    strides = {m.stride(0) for m in mods} if B > 1 else {max(m.stride(0) for m in mods) if B else C}
    if len(strides) != 1:
        raise MmditError("shift / scale / gate must share one batch stride")
    ms = max(strides.pop(), C)
    if y is None:
        y = torch.empty((B, N, C), dtype=y_dtype, device=x.device)
    st = lib().mmdit_modulate_ln(x.data_ptr(), _dt(x), _ptr(branch), _dt(branch) if branch is not None else BF16,
                                 _ptr(gate), _ptr(x_out), shift.data_ptr(), scale.data_ptr(), ms,
                                 y.data_ptr(), _dt(y), B, N, C, eps, _stream(x))
    _check(st, "mmdit_modulate_ln")
    return y


def qk_norm_rope(q: torch.Tensor, k: torch.Tensor, q_scale: torch.Tensor, k_scale: torch.Tensor, *,
                 rope: Optional[Rope3D] = None, eps: float = 1e-6,
                 q_out: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None,
                 out_dtype=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-head RMSNorm of q and k (+ 3D RoPE when ``rope`` is given).  q, k: [B, N, H, D]
    views sharing one row stride; pass q_out=q, k_out=k for in place."""
    _need_gpu(q, k, q_scale, k_scale, q_out, k_out)
    B, N, rs = _rows(q, "q")
    _, _, rsk = _rows(k, "k")
    if k.shape != q.shape or rsk != rs or k.dtype != q.dtype:
        raise MmditError("q and k must share shape, dtype and row stride")
    H, D = q.shape[2], q.shape[3]
    od = out_dtype or q.dtype
    if q_out is None:
        q_out = torch.empty(q.shape, dtype=od, device=q.device)
    if k_out is None:
        k_out = torch.empty(q.shape, dtype=od, device=q.device)
    _, _, ors = _rows(q_out, "q_out")
    _, _, orsk = _rows(k_out, "k_out")
    if orsk != ors or k_out.dtype != q_out.dtype:
        raise MmditError("q_out and k_out must share dtype and row stride")
    if q_scale.dtype != k_scale.dtype or q_scale.shape != k_scale.shape:
        raise MmditError("q_scale and k_scale must match")
    shs = 0 if q_scale.dim() == 1 else D
    st = lib().mmdit_qk_norm_rope(q.data_ptr(), k.data_ptr(), _dt(q), rs, q_scale.data_ptr(),
                                  k_scale.data_ptr(), _dt(q_scale), shs, q_out.data_ptr(),
                                  k_out.data_ptr(), _dt(q_out), ors, B, N, H, D, eps,
                                  ctypes.byref(rope) if rope is not None else None, _stream(q))
    _check(st, "mmdit_qk_norm_rope")
    return q_out, k_out


# bytes of key-range results the attention kernels' split tails can use: 256 slots of
# 256 x 128 outputs plus (m, l) for 256 queries, f32
ATTN_SPLIT_BYTES = 256 * (256 * 128 + 256 * 2) * 4
ATTN8_SPLIT_BYTES = ATTN_SPLIT_BYTES


def joint_attention(q_vis, k_vis, v_vis, q_cond=None, k_cond=None, v_cond=None, *,
                    softmax_scale: Optional[float] = None, out_dtype=torch.float32,
                    o_vis: Optional[torch.Tensor] = None, o_cond: Optional[torch.Tensor] = None,
                    return_lse: bool = False, workspace: Optional[torch.Tensor] = None):
    """softmax(Q K^T * scale) V over [cond | vis] per head, outputs split per stream.
    Inputs [B, N_s, H, D] views with one common row stride.  ``workspace`` (optional device
    bytes, 256-byte aligned; ATTN_SPLIT_BYTES is always enough) lets a partly empty last
    round of workgroups split its items over key ranges."""
    ts = [t for t in (q_vis, k_vis, v_vis, q_cond, k_cond, v_cond) if t is not None]
    _need_gpu(*ts)
    _on_device(q_vis.device, k_vis=k_vis, v_vis=v_vis, q_cond=q_cond, k_cond=k_cond, v_cond=v_cond,
               o_vis=o_vis, o_cond=o_cond, workspace=workspace)
    ws_bytes = _workspace_bytes(workspace)
    B, n_vis, rs = _rows(q_vis, "q_vis")
    H, D = q_vis.shape[2], q_vis.shape[3]
    n_cond = 0 if q_cond is None else q_cond.shape[1]
    for nm, t in zip(("k_vis", "v_vis", "q_cond", "k_cond", "v_cond"), (k_vis, v_vis, q_cond, k_cond, v_cond)):
        if t is None:
            continue
        b, n, r = _rows(t, nm)
        ref_dt = v_vis.dtype if nm.startswith("v") else q_vis.dtype
        if t.dtype != ref_dt or t.shape[0] != B or t.shape[2:] != q_vis.shape[2:]:
            raise MmditError(f"{nm}: dtype / shape mismatch")
        if n > 0 and r != rs and not (n == 1 or rs == 0):
            raise MmditError(f"{nm}: all inputs must share one row stride")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    dev = q_vis.device
    if o_vis is None:
        o_vis = torch.empty((B, n_vis, H, D), dtype=out_dtype, device=dev)
    if o_cond is None and n_cond > 0:
        o_cond = torch.empty((B, n_cond, H, D), dtype=out_dtype, device=dev)
    _, _, ors = _rows(o_vis, "o_vis")
    lse = torch.empty((B, H, n_vis + n_cond), dtype=torch.float32, device=dev) if return_lse else None
    st = lib().mmdit_joint_attention(q_vis.data_ptr(), k_vis.data_ptr(), v_vis.data_ptr(), n_vis,
                                     _ptr(q_cond) if n_cond else None, _ptr(k_cond) if n_cond else None,
                                     _ptr(v_cond) if n_cond else None, n_cond, _dt(q_vis), _dt(v_vis), rs, B, H, D,
                                     softmax_scale, o_vis.data_ptr(), _ptr(o_cond) if n_cond else None,
                                     _dt(o_vis), ors, _ptr(lse), _ptr(workspace), ws_bytes, _stream(q_vis))
    _check(st, "mmdit_joint_attention")
    if return_lse:
        return o_vis, o_cond, lse
    return o_vis, o_cond


def joint_attention_noalloc(q_vis, k_vis, v_vis, q_cond=None, k_cond=None, v_cond=None, *,
                            softmax_scale: Optional[float] = None, o_vis: torch.Tensor, o_cond: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None):
    """mmdit_joint_attention_noalloc: joint_attention whose split tail uses the library's static
    scratch (no allocation anywhere: the caller passes every output, ``o_vis`` / ``o_cond`` and
    optionally ``lse`` [B, H, n_cond + n_vis] f32).  Calls on one GPU must not overlap in time."""
    ts = [t for t in (q_vis, k_vis, v_vis, q_cond, k_cond, v_cond) if t is not None]
    _need_gpu(*ts)
    _on_device(q_vis.device, k_vis=k_vis, v_vis=v_vis, q_cond=q_cond, k_cond=k_cond, v_cond=v_cond,
               o_vis=o_vis, o_cond=o_cond, lse=lse)
    B, n_vis, rs = _rows(q_vis, "q_vis")
    H, D = q_vis.shape[2], q_vis.shape[3]
    n_cond = 0 if q_cond is None else q_cond.shape[1]
    for nm, t in zip(("k_vis", "v_vis", "q_cond", "k_cond", "v_cond"), (k_vis, v_vis, q_cond, k_cond, v_cond)):
        if t is None:
            continue
        _, n, r = _rows(t, nm)
        ref_dt = v_vis.dtype if nm.startswith("v") else q_vis.dtype
        if t.dtype != ref_dt or t.shape[0] != B or t.shape[2:] != q_vis.shape[2:]:
            raise MmditError(f"{nm}: dtype / shape mismatch")
        if n > 0 and r != rs and not (n == 1 or rs == 0):
            raise MmditError(f"{nm}: all inputs must share one row stride")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(D)
    _, _, ors = _rows(o_vis, "o_vis")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (B, H, n_vis + n_cond)):
        raise MmditError("lse must be a contiguous f32 [B, H, n_cond + n_vis] tensor")
    st = lib().mmdit_joint_attention_noalloc(q_vis.data_ptr(), k_vis.data_ptr(), v_vis.data_ptr(), n_vis,
                                             _ptr(q_cond) if n_cond else None, _ptr(k_cond) if n_cond else None,
                                             _ptr(v_cond) if n_cond else None, n_cond, _dt(q_vis), _dt(v_vis), rs,
                                             B, H, D, softmax_scale, o_vis.data_ptr(),
                                             _ptr(o_cond) if n_cond else None, _dt(o_vis), ors, _ptr(lse),
                                             _stream(q_vis))
    _check(st, "mmdit_joint_attention_noalloc")
    return o_vis, o_cond


NOALLOC_SCRATCH_BYTES = 34078720


def cast(x: torch.Tensor, dtype: torch.dtype, *, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mmdit_cast: a contiguous copy of ``x`` in ``dtype`` (f32, bf16 or f16; rounding to
    nearest even), into ``out`` if given (``out`` may be ``x`` for a 16-bit to 16-bit cast)."""
    _need_gpu(x)
    if not x.is_contiguous():
        raise MmditError("cast: x must be contiguous")
    if out is None:
        out = torch.empty(x.shape, dtype=dtype, device=x.device)
    _on_device(x.device, out=out)
    if out.dtype != dtype or not out.is_contiguous() or out.numel() != x.numel():
        raise MmditError("cast: out must be a contiguous tensor of dtype with x's element count")
    _check(lib().mmdit_cast(x.data_ptr(), _dt(x), out.data_ptr(), _dt(out), x.numel(), _stream(x)), "mmdit_cast")
    return out


def linear(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor] = None, *,
           epilogue: int = EPI_NONE, res: Optional[torch.Tensor] = None,
           gate: Optional[torch.Tensor] = None, rows_per_batch: Optional[int] = None,
           y: Optional[torch.Tensor] = None, y_dtype=torch.bfloat16) -> torch.Tensor:
    """y = epilogue(x W^T + bias).  x [M, K], w [N, K] (bf16 or f16, contiguous)."""
    _need_gpu(x, w, bias, res, gate, y)
    M, K = x.shape
    N = w.shape[0]
    if not (x.is_contiguous() and w.is_contiguous()) or w.shape[1] != K:
        raise MmditError("x [M, K] and w [N, K] must be contiguous")
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=x.device)
    gs = 0
    if gate is not None:
        if gate.dtype != torch.float32 or gate.stride(-1) != 1:
            raise MmditError("gate must be f32 with unit inner stride")
        gs = gate.stride(0) if gate.dim() == 2 else N
    st = lib().mmdit_linear(x.data_ptr(), w.data_ptr(), _dt(x), _ptr(bias),
                            _dt(bias) if bias is not None else BF16, y.data_ptr(), _dt(y), M, N, K,
                            epilogue, _ptr(res), _dt(res) if res is not None else F32, _ptr(gate), gs,
                            rows_per_batch or M, _stream(x))
    _check(st, "mmdit_linear")
    return y


class Attn8Operands:
    """Tensors of the 8-bit attention operands (mmdit_attn8_stream per stream + V scales)."""

    def __init__(self, B: int, H: int, n_vis: int, n_cond: int, device):
        self.B, self.H, self.n = B, H, (n_vis, n_cond)
        self.t = []
        for n in (n_vis, n_cond):
            nb = (n + 63) // 64
            self.t.append({
                "q8": torch.empty((B, n, H, 128), dtype=torch.int8, device=device),
                "q_scale": torch.empty((B, H, n), dtype=torch.float32, device=device),
                "k8": torch.empty((B, n, H, 128), dtype=torch.int8, device=device),
                "k_scale": torch.empty((B, H, nb), dtype=torch.float32, device=device),
                "v8t": torch.empty((B, H, 128, nb * 64), dtype=torch.uint8, device=device)})
        self.v_scale = torch.empty((B, H, 128), dtype=torch.float32, device=device)

    def struct(self, s: int) -> Attn8Stream:
        t = self.t[s]
        return Attn8Stream(*(t[k].data_ptr() if t[k].numel() else None for k in ("q8", "q_scale", "k8", "k_scale", "v8t")))


def attn8_quantize(q_vis, k_vis, v_vis, q_cond=None, k_cond=None, v_cond=None,
                   out: Optional[Attn8Operands] = None) -> Attn8Operands:
    """INT8 Q/K and channel-major E4M3 V operands of the 8-bit joint attention from
    [B, n, H, 128] views sharing one row stride (as joint_attention takes them)."""
    ts = [t for t in (q_vis, k_vis, v_vis, q_cond, k_cond, v_cond) if t is not None]
    _need_gpu(*ts)
    B, n_vis, rs = _rows(q_vis, "q_vis")
    H, D = q_vis.shape[2], q_vis.shape[3]
    n_cond = 0 if q_cond is None else q_cond.shape[1]
    for nm, t in zip(("k_vis", "v_vis", "q_cond", "k_cond", "v_cond"), (k_vis, v_vis, q_cond, k_cond, v_cond)):
        if t is None:
            continue
        _, n, r = _rows(t, nm)
        if t.dtype != q_vis.dtype or t.shape[0] != B or t.shape[2:] != q_vis.shape[2:]:
            raise MmditError(f"{nm}: dtype / shape mismatch")
        if n > 0 and r != rs and n != 1:
            raise MmditError(f"{nm}: all inputs must share one row stride")
    if out is None:
        out = Attn8Operands(B, H, n_vis, n_cond, q_vis.device)
    sv, sc = out.struct(0), out.struct(1)
    st = lib().mmdit_attn8_quantize(q_vis.data_ptr(), k_vis.data_ptr(), v_vis.data_ptr(), n_vis,
                                    _ptr(q_cond) if n_cond else None, _ptr(k_cond) if n_cond else None,
                                    _ptr(v_cond) if n_cond else None, n_cond, _dt(q_vis), rs, B, H, D,
                                    ctypes.byref(sv), ctypes.byref(sc), out.v_scale.data_ptr(), _stream(q_vis))
    _check(st, "mmdit_attn8_quantize")
    return out





def joint_attention_8bit(ops: Attn8Operands, *, softmax_scale: Optional[float] = None, out_dtype=torch.float32,
                         o_vis: Optional[torch.Tensor] = None, o_cond: Optional[torch.Tensor] = None,
                         return_lse: bool = False, workspace: Optional[torch.Tensor] = None):
    """8-bit joint attention over the operands of attn8_quantize; outputs [B, n_s, H, 128].
    ``workspace`` (optional device bytes, 256-byte aligned) lets a partly empty last round of
    workgroups split its items over key ranges (ATTN8_SPLIT_BYTES is always enough)."""
    B, H = ops.B, ops.H
    n_vis, n_cond = ops.n
    dev = ops.v_scale.device
    _on_device(dev, v_scale=ops.v_scale, o_vis=o_vis, o_cond=o_cond, workspace=workspace)
    ws_bytes = _workspace_bytes(workspace)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(128)
    if o_vis is None:
        o_vis = torch.empty((B, n_vis, H, 128), dtype=out_dtype, device=dev)
    if o_cond is None and n_cond > 0:
        o_cond = torch.empty((B, n_cond, H, 128), dtype=out_dtype, device=dev)
    _, _, ors = _rows(o_vis, "o_vis")
    lse = torch.empty((B, H, n_vis + n_cond), dtype=torch.float32, device=dev) if return_lse else None
    sv, sc = ops.struct(0), ops.struct(1)
    st = lib().mmdit_joint_attention_8bit(ctypes.byref(sv), n_vis, ctypes.byref(sc), n_cond, ops.v_scale.data_ptr(),
                                          B, H, 128, softmax_scale, o_vis.data_ptr(),
                                          _ptr(o_cond) if n_cond else None, _dt(o_vis), ors, _ptr(lse),
                                          _ptr(workspace), ws_bytes, torch.cuda.current_stream(dev).cuda_stream)
    _check(st, "mmdit_joint_attention_8bit")
    if return_lse:
        return o_vis, o_cond, lse
    return o_vis, o_cond


def quantize_fp8(x: torch.Tensor, per_row: bool = True, q: Optional[torch.Tensor] = None,
                 scales: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """FP8 E4M3 codes (torch.uint8, same shape as x) and f32 scales ([rows] per row, [1] per
    tensor) of a contiguous 2-D x."""
    _need_gpu(x, q, scales)
    if x.dim() != 2 or not x.is_contiguous():
        raise MmditError("x must be a contiguous [rows, cols] tensor")
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if q is None else q
    scales = torch.empty((rows if per_row else 1,), dtype=torch.float32, device=x.device) if scales is None else scales
    if q.dtype != torch.uint8 or q.shape != (rows, cols) or scales.dtype != torch.float32:
        raise MmditError("q must be uint8 [rows, cols] and scales f32")
    st = lib().mmdit_quantize_fp8(x.data_ptr(), _dt(x), rows, cols, 1 if per_row else 0, q.data_ptr(),
                                  scales.data_ptr(), _stream(x))
    _check(st, "mmdit_quantize_fp8")
    return q, scales


def linear_fp8(xq: torch.Tensor, x_scale: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
               bias: Optional[torch.Tensor] = None, *, epilogue: int = EPI_NONE,
               res: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None,
               rows_per_batch: Optional[int] = None, y: Optional[torch.Tensor] = None,
               y_dtype=torch.bfloat16) -> torch.Tensor:
    """y = epilogue((xq wq^T) x_scale[m] w_scale + bias) on E4M3 codes (uint8 tensors)."""
    _need_gpu(xq, x_scale, wq, w_scale, bias, res, gate, y)
    M, K = xq.shape
    N = wq.shape[0]
    if xq.dtype != torch.uint8 or wq.dtype != torch.uint8 or wq.shape[1] != K:
        raise MmditError("xq [M, K] and wq [N, K] must be uint8 E4M3 codes")
    if not (xq.is_contiguous() and wq.is_contiguous()):
        raise MmditError("xq and wq must be contiguous")
    if y is None:
        y = torch.empty((M, N), dtype=y_dtype, device=xq.device)
    gs = 0
    if gate is not None:
        if gate.dtype != torch.float32 or gate.stride(-1) != 1:
            raise MmditError("gate must be f32 with unit inner stride")
        gs = gate.stride(0) if gate.dim() == 2 else N
    st = lib().mmdit_linear_fp8(xq.data_ptr(), x_scale.data_ptr(), wq.data_ptr(), w_scale.data_ptr(), _ptr(bias),
                                _dt(bias) if bias is not None else BF16, y.data_ptr(), _dt(y), M, N, K, epilogue,
                                _ptr(res), _dt(res) if res is not None else F32, _ptr(gate), gs,
                                rows_per_batch or M, _stream(xq))
    _check(st, "mmdit_linear_fp8")
    return y


def modulation(w_mod: torch.Tensor, b_mod: Optional[torch.Tensor], tvec: torch.Tensor,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mod [B, 6C] f32 = W_mod tvec + b_mod."""
    _need_gpu(w_mod, b_mod, tvec, out)
    C6, Dt = w_mod.shape
    B = tvec.shape[0]
    if out is None:
        out = torch.empty((B, C6), dtype=torch.float32, device=w_mod.device)
    st = lib().mmdit_modulation(w_mod.data_ptr(), _ptr(b_mod), tvec.data_ptr(), _dt(tvec), out.data_ptr(),
                                B, C6, Dt, _stream(w_mod))
    _check(st, "mmdit_modulation")
    return out


def timestep_embed(t: torch.Tensor, w1: torch.Tensor, b1: Optional[torch.Tensor], w2: torch.Tensor,
                   b2: Optional[torch.Tensor], w3: torch.Tensor, b3: Optional[torch.Tensor], *,
                   max_period: float = 10000.0, hidden: Optional[torch.Tensor] = None,
                   temb: Optional[torch.Tensor] = None, tvec: Optional[torch.Tensor] = None):
    """Timestep path: sinusoid(t) -> W1 -> SiLU -> W2 (= temb) -> SiLU -> W3 (= tvec).
    t [B] f32; w1 [Dh, freq_dim], w2 [Dh, Dh], w3 [Dt, Dh] (f32 or bf16, contiguous).
    Returns (hidden, temb, tvec), f32."""
    _need_gpu(t, w1, b1, w2, b2, w3, b3, hidden, temb, tvec)
    if t.dtype != torch.float32 or t.dim() != 1 or not t.is_contiguous():
        raise MmditError("t must be a contiguous f32 [B] tensor")
    dh, fd = w1.shape
    dt = w3.shape[0]
    if w2.shape != (dh, dh) or w3.shape[1] != dh:
        raise MmditError("w1 [Dh, freq_dim], w2 [Dh, Dh], w3 [Dt, Dh] expected")
    for nm, w in (("w1", w1), ("w2", w2), ("w3", w3), ("b1", b1), ("b2", b2), ("b3", b3)):
        if w is not None and (w.dtype != w1.dtype or not w.is_contiguous()):
            raise MmditError(f"{nm} must be contiguous and of w1's dtype")
    B = t.shape[0]
    dev = t.device
    hidden = torch.empty((B, dh), dtype=torch.float32, device=dev) if hidden is None else hidden
    temb = torch.empty((B, dh), dtype=torch.float32, device=dev) if temb is None else temb
    tvec = torch.empty((B, dt), dtype=torch.float32, device=dev) if tvec is None else tvec
    for nm, o, n in (("hidden", hidden, dh), ("temb", temb, dh), ("tvec", tvec, dt)):
        if o.dtype != torch.float32 or o.shape != (B, n) or not o.is_contiguous():
            raise MmditError(f"{nm} must be a contiguous f32 [B, {n}] tensor")
    st = lib().mmdit_timestep_embed(t.data_ptr(), B, w1.data_ptr(), _ptr(b1), w2.data_ptr(), _ptr(b2),
                                    w3.data_ptr(), _ptr(b3), _dt(w1), fd, dh, dt, max_period,
                                    hidden.data_ptr(), temb.data_ptr(), tvec.data_ptr(), _stream(t))
    _check(st, "mmdit_timestep_embed")
    return hidden, temb, tvec


def _lite(name: str, x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], grid: Sequence[int],
          y: Optional[torch.Tensor], y_dtype, merge: bool) -> torch.Tensor:
    _need_gpu(x, w, bias, y)
    T, H, W = (int(g) for g in grid)
    if x.dim() != 3 or not x.is_contiguous() or not w.is_contiguous() or w.dtype != x.dtype:
        raise MmditError(f"{name}: x [B, n, C] and w must be contiguous and of one dtype")
    B, n, C = x.shape
    full, merged = T * H * W, T * (H // 2) * (W // 2)
    if n != (full if merge else merged) or w.shape != ((C, 4 * C) if merge else (4 * C, C)):
        raise MmditError(f"{name}: shapes do not match the (T, H, W) grid {grid}")
    if y is None:
        y = torch.empty((B, merged if merge else full, C), dtype=y_dtype, device=x.device)
    fn = lib().mmdit_lite_merge if merge else lib().mmdit_lite_unpatchify
    st = fn(x.data_ptr(), _dt(x), w.data_ptr(), _ptr(bias), _dt(bias) if bias is not None else BF16,
            y.data_ptr(), _dt(y), B, T, H, W, C, _stream(x))
    _check(st, f"mmdit_{name}")
    return y


def lite_merge(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], grid: Sequence[int], *,
               y: Optional[torch.Tensor] = None, y_dtype=torch.bfloat16) -> torch.Tensor:
    """Lite 2x2 merge: x [B, T*H*W, C] -> [B, T*(H/2)*(W/2), C] = concat4(x) w^T + bias; w [C, 4C]."""
    return _lite("lite_merge", x, w, bias, grid, y, y_dtype, True)


def lite_unpatchify(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor], grid: Sequence[int], *,
                    y: Optional[torch.Tensor] = None, y_dtype=torch.float32) -> torch.Tensor:
    """Lite unpatchify: x [B, T*(H/2)*(W/2), C] -> [B, T*H*W, C]; w [4C, C]; ``grid`` is the
    full (T, H, W) grid."""
    return _lite("lite_unpatchify", x, w, bias, grid, y, y_dtype, False)


STREAM_KEYS = ("w_mod", "b_mod", "w_qkv", "b_qkv", "q_norm", "k_norm", "w_o", "b_o", "w_fc1", "b_fc1",
               "w_fc2", "b_fc2")


MATRIX_KEYS = ("w_qkv", "w_o", "w_fc1", "w_fc2")
SCALE_KEYS = ("s_qkv", "s_o", "s_fc1", "s_fc2")   # E4M3 matrices: their per-tensor scales


def fp8_block_weights(w: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    """The weights of one stream for the 8-bit block: the four GEMM matrices as E4M3 codes
    (uint8) quantized per tensor by mmdit_quantize_fp8, with their f32 scales under s_qkv,
    s_o, s_fc1, s_fc2; every other weight unchanged.  Done once, at load."""
    out = dict(w)
    for k, sk in zip(MATRIX_KEYS, SCALE_KEYS):
        out[k], out[sk] = quantize_fp8(w[k].contiguous(), per_row=False)
    return out


def _stream_weights(w: Dict[str, torch.Tensor], device: torch.device, matrix_dt: int = BF16) -> StreamWeights:
    sw = StreamWeights()
    mat_want = {F16: torch.float16, FP8_E4M3: torch.uint8}.get(matrix_dt, torch.bfloat16)
    for k in STREAM_KEYS:
        t = w.get(k)
        want = mat_want if k in MATRIX_KEYS else torch.bfloat16
        if t is not None and (not t.is_contiguous() or t.dtype != want):
            raise MmditError(f"weight {k} must be contiguous {want}")
        _on_device(device, **{f"weight {k}": t})
        setattr(sw, k, None if t is None else t.data_ptr())
    if matrix_dt == FP8_E4M3:
        for k in SCALE_KEYS:
            t = w.get(k)
            if t is None or t.dtype != torch.float32 or t.numel() != 1:
                raise MmditError(f"the 8-bit block needs {k}, a one-element f32 tensor")
            _on_device(device, **{f"weight {k}": t})
            setattr(sw, k, t.data_ptr())
    return sw


def block_workspace_bytes(dims: BlockDims, B: int, n_vis: int, n_cond: int) -> int:
    return lib().mmdit_block_workspace_bytes(ctypes.byref(dims), B, n_vis, n_cond)


def block_workspace_offsets(dims: BlockDims, B: int, n_vis: int, n_cond: int):
    arr = (c_size_t * (2 * WS_COUNT))()
    _check(lib().mmdit_block_workspace_offsets(ctypes.byref(dims), B, n_vis, n_cond, arr),
           "mmdit_block_workspace_offsets")
    return [list(arr[:WS_COUNT]), list(arr[WS_COUNT:])]


def block_fwd(dims: BlockDims, w_vis: Dict[str, torch.Tensor], w_cond: Dict[str, torch.Tensor],
              x_vis: torch.Tensor, x_cond: Optional[torch.Tensor], tvec: torch.Tensor, rope: Rope3D, *,
              out_dtype=torch.float32, workspace: Optional[torch.Tensor] = None,
              out_vis: Optional[torch.Tensor] = None, out_cond: Optional[torch.Tensor] = None,
              stage_events: Optional[Sequence[int]] = None):
    """One dual-stream block forward.  Returns (out_vis, out_cond, workspace).
    ``stage_events``: optional 2 * STAGE_COUNT raw hipEvent_t handles (ints or None)
    recorded around each stage on the current stream."""
    _need_gpu(x_vis, x_cond, tvec, workspace)
    _on_device(x_vis.device, x_cond=x_cond, tvec=tvec, workspace=workspace, out_vis=out_vis, out_cond=out_cond)
    B, n_vis, C = x_vis.shape
    n_cond = 0 if x_cond is None else x_cond.shape[1]
    need = block_workspace_bytes(dims, B, n_vis, n_cond)
    if need == 0:
        raise MmditError("invalid block dims")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x_vis.device)
    if out_vis is None:
        out_vis = torch.empty((B, n_vis, C), dtype=out_dtype, device=x_vis.device)
    if out_cond is None and n_cond > 0:
        out_cond = torch.empty((B, n_cond, C), dtype=out_dtype, device=x_vis.device)
    swv = _stream_weights(w_vis, x_vis.device, dims.w_dtype)
    swc = _stream_weights(w_cond, x_vis.device, dims.w_dtype)
    args = (ctypes.byref(dims), ctypes.byref(swv), ctypes.byref(swc), x_vis.data_ptr(),
            _ptr(x_cond) if n_cond else None, _dt(x_vis), tvec.data_ptr(), _dt(tvec),
            ctypes.byref(rope), n_cond, out_vis.data_ptr(), _ptr(out_cond) if n_cond else None,
            _dt(out_vis), workspace.data_ptr(), _workspace_bytes(workspace), B, _stream(x_vis))
    if stage_events is None:
        _check(lib().mmdit_block_fwd(*args), "mmdit_block_fwd")
    else:
        if len(stage_events) != 2 * STAGE_COUNT:
            raise MmditError(f"stage_events needs {2 * STAGE_COUNT} entries")
        arr = (c_void_p * (2 * STAGE_COUNT))(*stage_events)
        _check(lib().mmdit_block_fwd_events(*args, arr), "mmdit_block_fwd_events")
    return out_vis, out_cond, workspace
