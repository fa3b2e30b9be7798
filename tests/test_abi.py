"""The C-ABI library loads, exports every function include/mmdit.h declares, and rejects
invalid arguments with the documented status before any HIP call (no GPU needed: these
calls return from host-side validation)."""
import ctypes
import os
import re

import pytest

import video_diffusion_transformer_mmdit_amd as mm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmdit.h")

ERR_NULL, ERR_ALIGN, ERR_SHAPE, ERR_DTYPE, ERR_WS, ERR_HIP, ERR_ALIAS = 1, 2, 3, 4, 5, 6, 7


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(mmdit_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mm.library_path()):
        pytest.skip("libmmdit.so not built")
    return mm.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in mmdit.h but not exported"
    for n in ("mmdit_modulate_ln", "mmdit_qk_norm_rope", "mmdit_joint_attention", "mmdit_block_fwd"):
        assert n in names


def test_status_strings_and_version(L):
    assert mm.abi_version() == 8
    assert L.mmdit_status_str(0) == b"MMDIT_OK"
    assert L.mmdit_status_str(ERR_ALIAS) == b"MMDIT_ERR_ALIAS"
    assert L.mmdit_status_str(99) == b"MMDIT_ERR_UNKNOWN"


def _fake(addr):
    """A non-null, 16-byte aligned address that is never dereferenced (validation fails first)."""
    return ctypes.c_void_p(addr)


def test_qk_norm_rope_validation(L):
    p = _fake(0x10000)
    rope = mm.Rope3D.make((2, 2, 2))
    f = L.mmdit_qk_norm_rope
    args = [p, _fake(0x20000), mm.BF16, 3 * 128, p, p, mm.BF16, 0, p, _fake(0x20000), mm.BF16, 3 * 128,
            1, 8, 1, 128, 1e-6, ctypes.byref(rope), None]
    a = list(args); a[15] = 64
    assert f(*a) == ERR_SHAPE                                       # D != 128
    a = list(args); a[13] = 9
    assert f(*a) == ERR_SHAPE and b"T * H * W" in L.mmdit_last_error()
    bad = mm.Rope3D.make((2, 2, 2), (16, 55, 57))
    a = list(args); a[17] = ctypes.byref(bad)
    assert f(*a) == ERR_SHAPE                                       # odd band
    a = list(args); a[0] = None
    assert f(*a) == ERR_NULL
    a = list(args); a[0] = _fake(0x10008)
    assert f(*a) == ERR_ALIGN
    a = list(args); a[2] = 5
    assert f(*a) == ERR_DTYPE
    a = list(args); a[8] = _fake(0x10000 + 64 * 2)                  # q_out half-overlapping q
    assert f(*a) == ERR_ALIAS
    a = list(args); a[13] = 0                                       # N = 0 with a grid of 8 -> shape
    assert f(*a) == ERR_SHAPE


def test_joint_attention_validation(L):
    p, o = _fake(0x10000), _fake(0x900000)
    f = L.mmdit_joint_attention
    args = [p, p, p, 10, p, p, p, 3, mm.BF16, mm.BF16, 256, 1, 2, 128, 0.088, o, _fake(0xA00000), mm.F32, 256, None,
            None, 0, None]
    a = list(args); a[13] = 96
    assert f(*a) == ERR_SHAPE
    a = list(args); a[3] = 0; a[7] = 0
    assert f(*a) == ERR_SHAPE                                       # no tokens at all
    a = list(args); a[15] = None
    assert f(*a) == ERR_NULL
    a = list(args); a[8] = mm.F32
    assert f(*a) == ERR_DTYPE                                       # f32 Q/K with a 16-bit V
    a = list(args); a[9] = 7
    assert f(*a) == ERR_DTYPE
    a = list(args); a[15] = p
    assert f(*a) == ERR_ALIAS                                       # output on top of the inputs
    a = list(args); a[14] = 0.0
    assert f(*a) == ERR_SHAPE
    a = list(args); a[10] = 100
    assert f(*a) == ERR_SHAPE                                       # row stride < H*D
    a = list(args); a[20] = _fake(0xB00010); a[21] = 1 << 20
    assert f(*a) == ERR_ALIGN                                       # workspace not 256-byte aligned
    a = list(args); a[20] = p; a[21] = 1 << 20
    assert f(*a) == ERR_ALIAS                                       # workspace on top of the inputs
    a = list(args); a[20] = _fake(0x8FFF00); a[21] = 1 << 20
    assert f(*a) == ERR_ALIAS                                       # workspace running into o_vis
    a = list(args); a[20] = _fake(0xA00000); a[21] = 256
    assert f(*a) == ERR_ALIAS                                       # workspace on o_cond
    a = list(args); a[19] = _fake(0xC00000); a[20] = _fake(0xC00000); a[21] = 256
    assert f(*a) == ERR_ALIAS                                       # workspace on lse


def test_linear_modulate_modulation_validation(L):
    p = _fake(0x10000)
    assert L.mmdit_linear(p, p, mm.BF16, None, mm.BF16, _fake(0x900000), mm.BF16, 10, 256, 100,
                          mm.EPI_NONE, None, mm.F32, None, 0, 10, None) == ERR_SHAPE      # K % 64
    assert L.mmdit_linear(p, p, mm.BF16, None, mm.BF16, _fake(0x900000), mm.BF16, 10, 258, 128,
                          mm.EPI_NONE, None, mm.F32, None, 0, 10, None) == ERR_SHAPE      # N % 4
    assert L.mmdit_linear(p, p, mm.BF16, None, mm.BF16, _fake(0x900000), mm.BF16, 1 << 20, 256, 1024,
                          mm.EPI_NONE, None, mm.F32, None, 0, 10, None) == ERR_SHAPE      # 32-bit offsets
    assert L.mmdit_linear(p, p, mm.BF16, None, mm.BF16, _fake(0x900000), mm.F32, 10, 256, 128,
                          mm.EPI_GATED_RES, p, mm.F32, p, 258, 10, None) == ERR_SHAPE     # gate_stride % 4
    assert L.mmdit_linear(p, p, mm.F32, None, mm.BF16, _fake(0x900000), mm.BF16, 10, 256, 128,
                          mm.EPI_NONE, None, mm.F32, None, 0, 10, None) == ERR_DTYPE
    assert L.mmdit_linear(p, p, mm.BF16, None, mm.BF16, _fake(0x900000), mm.F32, 10, 256, 128,
                          mm.EPI_GATED_RES, None, mm.F32, None, 256, 10, None) == ERR_NULL
    assert L.mmdit_modulate_ln(p, mm.BF16, None, mm.BF16, None, None, p, p, 3072, _fake(0x900000), mm.BF16,
                               1, 4, 3004, 1e-6, None) == ERR_SHAPE                      # C % 8
    assert L.mmdit_modulate_ln(p, mm.BF16, p, mm.BF16, None, None, p, p, 3072, _fake(0x900000), mm.BF16,
                               1, 4, 3072, 1e-6, None) == ERR_NULL                       # branch w/o gate
    assert L.mmdit_modulate_ln(p, mm.BF16, None, mm.BF16, None, None, p, p, 3072, p, mm.BF16,
                               1, 4, 3072, 1e-6, None) == ERR_ALIAS
    assert L.mmdit_modulation(p, None, p, mm.BF16, _fake(0x900000), 1, 18432, 1500, None) == ERR_SHAPE


def test_block_workspace_and_validation(L):
    import torch
    dims = mm.BlockDims.make(3072, 24, 12288, 1536, act_dtype=torch.bfloat16)
    n = mm.block_workspace_bytes(dims, 1, 32760, 512)
    # mod + h + qkv + x1 + g per stream, f32 residual, bf16 intermediates: no weight copies
    expect = 0
    for s, rows in enumerate((32760, 512)):
        for sz in (6 * 3072 * 4, rows * 3072 * 2, rows * 9216 * 2, rows * 3072 * 4, rows * 12288 * 2):
            expect += (sz + 255) // 256 * 256
        if s == 0:
            expect += 256 * 256 * 256 * 4          # split-tail partial sums
    assert n == expect
    offs = mm.block_workspace_offsets(dims, 1, 32760, 512)
    assert offs[0][mm.WS_MOD] == 0 and offs[0][mm.WS_W1] == 2 ** 64 - 1
    d16 = mm.BlockDims.make(3072, 24, 12288, 1536, act_dtype=torch.float16)
    per_stream = (3 * 3072 * 3072 + 3072 * 3072 + 2 * 12288 * 3072) * 2
    assert mm.block_workspace_bytes(d16, 1, 32760, 512) == n + 2 * per_stream
    d16w = mm.BlockDims.make(3072, 24, 12288, 1536, act_dtype=torch.float16, matrix_dtype=torch.float16)
    assert mm.block_workspace_bytes(d16w, 1, 32760, 512) == n      # f16 matrices given: no copies
    mixed = mm.BlockDims.make(3072, 24, 12288, 1536, act_dtype=torch.bfloat16, matrix_dtype=torch.float16)
    assert mm.block_workspace_bytes(mixed, 1, 100, 5) == 0          # f16 matrices need f16 operands
    bad = mm.BlockDims.make(3000, 24, 12288, 1536)
    assert mm.block_workspace_bytes(bad, 1, 100, 5) == 0
    rope = mm.Rope3D.make((21, 30, 52))
    sw = mm._abi.StreamWeights()
    p = _fake(0x10000)
    st = L.mmdit_block_fwd(ctypes.byref(dims), ctypes.byref(sw), ctypes.byref(sw), p, p, mm.BF16, p, mm.BF16,
                           ctypes.byref(rope), 512, p, p, mm.F32, _fake(0x100000), 1024, 1, None)
    assert st == ERR_NULL                                            # weights missing
    for k in mm._abi.STREAM_KEYS:
        setattr(sw, k, 0x20000)
    st = L.mmdit_block_fwd(ctypes.byref(dims), ctypes.byref(sw), ctypes.byref(sw), p, p, mm.BF16, p, mm.BF16,
                           ctypes.byref(rope), 512, p, p, mm.F32, _fake(0x100000), 1024, 1, None)
    assert st == ERR_WS


def test_timestep_embed_validation(L):
    p, o1, o2, o3 = _fake(0x10000), _fake(0x900000), _fake(0xA00000), _fake(0xB00000)
    args = lambda B, fd, dh, dt, wdt=mm.BF16, mp=10000.0, t=p, h=o1, e=o2, v=o3: (  # noqa: E731
        t, B, p, None, p, None, p, None, wdt, fd, dh, dt, mp, h, e, v, None)
    assert L.mmdit_timestep_embed(*args(2, 250, 3072, 1536)) == ERR_SHAPE     # freq_dim % 16
    assert L.mmdit_timestep_embed(*args(2, 256, 3070, 1536)) == ERR_SHAPE     # hidden % 8
    assert L.mmdit_timestep_embed(*args(2, 256, 3072, 0)) == ERR_SHAPE        # Dt >= 1
    assert L.mmdit_timestep_embed(*args(2, 256, 3072, 16, mp=1.0)) == ERR_SHAPE
    assert L.mmdit_timestep_embed(*args(2, 256, 3072, 16, wdt=mm.F16)) == ERR_DTYPE
    assert L.mmdit_timestep_embed(*args(2, 256, 3072, 16, t=None)) == ERR_NULL
    assert L.mmdit_timestep_embed(*args(2, 256, 3072, 16, h=_fake(0x900008))) == ERR_ALIGN
    assert L.mmdit_timestep_embed(*args(2, 256, 3072, 16, e=o1)) == ERR_ALIAS  # outputs overlap
    assert L.mmdit_timestep_embed(*args(2, 256, 3072, 16, v=p)) == ERR_ALIAS   # tvec over t / weights
    assert L.mmdit_timestep_embed(*args(0, 256, 3072, 16, t=None)) == 0        # empty batch: no work


def test_lite_merge_unpatchify_validation(L):
    p, y = _fake(0x10000), _fake(0x90000000)
    for fn in (L.mmdit_lite_merge, L.mmdit_lite_unpatchify):
        assert fn(p, mm.BF16, p, None, mm.BF16, y, mm.F32, 1, 21, 45, 80, 3072, None) == ERR_SHAPE   # odd H
        assert fn(p, mm.BF16, p, None, mm.BF16, y, mm.F32, 1, 21, 30, 51, 3072, None) == ERR_SHAPE   # odd W
        assert fn(p, mm.BF16, p, None, mm.BF16, y, mm.F32, 1, 21, 30, 52, 3000, None) == ERR_SHAPE   # C % 256
        assert fn(p, mm.F32, p, None, mm.BF16, y, mm.F32, 1, 21, 30, 52, 3072, None) == ERR_DTYPE
        assert fn(p, mm.BF16, p, p, mm.F16, y, mm.F32, 1, 21, 30, 52, 3072, None) == ERR_DTYPE      # bias dtype
        assert fn(None, mm.BF16, p, None, mm.BF16, y, mm.F32, 1, 21, 30, 52, 3072, None) == ERR_NULL
        assert fn(p, mm.BF16, p, None, mm.BF16, _fake(0x90000008), mm.F32, 1, 21, 30, 52, 3072, None) == ERR_ALIGN
        assert fn(p, mm.BF16, p, None, mm.BF16, p, mm.F32, 1, 21, 30, 52, 3072, None) == ERR_ALIAS
        assert fn(p, mm.BF16, p, None, mm.BF16, y, mm.F32, 16, 21, 30, 52, 3072, None) == ERR_SHAPE  # > 2^31 B
        assert fn(None, mm.BF16, None, None, mm.BF16, None, mm.F32, 0, 21, 30, 52, 3072, None) == 0  # empty


def test_fp8_validation(L):
    p, y = _fake(0x10000), _fake(0x900000)
    assert L.mmdit_quantize_fp8(p, mm.BF16, 4, 12, 1, y, _fake(0xA00000), None) == ERR_SHAPE      # cols % 8
    assert L.mmdit_quantize_fp8(p, mm.FP8_E4M3, 4, 16, 1, y, _fake(0xA00000), None) == ERR_DTYPE
    assert L.mmdit_quantize_fp8(p, mm.BF16, 4, 16, 1, None, _fake(0xA00000), None) == ERR_NULL
    assert L.mmdit_quantize_fp8(p, mm.BF16, 4, 16, 1, _fake(0x900008), _fake(0xA00000), None) == ERR_ALIGN
    assert L.mmdit_quantize_fp8(p, mm.BF16, 4, 16, 1, p, _fake(0xA00000), None) == ERR_ALIAS
    assert L.mmdit_quantize_fp8(None, mm.BF16, 0, 16, 1, None, None, None) == 0
    s = _fake(0xB00000)
    assert L.mmdit_linear_fp8(p, s, p, s, None, mm.BF16, y, mm.F32, 10, 256, 100, mm.EPI_NONE, None, mm.F32,
                              None, 0, 10, None) == ERR_SHAPE                                     # K % 64
    assert L.mmdit_linear_fp8(p, None, p, s, None, mm.BF16, y, mm.F32, 10, 256, 128, mm.EPI_NONE, None, mm.F32,
                              None, 0, 10, None) == ERR_NULL                                      # x_scale
    assert L.mmdit_linear_fp8(p, s, p, s, None, mm.BF16, p, mm.F32, 10, 256, 128, mm.EPI_NONE, None, mm.F32,
                              None, 0, 10, None) == ERR_ALIAS
    assert L.mmdit_linear_fp8(p, s, p, s, None, mm.BF16, y, mm.F32, 1 << 24, 256, 256, mm.EPI_NONE, None, mm.F32,
                              None, 0, 10, None) == ERR_SHAPE                                     # 2^31 bytes


def test_cast_validation(L):
    p, y = _fake(0x10000), _fake(0x900000)
    assert L.mmdit_cast(p, mm.BF16, y, mm.F16, -1, None) == ERR_SHAPE
    assert L.mmdit_cast(p, mm.BF16, y, mm.F16, 1 << 31, None) == ERR_SHAPE
    assert L.mmdit_cast(p, mm.BF16, y, mm.BF16, 16, None) == ERR_DTYPE                  # same type
    assert L.mmdit_cast(p, mm.FP8_E4M3, y, mm.F16, 16, None) == ERR_DTYPE
    assert L.mmdit_cast(None, mm.BF16, y, mm.F16, 16, None) == ERR_NULL
    assert L.mmdit_cast(_fake(0x10008), mm.BF16, y, mm.F16, 16, None) == ERR_ALIGN
    assert L.mmdit_cast(p, mm.F32, _fake(0x10010), mm.F16, 16, None) == ERR_ALIAS        # partial overlap
    assert L.mmdit_cast(p, mm.F32, p, mm.F16, 16, None) == ERR_ALIAS                     # in place across sizes
    assert L.mmdit_cast(None, mm.BF16, None, mm.F16, 0, None) == 0


def test_attention_8bit_validation(L):
    import ctypes as C
    p = _fake(0x10000)
    st = mm._abi.Attn8Stream(0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000)
    bad = mm._abi.Attn8Stream(0x10000000, None, 0x30000000, 0x40000000, 0x50000000)
    sv = _fake(0x60000000)
    q = L.mmdit_attn8_quantize
    assert q(p, p, p, 100, None, None, None, 0, mm.BF16, 3072, 1, 24, 64, C.byref(st), None, sv, None) == ERR_SHAPE
    assert q(p, p, p, 100, None, None, None, 0, mm.FP8_E4M3, 3072, 1, 24, 128, C.byref(st), None, sv, None) == ERR_DTYPE
    assert q(p, p, p, 100, None, None, None, 0, mm.BF16, 3000, 1, 24, 128, C.byref(st), None, sv, None) == ERR_ALIGN
    assert q(p, p, p, 100, None, None, None, 0, mm.BF16, 3072, 1, 24, 128, C.byref(bad), None, sv, None) == ERR_NULL
    assert q(p, p, p, 100, p, p, p, 5, mm.BF16, 3072, 1, 24, 128, C.byref(st), None, sv, None) == ERR_NULL
    assert q(None, None, None, 0, None, None, None, 0, mm.BF16, 3072, 1, 24, 128, None, None, None, None) == 0
    a = L.mmdit_joint_attention_8bit
    assert a(C.byref(st), 100, None, 0, sv, 1, 24, 128, 0.0, p, None, mm.F32, 3072, None, None, 0, None) == ERR_SHAPE
    assert a(C.byref(st), 100, None, 0, None, 1, 24, 128, 0.088, p, None, mm.F32, 3072, None, None, 0, None) == ERR_NULL
    assert a(C.byref(st), 100, None, 0, sv, 1, 24, 128, 0.088, p, None, mm.FP8_E4M3, 3072, None, None, 0, None) == ERR_DTYPE
    assert a(C.byref(st), 100, C.byref(st), 5, sv, 1, 24, 128, 0.088, p, None, mm.F32, 3072, None, None, 0, None) == ERR_NULL
    assert a(C.byref(st), 100, None, 0, _fake(0x60000004), 1, 24, 128, 0.088, p, None, mm.F32, 3072, None, None, 0, None) == ERR_ALIGN
    o = _fake(0x70000000)
    assert a(C.byref(st), 100, None, 0, sv, 1, 24, 128, 0.088, _fake(0x10000000), None, mm.F32, 3072, None, None, 0,
             None) == ERR_ALIAS                                     # output on the Q codes
    assert a(C.byref(st), 100, None, 0, sv, 1, 24, 128, 0.088, o, None, mm.F32, 3072, None, _fake(0x50000000),
             1 << 20, None) == ERR_ALIAS                            # workspace on the V codes
    assert a(C.byref(st), 100, None, 0, sv, 1, 24, 128, 0.088, o, None, mm.F32, 3072, None, o, 1 << 20,
             None) == ERR_ALIAS                                     # workspace on the output
    assert a(C.byref(st), 100, None, 0, sv, 1, 24, 128, 0.088, o, None, mm.F32, 3072, _fake(0x7F000000),
             _fake(0x7F000000), 256, None) == ERR_ALIAS             # workspace on lse

    assert a(C.byref(st), 100, None, 0, sv, 1, 24, 128, 0.088, p, None, mm.F32, 3072, None, _fake(0x60000010), 1 << 20, None) == ERR_ALIGN

def test_binding_rejects_host_or_foreign_workspace_before_any_launch():
    """A workspace (or output) that is not a GPU tensor on the inputs' device raises in the
    binding: its host address would otherwise reach the split-tail kernels, which write
    through it."""
    import torch
    from video_diffusion_transformer_mmdit_amd import _abi
    cuda0 = torch.device("cuda", 0)
    host = torch.empty(256, dtype=torch.uint8)
    with pytest.raises(mm.MmditError, match="workspace must be a GPU tensor"):
        _abi._on_device(cuda0, workspace=host)
    with pytest.raises(mm.MmditError, match="o_vis must be a GPU tensor"):
        _abi._on_device(cuda0, o_vis=host)
    with pytest.raises(mm.MmditError, match="must be a GPU tensor"):
        _abi._on_device(torch.device("cpu"), workspace=host)
    _abi._on_device(cuda0, workspace=None, o_cond=None)       # absent tensors are fine
    with pytest.raises(mm.MmditError, match="contiguous"):
        _abi._workspace_bytes(torch.empty((4, 64), dtype=torch.uint8)[:, ::2])
    assert _abi._workspace_bytes(torch.empty(300, dtype=torch.float32)) == 1200
    # through the public entry points (host inputs fail first here; on a GPU machine the
    # workspace check is reached, see test_gpu_attention)
    q = torch.empty((1, 8, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(mm.MmditError):
        mm.joint_attention(q, q, q, workspace=host)
