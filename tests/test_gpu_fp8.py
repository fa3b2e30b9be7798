"""GPU parity of the FP8 path (OCP E4M3 codes, per-token activation scales, per-tensor
weight scales) against the float64 oracle: the quantized codes and scales bit for bit, the
FP8 Linear against the oracle's exact product of the same codes.

Bar for the FP8 Linear: max|err| / rms <= 3e-4.  The codes and scales are identical on both
sides, so only the summation differs: the gfx950 32x32x64 FP8 MFMA does not add its 64
products exactly (on exactly representable operands one instruction deviates by up to ~4e-5
of its result's rms; over the few million outputs of these tests the largest deviation seen
is ~1.1e-4), and f32 accumulation over K / 64 instructions adds a few 1e-7."""
import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_mmdit_amd as mm
from tests.util import assert_close, log, to_host64

pytestmark = pytest.mark.gpu
TOL_FP8_LINEAR = 3e-4


def _rand(shape, seed, std=1.0, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(dtype).cuda()


@pytest.mark.parametrize("dtype,rows,cols", [(torch.bfloat16, 300, 3072), (torch.float16, 77, 12288),
                                             (torch.float16, 6, 3072), (torch.bfloat16, 3, 12288),
                                             (torch.float32, 5, 136), (torch.bfloat16, 1, 8)])
@pytest.mark.parametrize("per_row", [True, False])
def test_quantize_fp8_codes_bit_exact(dtype, rows, cols, per_row):
    x = _rand((rows, cols), rows + cols, 1.0, dtype)
    if rows > 2:
        x[1] = 0                              # all-zero row: scale 1, codes 0
        x[2] *= 1e-3                          # small row: exercises the subnormal codes
    q, s = mm.quantize_fp8(x, per_row=per_row)
    torch.cuda.synchronize()
    vals, ref_s = oracle.quantize_fp8(to_host64(x), per_row=per_row)
    ref_q = oracle.fp8_e4m3_code(vals)
    got_q = q.cpu().numpy()
    bad = np.count_nonzero(got_q != ref_q)
    log(f"  codes differing: {bad} of {got_q.size}")
    assert bad == 0
    np.testing.assert_array_equal(s.cpu().numpy(), ref_s)


@pytest.mark.parametrize("M,N,K,epi,ydt", [
    (300, 768, 256, mm.EPI_NONE, torch.bfloat16),
    (513, 512, 512, mm.EPI_NONE, torch.float32),
    (77, 1024, 3072, mm.EPI_GELU, torch.float32),
    (40, 300, 128, mm.EPI_NONE, torch.float32),
    (1, 256, 64, mm.EPI_NONE, torch.float32),
    (260, 256, 12288, mm.EPI_NONE, torch.float32),
])
def test_linear_fp8(M, N, K, epi, ydt):
    x = _rand((M, K), 7, 1.0)
    w = _rand((N, K), 8, 0.02)
    b = _rand((N,), 9, 0.02)
    xq, xs = mm.quantize_fp8(x, per_row=True)
    wq, ws = mm.quantize_fp8(w, per_row=False)
    y = mm.linear_fp8(xq, xs, wq, ws, b, epilogue=epi, y_dtype=ydt)
    torch.cuda.synchronize()
    ref = oracle.fp8_linear(to_host64(x), to_host64(w), to_host64(b))
    if epi == mm.EPI_GELU:
        ref = oracle.gelu(ref)
    if ydt == torch.float32:
        assert_close("y", to_host64(y), ref, TOL_FP8_LINEAR)
    else:
        from tests.util import assert_close_stored
        assert_close_stored("y", to_host64(y), ref, ydt, TOL_FP8_LINEAR)
    exact = oracle.linear(to_host64(x), to_host64(w), to_host64(b))
    if epi == mm.EPI_GELU:
        exact = oracle.gelu(exact)
    log(f"  FP8 quantization error vs the unquantized product: {oracle.rel_max_err(to_host64(y), exact):.3e}")


def test_linear_fp8_gated_residual():
    B, n, C, K = 2, 150, 512, 1024
    x = _rand((B * n, K), 10, 1.0)
    w = _rand((C, K), 11, 0.02)
    b = _rand((C,), 12, 0.02)
    res = _rand((B * n, C), 13, 1.0, torch.float32)
    gate = _rand((B, 6 * C), 14, 0.8, torch.float32)[:, 5 * C:]
    xq, xs = mm.quantize_fp8(x)
    wq, ws = mm.quantize_fp8(w, per_row=False)
    y = mm.linear_fp8(xq, xs, wq, ws, b, epilogue=mm.EPI_GATED_RES, res=res, gate=gate, rows_per_batch=n,
                      y_dtype=torch.float32)
    torch.cuda.synchronize()
    a = oracle.fp8_linear(to_host64(x), to_host64(w), to_host64(b)).reshape(B, n, C)
    ref = to_host64(res).reshape(B, n, C) + to_host64(gate)[:, None, :] * a
    assert_close("y", to_host64(y).reshape(B, n, C), ref, TOL_FP8_LINEAR)


def test_linear_fp8_block_shapes():
    """The block's four GEMM shapes at full width on a few hundred rows (ragged M)."""
    for N, K in ((9216, 3072), (3072, 3072), (12288, 3072), (3072, 12288)):
        log(f"  N={N} K={K}")
        x = _rand((333, K), 1000 + N, 1.0)
        w = _rand((N, K), 2000 + K, 0.02)
        xq, xs = mm.quantize_fp8(x)
        wq, ws = mm.quantize_fp8(w, per_row=False)
        y = mm.linear_fp8(xq, xs, wq, ws, None, y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close(f"y[{N}x{K}]", to_host64(y), oracle.fp8_linear(to_host64(x), to_host64(w), None), TOL_FP8_LINEAR)
