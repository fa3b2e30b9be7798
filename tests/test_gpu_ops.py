"""GPU parity of the modulation GEMV, LayerNorm-modulate and the MFMA GEMM (with each
epilogue) against the float64 oracle's steps, on seeded inputs with ragged tiles."""
import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_mmdit_amd as mm
from tests.util import assert_close, assert_close_stored, log, to_host64

pytestmark = pytest.mark.gpu


def _rand(shape, seed, std=1.0, dtype=torch.bfloat16, mean=0.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std + mean).to(dtype).cuda()


@pytest.mark.parametrize("B,C6,Dt,tdt", [(1, 18432, 1536, torch.bfloat16), (2, 6 * 256, 64, torch.float32),
                                          (1, 6 * 3072 + 0, 16, torch.bfloat16)])
def test_modulation_gemv(B, C6, Dt, tdt):
    w = _rand((C6, Dt), 1, 0.02)
    b = _rand((C6,), 2, 0.02)
    t = _rand((B, Dt), 3, 1.0, tdt)
    mod = mm.modulation(w, b, t)
    torch.cuda.synchronize()
    ref = to_host64(t) @ to_host64(w).T + to_host64(b)[None, :]
    assert_close("mod", to_host64(mod), ref, 1e-5)


@pytest.mark.parametrize("xdt,ydt,branch,C,N", [
    (torch.bfloat16, torch.bfloat16, False, 3072, 77),
    (torch.float32, torch.float16, False, 3072, 130),
    (torch.float32, torch.float32, True, 256, 40),
    (torch.bfloat16, torch.float32, True, 3072, 5),
    (torch.float32, torch.bfloat16, False, 1024, 1),
])
def test_modulate_ln(xdt, ydt, branch, C, N):
    B = 2
    x = _rand((B, N, C), 4, 1.3, xdt, mean=0.5)
    mod = _rand((B, 6 * C), 5, 0.8, torch.float32)
    shift, scale, gate = mod[:, 0:C], mod[:, C:2 * C], mod[:, 2 * C:3 * C]
    br = _rand((B, N, C), 6, 1.0, xdt) if branch else None
    xo = torch.empty((B, N, C), dtype=torch.float32, device="cuda") if branch else None
    y = mm.modulate_ln(x, shift, scale, branch=br, gate=gate if branch else None, x_out=xo, y_dtype=ydt)
    torch.cuda.synchronize()
    x64 = to_host64(x)
    if branch:
        x64 = x64 + to_host64(gate)[:, None, :] * to_host64(br)
        assert_close("x_out", to_host64(xo), x64, 1e-6)
    ref = oracle.modulate(oracle.layer_norm(x64, 1e-6), to_host64(shift), to_host64(scale))
    if ydt == torch.float32:
        assert_close("y", to_host64(y), ref, 1e-5)
    else:
        assert_close_stored("y", to_host64(y), ref, ydt, 1e-4)


@pytest.mark.parametrize("M,N,K,dt,epi,ydt", [
    (300, 768, 256, torch.bfloat16, mm.EPI_NONE, torch.bfloat16),
    (513, 512, 512, torch.bfloat16, mm.EPI_NONE, torch.float32),
    (77, 1024, 3072, torch.float16, mm.EPI_GELU, torch.float16),
    (260, 256, 1024, torch.bfloat16, mm.EPI_GELU, torch.float32),
    (1, 256, 64, torch.bfloat16, mm.EPI_NONE, torch.float32),
    (40, 300, 128, torch.bfloat16, mm.EPI_NONE, torch.float32),
    # odd counts of K = 64 stages past the first (the two-stage loop's trailing stage)
    (200, 512, 192, torch.float16, mm.EPI_GELU, torch.float16),
    (129, 260, 320, torch.bfloat16, mm.EPI_NONE, torch.float32),
])
def test_linear(M, N, K, dt, epi, ydt):
    x = _rand((M, K), 7, 1.0, dt)
    w = _rand((N, K), 8, 0.02, dt)
    b = _rand((N,), 9, 0.02)
    y = mm.linear(x, w, b, epilogue=epi, y_dtype=ydt)
    torch.cuda.synchronize()
    ref = oracle.linear(to_host64(x), to_host64(w), to_host64(b))
    if epi == mm.EPI_GELU:
        ref = oracle.gelu(ref)
    if ydt == torch.float32:
        assert_close("y", to_host64(y), ref, 1e-4)
    else:
        assert_close_stored("y", to_host64(y), ref, ydt, 1e-4)


@pytest.mark.parametrize("resdt,ydt", [(torch.bfloat16, torch.float32), (torch.float32, torch.float32),
                                       (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("B,n", [(2, 150), (3, 128), (3, 127), (2, 300)])
def test_linear_gated_residual(resdt, ydt, B, n):
    """Batch items of 150 rows start inside a wave's 128 rows, of 128 rows on a wave's first
    row, of 300 rows inside the second 256-row tile; items shorter than 128 rows take the
    epilogue's per-row gate lookup."""
    C, K = 512, 1024
    x = _rand((B * n, K), 10, 1.0)
    w = _rand((C, K), 11, 0.02)
    b = _rand((C,), 12, 0.02)
    res = _rand((B * n, C), 13, 1.0, resdt)
    mod = _rand((B, 6 * C), 14, 0.8, torch.float32)
    gate = mod[:, 5 * C:]
    y = mm.linear(x, w, b, epilogue=mm.EPI_GATED_RES, res=res, gate=gate, rows_per_batch=n, y_dtype=ydt)
    torch.cuda.synchronize()
    a = oracle.linear(to_host64(x), to_host64(w), to_host64(b)).reshape(B, n, C)
    ref = to_host64(res).reshape(B, n, C) + to_host64(gate)[:, None, :] * a
    if ydt == torch.float32:
        assert_close("y", to_host64(y).reshape(B, n, C), ref, 1e-4)
    else:
        assert_close_stored("y", to_host64(y).reshape(B, n, C), ref, ydt, 1e-4)


def test_linear_full_width_shapes():
    """The block's GEMM shapes at full width on a few hundred rows (ragged M)."""
    for N, K in ((9216, 3072), (3072, 3072), (12288, 3072), (3072, 12288)):
        log(f"  N={N} K={K}")
        x = _rand((333, K), 1000 + N, 1.0)
        w = _rand((N, K), 2000 + K, 0.02)
        y = mm.linear(x, w, None, y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert_close(f"y[{N}x{K}]", to_host64(y), to_host64(x) @ to_host64(w).T, 1e-4)


@pytest.mark.parametrize("src,dst", [(torch.bfloat16, torch.float16), (torch.float16, torch.bfloat16),
                                     (torch.float32, torch.float16), (torch.float32, torch.bfloat16),
                                     (torch.bfloat16, torch.float32)])
@pytest.mark.parametrize("n", [0, 5, 8 * 1000 + 3, 3 * 1024 * 1024])
def test_cast_matches_round_to_nearest_even(src, dst, n):
    """mmdit_cast against the CPU's round-to-nearest-even conversion, bit for bit (values span
    f16's subnormal and overflow ranges)."""
    g = torch.Generator().manual_seed(n + 7)
    x = (torch.randn(n, generator=g) * torch.exp2(torch.randint(-20, 18, (n,), generator=g).float())).to(src)
    y = mm.cast(x.cuda(), dst)
    torch.cuda.synchronize()
    ref = x.to(dst)
    assert torch.equal(y.cpu().view(torch.int16 if dst != torch.float32 else torch.int32),
                       ref.view(torch.int16 if dst != torch.float32 else torch.int32))


def test_cast_in_place_bf16_to_f16():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(4099, generator=g).to(torch.bfloat16)
    d = x.cuda()
    mm.cast(d, torch.float16, out=d.view(torch.float16))
    torch.cuda.synchronize()
    assert torch.equal(d.view(torch.float16).cpu(), x.to(torch.float16))


def test_f16_outputs_saturate_instead_of_overflowing():
    """f16 GEMM and LN-modulate outputs beyond the f16 range saturate at +-65504 (an
    infinity there would become NaN in the next LayerNorm or softmax); NaN stays NaN."""
    M, N, K = 64, 256, 64
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    x[:, 0] = 300.0
    x[1, 0] = -300.0
    x[2, 0] = float("nan")
    w = torch.zeros((N, K), dtype=torch.bfloat16)
    w[:, 0] = 1000.0                                   # products 3e5, beyond 65504
    w[0, 0] = 1.0                                      # column 0 stays in range: 300
    y = mm.linear(x.cuda(), w.cuda(), None, y_dtype=torch.float16)
    torch.cuda.synchronize()
    y = y.float().cpu()
    assert torch.all(y[0, 1:] == 65504.0) and torch.all(y[1, 1:] == -65504.0)
    assert y[0, 0] == 300.0 and torch.isnan(y[2]).all()
    assert torch.all(y[3:, 1:] == 65504.0)
    # LN-modulate: shift 1e6 pushes every output past the f16 range
    B, Nt, C = 1, 4, 256
    xs = torch.randn((B, Nt, C)).to(torch.bfloat16).cuda()
    mod = torch.zeros((B, 6 * C), dtype=torch.float32)
    mod[:, :C] = 1e6
    mod = mod.cuda()
    h = mm.modulate_ln(xs, mod[:, :C], mod[:, C:2 * C], y_dtype=torch.float16)
    torch.cuda.synchronize()
    assert torch.all(h.float().cpu() == 65504.0)
