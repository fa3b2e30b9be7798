"""GPU parity of the Lite model's hidden-space 2x2 merge and unpatchify (the neighbour
gather fused into the GEMM's loads, the scatter into its stores) against the float64
oracle: small grids with ragged tiles, a single-region grid, and the full 480p grid."""
import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_mmdit_amd as mm
import workloads as wl
from tests.util import assert_close, assert_close_stored, log, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _check(cfg, in_dtype=torch.bfloat16, y_dtype=torch.float32, bias_f32=False):
    raw = wl.lite_inputs(cfg)
    t = {k: to_dev(v, wl.BF16) for k, v in raw.items()}
    if in_dtype == torch.float16:
        for k in ("x", "y", "w_merge", "w_unpatch"):
            t[k] = t[k].to(torch.float16)     # bf16 -> f16 is exact for these magnitudes
    bm, bu = t["b_merge"], t["b_unpatch"]
    if bias_f32:
        bm, bu = bm.float(), bu.float()
    log(f"  {cfg.name}: merge")
    ym = mm.lite_merge(t["x"], t["w_merge"], bm, cfg.grid, y_dtype=y_dtype)
    log(f"  {cfg.name}: unpatchify")
    yu = mm.lite_unpatchify(t["y"], t["w_unpatch"], bu, cfg.grid, y_dtype=y_dtype)
    torch.cuda.synchronize()
    f64 = {k: to_host64(v) for k, v in t.items()}
    ref_m = oracle.lite_merge(f64["x"], f64["w_merge"], f64["b_merge"], cfg.grid)
    ref_u = oracle.lite_unpatchify(f64["y"], f64["w_unpatch"], f64["b_unpatch"], cfg.grid)
    assert ym.shape == ref_m.shape and yu.shape == ref_u.shape
    if y_dtype == torch.float32:
        assert_close("merge", to_host64(ym), ref_m, 1e-4)
        assert_close("unpatchify", to_host64(yu), ref_u, 1e-4)
    else:
        assert_close_stored("merge", to_host64(ym), ref_m, y_dtype, 1e-4)
        assert_close_stored("unpatchify", to_host64(yu), ref_u, y_dtype, 1e-4)


@pytest.mark.parametrize("cfg,in_dtype,y_dtype,bias_f32", [
    (wl.LITE_SMALL, torch.bfloat16, torch.float32, False),
    (wl.LITE_SMALL, torch.float16, torch.bfloat16, True),
    (wl.LiteConfig("lite_c256_grid2x30x52", 256, (2, 30, 52), seed=33), torch.bfloat16, torch.float32, False),
    (wl.LiteConfig("lite_c768_grid1x2x2_b3", 768, (1, 2, 2), batch=3, seed=34), torch.bfloat16, torch.float16, False),
], ids=lambda v: getattr(v, "name", str(v)))
def test_lite_merge_unpatchify(cfg, in_dtype, y_dtype, bias_f32):
    _check(cfg, in_dtype, y_dtype, bias_f32)


def test_lite_merge_unpatchify_480p():
    """The full 480p grid (21 x 30 x 52 -> 21 x 15 x 26 = 8190 merged tokens, C = 3072),
    every output element against the oracle."""
    _check(wl.LITE_480P)


def test_lite_round_trip_selector_weights():
    """Selector weights (merge keeps slot s only; unpatchify places it at position s) give
    back the input bit for bit at every position of the 2x2 regions."""
    c, grid = 256, (2, 4, 6)
    x = torch.randn((1, 48, c), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).cuda()
    eye = torch.eye(c, dtype=torch.bfloat16, device="cuda")
    wm = torch.zeros((c, 4 * c), dtype=torch.bfloat16, device="cuda")
    wu = torch.zeros((4 * c, c), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((1, 48, c), dtype=torch.float32, device="cuda")
    for s in range(4):
        wm.zero_()
        wm[:, s * c:(s + 1) * c] = eye
        y = mm.lite_merge(x, wm, None, grid, y_dtype=torch.bfloat16)
        wu.zero_()
        wu[s * c:(s + 1) * c] = eye
        out += mm.lite_unpatchify(y, wu, None, grid, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(out, x.float())
