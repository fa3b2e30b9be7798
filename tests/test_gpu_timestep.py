"""GPU parity of the timestep path (sinusoid -> MLP(SiLU) -> SiLU -> bottleneck Linear) and of
the 16-wide Lite bottleneck through the modulation GEMV and the whole block, against the
float64 oracle on seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_mmdit_amd as mm
import workloads as wl
from tests.util import assert_close, log, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _run(raw, dtype, max_period=10000.0):
    t = to_dev(raw["t"], wl.F32)
    ws = [to_dev(raw[k], dtype) for k in wl.TIMESTEP_WEIGHTS]
    hidden, temb, tvec = mm.timestep_embed(t, *ws, max_period=max_period)
    torch.cuda.synchronize()
    ref = oracle.timestep_path(raw["t"].astype(np.float64), *[wl.to_f64(raw[k], dtype) for k in wl.TIMESTEP_WEIGHTS],
                               dim=raw["w1"].shape[1], max_period=max_period)
    return {"hidden": hidden, "temb": temb, "tvec": tvec}, ref


@pytest.mark.parametrize("cfg", [wl.TIMESTEP_FULL, wl.TIMESTEP_LITE], ids=lambda c: c.name)
def test_timestep_path_bf16_weights(cfg):
    raw = wl.timestep_inputs(cfg)
    got, ref = _run(raw, wl.BF16)
    for k in ("hidden", "temb", "tvec"):
        assert_close(k, to_host64(got[k]), ref[k], 1e-4)


def test_timestep_path_edges_f32_weights_and_batch_chunks():
    """t = 0 and t = 1000 and a batch of 7 (more vectors than one launch stages in LDS at
    3072 wide), f32 weights, a non-default frequency count and max_period."""
    cfg = wl.TimestepConfig("timestep_b7_f128_h3072_dt40", 7, freq_dim=128, hidden=3072, t_dim=40, seed=23)
    raw = wl.timestep_inputs(cfg, weight_dtype=wl.F32, weight_std=0.05)
    raw["t"][0], raw["t"][1] = 0.0, 1000.0
    got, ref = _run(raw, wl.F32, max_period=5000.0)
    for k in ("hidden", "temb", "tvec"):
        assert_close(k, to_host64(got[k]), ref[k], 1e-4)


def test_timestep_path_empty_batch():
    cfg = wl.TIMESTEP_LITE
    raw = wl.timestep_inputs(cfg)
    ws = [to_dev(raw[k], wl.BF16) for k in wl.TIMESTEP_WEIGHTS]
    t = torch.empty(0, dtype=torch.float32, device="cuda")
    h, e, v = mm.timestep_embed(t, *ws)
    assert h.shape == (0, 3072) and v.shape == (0, 16)


@pytest.mark.parametrize("Dt", [8, 16, 24, 40])
def test_modulation_short_bottleneck(Dt):
    """The per-(block, stream) modulation Linear for narrow bottlenecks (Lite: 16)."""
    rng = np.random.default_rng(100 + Dt)
    w = wl.round_to_bf16_bits(rng.standard_normal((18432, Dt)).astype(np.float32) * 0.02)
    b = wl.round_to_bf16_bits(rng.standard_normal(18432).astype(np.float32) * 0.02)
    t = rng.standard_normal((3, Dt)).astype(np.float32)
    mod = mm.modulation(to_dev(w, wl.BF16), to_dev(b, wl.BF16), to_dev(t, wl.F32))
    torch.cuda.synchronize()
    ref = oracle.modulation(wl.to_f64(w, wl.BF16), wl.to_f64(b, wl.BF16), t.astype(np.float64))
    ref = np.concatenate([ref[k] for k in oracle.MOD_ORDER], axis=-1)
    assert_close(f"mod[Dt={Dt}]", to_host64(mod), ref, 1e-5)


def test_lite_block_from_timestep_path():
    """Lite conditioning end to end: t -> timestep path -> 16-d tvec (f32) -> block with a
    16-wide modulation Linear, at full width on a small grid with ragged tiles."""
    tcfg = wl.TIMESTEP_LITE
    traw = wl.timestep_inputs(tcfg)
    cfg = wl.BlockConfig("block_lite_c3072_h24_f12288_dt16_grid2x6x10_cond40",
                         3072, 24, 128, 12288, 16, (2, 6, 10), 40, seed=24, batch=2)
    raw = wl.block_inputs(cfg)
    # The 16-d tvec of N(0, 0.02) timestep weights has rms ~0.1; a 2.0-std modulation Linear
    # brings shift / scale / gate to the ~0.7 rms the full model's 1536-d path gives, so
    # both branches weigh on the output.
    rng = np.random.default_rng(25)
    for s in ("vis", "cond"):
        raw[f"{s}.w_mod"] = wl.round_to_bf16_bits(rng.standard_normal((6 * 3072, 16)).astype(np.float32) * 2.0)
    t = {k: to_dev(v, wl.BF16) for k, v in raw.items()}
    ws = [to_dev(traw[k], wl.BF16) for k in wl.TIMESTEP_WEIGHTS]
    _, _, tvec = mm.timestep_embed(to_dev(traw["t"], wl.F32), *ws)
    dims = mm.BlockDims.make(cfg.width, cfg.heads, cfg.ffn, cfg.t_dim, act_dtype=torch.float16)
    rope = mm.Rope3D.make(cfg.grid)
    wv = {k: t[f"vis.{k}"] for k in wl.STREAM_WEIGHTS}
    wc = {k: t[f"cond.{k}"] for k in wl.STREAM_WEIGHTS}
    out_v, out_c, _ = mm.block_fwd(dims, wv, wc, t["x_vis"], t["x_cond"], tvec, rope)
    torch.cuda.synchronize()
    tref = oracle.timestep_path(traw["t"].astype(np.float64), *[wl.to_f64(traw[k], wl.BF16) for k in wl.TIMESTEP_WEIGHTS])
    f64 = lambda k: wl.to_f64(raw[k], wl.BF16)  # noqa: E731
    log("  oracle block")
    ref = oracle.block_forward(f64("x_vis"), f64("x_cond"), tref["tvec"],
                               {k: f64(f"vis.{k}") for k in wl.STREAM_WEIGHTS},
                               {k: f64(f"cond.{k}") for k in wl.STREAM_WEIGHTS}, cfg.grid, cfg.heads)
    mod_rms = float(np.sqrt(np.mean(ref["mod_vis"] ** 2)))
    log(f"  rms of the Lite modulation vectors: {mod_rms:.3f}")
    assert mod_rms > 0.3
    assert_close("out_vis", to_host64(out_v), ref["out_vis"], 2e-2)
    assert_close("out_cond", to_host64(out_c), ref["out_cond"], 2e-2)
