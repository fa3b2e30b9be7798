"""GPU parity of the 8-bit block (mmdit_block_fwd with E4M3 matrices, the Wan report's
inference setup of section 4.4.3) against the float64 oracle's 8-bit block (reading r28).

An 8-bit pipeline is ill-conditioned end to end: each quantizer is a step function, so two
correct implementations whose inputs differ by one f16 ulp -- which the FP8 MFMA's inexact
sums (~1e-4 of a GEMM result) produce in a fair share of elements -- round a few percent of
the next codes one step apart, and the next GEMM output then differs by about 1e-2 rms.  The
block is therefore checked stage by stage: after the call the workspace still holds every
stage's output (the attention's operand codes and scales, O, x1, h2, the GELU output g and
g's codes), and each stage is compared with the oracle's step applied to the GPU's own stored
input, at the kernel-level bars of the FP8 GEMM and 8-bit attention tests:
  codes of g (per-token E4M3) bit for bit;
  O against the 8-bit attention of the GPU's codes: rms(err beyond f16 storage) <= 2e-4 and
    every element within two E4M3 weight steps of its row (the 8-bit attention test's bound);
  x1 - x, out - x1 (gated FP8 GEMMs): max|err|/rms <= 1e-3 (the FP8 GEMM's 3e-4, times the
    gates' crest);
  h2, g (f16-stored LN-modulate and FP8 GEMM + GELU): error beyond f16 storage <= 1e-4 / 1e-3;
  the attention operands against the oracle's q^ / k^ / v from the GPU's inputs: every
    dequantized element within one quantization step (plus 2e-3 of its group's amax).
The end-to-end distance from the oracle's own 8-bit block is logged beside the method's
distance from the 16-bit definition, and must stay below it.
"""
import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_mmdit_amd as mm
import workloads as wl
from tests.test_gpu_attention8 import _unpermute_v
from tests.util import assert_close, assert_close_stored, half_ulp, log, parity_rows, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _setup(cfg):
    raw = wl.block_inputs(cfg)
    dev = {k: to_dev(v, wl.BF16) for k, v in raw.items()}
    w8 = {s: mm.fp8_block_weights({k: dev[f"{s}.{k}"] for k in wl.STREAM_WEIGHTS}) for s in ("vis", "cond")}
    host = {s: {k: wl.to_f64(raw[f"{s}.{k}"], wl.BF16) for k in wl.STREAM_WEIGHTS} for s in ("vis", "cond")}
    dims = mm.BlockDims.make(cfg.width, cfg.heads, cfg.ffn, cfg.t_dim, cfg.ln_eps, cfg.qk_eps,
                             act_dtype=torch.float16, matrix_dtype=torch.float8_e4m3fn)
    rope = mm.Rope3D.make(cfg.grid, cfg.rope_split, cfg.rope_base)
    out_v, out_c, ws = mm.block_fwd(dims, w8["vis"], w8["cond"], dev["x_vis"], dev["x_cond"] if cfg.n_cond else None,
                                    dev["tvec"], rope)
    torch.cuda.synchronize()
    return raw, w8, host, dims, {"vis": out_v, "cond": out_c}, ws


class _Ws:
    """Typed views of one stream's workspace regions."""

    def __init__(self, dims, cfg, ws, s):
        self.off = mm.block_workspace_offsets(dims, cfg.batch, cfg.n_vis, cfg.n_cond)[s]
        self.off0 = mm.block_workspace_offsets(dims, cfg.batch, cfg.n_vis, cfg.n_cond)[0]
        self.ws, self.B, self.C, self.F, self.H = ws, cfg.batch, cfg.width, cfg.ffn, cfg.heads
        self.n = cfg.n_vis if s == 0 else cfg.n_cond

    def get(self, region, dtype, shape, base=None):
        o = (self.off if base is None else base)[region]
        nbytes = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        return self.ws[o:o + nbytes].view(dtype).view(shape)


def _e4m3(t):
    return t.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _excess_rms_and_two_step(name, got, ref, sums, vhat_all):
    """O (stored f16) against the oracle's attention of the same codes."""
    rms_ref = float(np.sqrt(np.mean(ref ** 2)))
    exc = np.maximum(np.abs(got - ref) - half_ulp(ref, torch.float16), 0.0)
    rms = float(np.sqrt(np.mean(exc ** 2))) / rms_ref
    spread = np.maximum(vhat_all.max(axis=1)[:, None] - ref, ref - vhat_all.min(axis=1)[:, None])
    bound = 2 * 16.0 * spread / np.transpose(sums, (0, 2, 1))[..., None] + 2e-3 * rms_ref
    ratio = float((exc / bound).max())
    log(f"  {name}: rms(err beyond f16)/rms = {rms:.3e} (tol 2e-4); max err / two-step bound = {ratio:.3f}")
    assert np.all(np.isfinite(got)) and rms <= 2e-4 and ratio <= 1.0, name


def _stages(cfg, raw, w8, host, dims, outs, ws, rows=None):
    """Stage-by-stage checks (rows: per-stream sampled query rows, or None for all)."""
    B, C = cfg.batch, cfg.width
    sl = {s: (slice(None) if rows is None else rows[s]) for s in ("vis", "cond")}
    wv = _Ws(dims, cfg, ws, 0)
    # the attention operands of both streams, from the workspace
    codes = {}
    for s, si, n in (("vis", 0, cfg.n_vis), ("cond", 1, cfg.n_cond)):
        w = _Ws(dims, cfg, ws, si)
        nb = (n + 63) // 64
        codes[s] = dict(
            q8=w.get(mm.WS_Q8, torch.int8, (B, n, cfg.heads, 128)).cpu().numpy().astype(np.float64),
            sq=np.transpose(w.get(mm.WS_QS, torch.float32, (B, cfg.heads, n)).cpu().numpy(), (0, 2, 1)),
            k8=w.get(mm.WS_K8, torch.int8, (B, n, cfg.heads, 128)).cpu().numpy().astype(np.float64),
            sk=w.get(mm.WS_KS, torch.float32, (B, cfg.heads, nb)).cpu().numpy(),
            v8=_unpermute_v(_e4m3(w.get(mm.WS_V8T, torch.uint8, (B, cfg.heads, 128, nb * 64))), n))
    sv = wv.get(mm.WS_VS, torch.float32, (B, cfg.heads, 128), base=wv.off0).cpu().numpy()
    vr, cr = (None, None) if rows is None else (rows["vis"], rows["cond"])
    o_ref_v, o_ref_c, sums_v, sums_c = oracle.attention_8bit_from_codes(
        codes["vis"]["q8"], codes["vis"]["sq"], codes["vis"]["k8"], codes["vis"]["sk"],
        codes["cond"]["q8"], codes["cond"]["sq"], codes["cond"]["k8"], codes["cond"]["sk"],
        codes["vis"]["v8"], codes["cond"]["v8"], sv, vis_rows=vr, cond_rows=cr, return_row_sums=True)
    vhat = np.concatenate([codes["vis"]["v8"], codes["cond"]["v8"]], axis=1) * sv[:, None]
    for s, si, n, o_ref, sums in (("vis", 0, cfg.n_vis, o_ref_v, sums_v), ("cond", 1, cfg.n_cond, o_ref_c, sums_c)):
        if n == 0:
            continue
        w = _Ws(dims, cfg, ws, si)
        idx = None if rows is None else torch.from_numpy(rows[s]).cuda()
        pick = (lambda t: t) if idx is None else (lambda t: t[:, idx])  # noqa: E731
        mod = to_host64(w.get(mm.WS_MOD, torch.float32, (B, 6 * C)))
        m = {nm: mod[:, i * C:(i + 1) * C] for i, nm in enumerate(oracle.MOD_ORDER)}
        x = wl.to_f64(raw[f"x_{s}"], wl.BF16)[:, sl[s]]
        o = to_host64(pick(w.get(mm.WS_H, torch.float16, (B, n, C))))
        x1 = to_host64(pick(w.get(mm.WS_X1, torch.float32, (B, n, C))))
        h2 = to_host64(pick(w.get(mm.WS_QKV, torch.float16, (B, n, C))))
        g = to_host64(pick(w.get(mm.WS_G, torch.float16, (B, n, cfg.ffn))))
        gq = pick(w.get(mm.WS_XQ, torch.uint8, (B, n, cfg.ffn)))
        gs = pick(w.get(mm.WS_XS, torch.float32, (B, n)))
        out = to_host64(pick(outs[s]))
        hw = host[s]
        # S5: O against the attention of the GPU's codes (o_ref [B, rows, H, D])
        _excess_rms_and_two_step(f"O_{s}", o.reshape(o_ref.shape), o_ref, sums, vhat)
        # S6: x1 = x + gate_a (fp8 linear of the stored O)
        a_ref = m["gate_a"][:, None] * oracle.fp8_linear_prequantized(o, *oracle.fp8_weight(hw["w_o"]), hw["b_o"])
        assert_close(f"x1_{s} - x", x1 - x, a_ref, 1e-3)
        # S7: h2 = LN(x1) (1 + scale_f) + shift_f, stored f16
        h2_ref = oracle.modulate(oracle.layer_norm(x1, cfg.ln_eps), m["shift_f"], m["scale_f"])
        assert_close_stored(f"h2_{s}", h2, h2_ref, torch.float16, 1e-4)
        # S8: g = GELU(fp8 linear of the stored h2), stored f16
        g_ref = oracle.gelu(oracle.fp8_linear_prequantized(h2, *oracle.fp8_weight(hw["w_fc1"]), hw["b_fc1"]))
        assert_close_stored(f"g_{s}", g, g_ref, torch.float16, 1e-3)
        # S9 input: g's per-token codes and scales bit for bit
        qg, sg = oracle.quantize_fp8(g, per_row=True)
        assert np.array_equal(_e4m3(gq), qg), f"g_{s}: E4M3 codes differ"
        assert np.array_equal(gs.cpu().numpy(), sg), f"g_{s}: scales differ"
        # S9: out = x1 + gate_f (fp8 linear of the stored g)
        f_ref = m["gate_f"][:, None] * oracle.fp8_linear_prequantized(g, *oracle.fp8_weight(hw["w_fc2"]), hw["b_fc2"])
        assert_close(f"out_{s} - x1", out - x1, f_ref, 1e-3)
    return codes, sv


def _end_to_end(cfg, raw, host, outs, rows=None):
    """Logged: distance of the GPU's outputs from the oracle's own 8-bit block beside the
    method's distance from the 16-bit definition (a wrong formula misses by far more)."""
    args = (wl.to_f64(raw["x_vis"], wl.BF16), wl.to_f64(raw["x_cond"], wl.BF16), wl.to_f64(raw["tvec"], wl.BF16),
            host["vis"], host["cond"], cfg.grid, cfg.heads, cfg.ln_eps, cfg.qk_eps)
    kw = {} if rows is None else {"vis_rows": rows["vis"], "cond_rows": rows["cond"]}
    r8 = oracle.block_forward_8bit(*args, **kw)
    r16 = oracle.block_forward(*args, **kw)
    for s in ("vis", "cond"):
        got = to_host64(outs[s] if rows is None else outs[s][:, torch.from_numpy(rows[s]).cuda()])
        x = wl.to_f64(raw[f"x_{s}"], wl.BF16)[:, slice(None) if rows is None else rows[s]]
        d_gpu = np.sqrt(np.mean((got - r8[f"out_{s}"]) ** 2))
        d_method = np.sqrt(np.mean((r8[f"out_{s}"] - r16[f"out_{s}"]) ** 2))
        branch = np.sqrt(np.mean((r16[f"out_{s}"] - x) ** 2))
        log(f"  out_{s}: rms distance / rms(block branches): GPU to the 8-bit oracle {d_gpu / branch:.3e}, "
            f"8-bit oracle to the 16-bit definition {d_method / branch:.3e}")
        assert d_gpu < d_method, f"out_{s}: the GPU is farther from the 8-bit oracle than the method from exact"


def test_block8_weight_codes_bit_exact():
    cfg = wl.BLOCK_SMALL
    raw, w8, host, dims, outs, ws = _setup(cfg)
    for s in ("vis", "cond"):
        for k, sk in zip(mm.MATRIX_KEYS, mm.SCALE_KEYS):
            qw, sw = oracle.fp8_weight(host[s][k])
            assert np.array_equal(_e4m3(w8[s][k]), qw), f"{s}.{k}: E4M3 codes differ"
            assert w8[s][sk].item() == np.float32(sw), f"{s}.{sk}: scale differs"


@pytest.mark.parametrize("cfg", [wl.BLOCK_TINY, wl.BLOCK_SMALL], ids=["tiny", "small"])
def test_block8_stage_parity(cfg):
    log(f"8-bit block, stage by stage: {cfg.name}")
    raw, w8, host, dims, outs, ws = _setup(cfg)
    codes, sv = _stages(cfg, raw, w8, host, dims, outs, ws)
    # the attention operands against the oracle's q^ / k^ / v computed from the GPU's h
    B, C = cfg.batch, cfg.width
    for s, si, n in (("vis", 0, cfg.n_vis), ("cond", 1, cfg.n_cond)):
        w = _Ws(dims, cfg, ws, si)
        mod = to_host64(w.get(mm.WS_MOD, torch.float32, (B, 6 * C)))
        x = wl.to_f64(raw[f"x_{s}"], wl.BF16)
        h = oracle.f16_round(oracle.modulate(oracle.layer_norm(x, cfg.ln_eps), mod[:, :C], mod[:, C:2 * C]))
        qw, swt = oracle.fp8_weight(host[s]["w_qkv"])
        qkv = oracle.f16_round(oracle.fp8_linear_prequantized(h, qw, swt, host[s]["b_qkv"])).reshape(B, n, 3, cfg.heads, 128)
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
        q = oracle.rms_norm_heads(q, host[s]["q_norm"], cfg.qk_eps)
        k = oracle.rms_norm_heads(k, host[s]["k_norm"], cfg.qk_eps)
        if s == "vis":
            ang = oracle.rope_angles(cfg.grid, cfg.rope_split, cfg.rope_base)
            q, k = oracle.rope_rotate(q, ang), oracle.rope_rotate(k, ang)
        q, k = oracle.f16_round(q), oracle.f16_round(k)
        c = codes[s]
        skr = np.repeat(c["sk"], 64, axis=2)[:, :, :n].transpose(0, 2, 1)[..., None]     # [B, n, H, 1]
        for nm, deq, ref, step in (("q^", c["q8"] * c["sq"][..., None], q, c["sq"][..., None]),
                                   ("k^", c["k8"] * skr, k, skr)):
            amax = np.abs(ref).max(axis=-1, keepdims=True)
            ratio = np.abs(deq - ref) / (step * (0.5 + 1e-3) + 2e-3 * amax)
            log(f"  {nm}_{s} codes: max |dequantized - oracle| / (half step + 2e-3 amax) = {ratio.max():.3f}; "
                f"codes differing from the oracle's own: {np.mean(deq != np.round(ref / step) * step):.2%}")
            assert ratio.max() <= 2.0, f"{nm}_{s}: a code is more than one step from the oracle's value"
        vd = c["v8"] * sv[:, None]
        vstep = np.maximum(np.abs(v) * 2.0 ** -3, 2.0 ** -9 * sv[:, None])
        ratio = np.abs(vd - v) / (vstep + 2e-3 * np.abs(v).max(axis=1, keepdims=True))
        log(f"  v_{s} codes: max |dequantized - oracle| / (E4M3 step + 2e-3 amax) = {ratio.max():.3f}")
        assert ratio.max() <= 1.0, f"v_{s}: a code is more than one E4M3 step from the oracle's value"
    _end_to_end(cfg, raw, host, outs)


def test_block8_480p_sampled_stage_parity():
    """480p in the launch configuration the bench times: 256 visual rows (first and last 32,
    rows of the last 1536, seeded ones) and 64 conditioning rows, every key."""
    cfg = wl.BLOCK_480P
    raw, w8, host, dims, outs, ws = _setup(cfg)
    rows = {"vis": parity_rows(cfg.n_vis, 256, 81, bands=((cfg.n_vis - 1536, cfg.n_vis, 24),)),
            "cond": parity_rows(cfg.n_cond, 64, 82)}
    log(f"8-bit 480p block: {rows['vis'].size} visual + {rows['cond'].size} conditioning rows")
    _stages(cfg, raw, w8, host, dims, outs, ws, rows)


def test_block8_rejects_missing_scales_and_wrong_act():
    cfg = wl.BLOCK_TINY
    raw = wl.block_inputs(cfg)
    dev = {k: to_dev(v, wl.BF16) for k, v in raw.items()}
    w8 = {s: mm.fp8_block_weights({k: dev[f"{s}.{k}"] for k in wl.STREAM_WEIGHTS}) for s in ("vis", "cond")}
    dims = mm.BlockDims.make(cfg.width, cfg.heads, cfg.ffn, cfg.t_dim, act_dtype=torch.float16,
                             matrix_dtype=torch.float8_e4m3fn)
    rope = mm.Rope3D.make(cfg.grid, cfg.rope_split, cfg.rope_base)
    bad = dict(w8["vis"])
    bad.pop("s_o")
    with pytest.raises(mm.MmditError, match="s_o"):
        mm.block_fwd(dims, bad, w8["cond"], dev["x_vis"], dev["x_cond"], dev["tvec"], rope)
    d16 = mm.BlockDims.make(cfg.width, cfg.heads, cfg.ffn, cfg.t_dim, act_dtype=torch.bfloat16,
                            matrix_dtype=torch.float8_e4m3fn)
    assert mm.block_workspace_bytes(d16, 1, cfg.n_vis, cfg.n_cond) == 0
