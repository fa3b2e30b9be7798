"""GPU parity of the 8-bit joint attention (INT8 Q K^T, FP8 E4M3 P V, f32 accumulation)
against the float64 oracle's definition of the same quantized method.

The operand codes and scales (the quantization rule, an f32 product rounded) are compared bit
for bit.  For the attention output the codes are identical and the integer products exact;
the oracle then evaluates the logits, the integer reference, the weights 2^(y + 8 - M) and
their E4M3 rounding in float64.  What separates the kernel from it is
  (a) the FP8 MFMA's inexact sum of its 64 products (up to ~1e-4 of its result's rms), and
  (b) the kernel's f32 logits (its factor s_q s_k scale log2(e) and the product with the
      integer dot product are rounded to f32, and exp2 is the hardware's): a weight whose exact
      value lies within a few f32 ulps of an E4M3 rounding boundary can land one E4M3 step
      (1/16 to 1/8 of the weight) away, and a row maximum within an f32 ulp of an integer can
      move the reference M by one, which rescales every weight of the row by 2 exactly and
      changes only weights in E4M3's subnormal range (below 2^-6 of the 2^8 ceiling).  One
      stepped weight moves its row by (step) |V_j - O| / sum P', a few 1e-3 of the output's
      rms at ~1.4 k keys, less as the sequence grows.
Bars (kernel against the float64 definition):
  rms(err) / rms <= 2e-4 -- systematic errors move every element;
  per element |err| <= 2 * 16 * max_j |V^_j - O_i| / sum_j P'_ij + 2e-3 rms -- two weights of
  row i moved by one E4M3 step each: P' <= 256 and the widest E4M3 step below 256 is 16, and a
  step of weight j moves O_i by step * (V^_j - O_i) / sum P' (V^ the dequantized values, the
  row sums from the oracle); 2e-3 rms covers the FP8 MFMA's inexact sums.  The expected number
  of boundary-straddling weights per row is far below one (f32 logits are within ~1e-6 relative
  of the exact ones, and E4M3 boundaries are 1/16 apart), so a wrong formula or layout, which
  misses by order one in most rows, cannot pass.  Kernel-against-kernel comparisons (split tail
  against one pass) keep flat bars: rms 2e-4 and max 1e-2 of the rms.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_mmdit_amd as mm
import workloads as wl
from tests.util import assert_close, log, parity_rows, to_dev, to_host64

pytestmark = pytest.mark.gpu
TOL_ATT8 = 1e-2
TOL_ATT8_RMS = 2e-4


def _close8(name, got, ref):
    """Kernel against kernel: flat bars."""
    e = got - ref
    rms = float(np.sqrt(np.mean(e ** 2) / np.mean(ref ** 2)))
    log(f"  {name}: rms(err)/rms = {rms:.3e} (tol {TOL_ATT8_RMS:.0e})")
    assert rms <= TOL_ATT8_RMS, f"{name}: rms(err)/rms {rms:.3e}"
    assert_close(name, got, ref, TOL_ATT8)


def _close8_oracle(name, got, ref, sums, vhat_all):
    """Kernel against the float64 oracle: the rms bar, then each element within two E4M3 steps
    of its row's weights (see the module docstring).  got / ref [B, rows, H, D]; sums [B, H, rows]
    the oracle's row sums of P'; vhat_all [B, N, H, D] the dequantized V of every key."""
    e = got - ref
    rms_ref = float(np.sqrt(np.mean(ref ** 2)))
    rms = float(np.sqrt(np.mean(e ** 2))) / rms_ref
    log(f"  {name}: rms(err)/rms = {rms:.3e} (tol {TOL_ATT8_RMS:.0e}); max|err|/rms = {np.max(np.abs(e)) / rms_ref:.3e}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert rms <= TOL_ATT8_RMS, f"{name}: rms(err)/rms {rms:.3e}"
    vmax = vhat_all.max(axis=1)[:, None]                    # [B, 1, H, D]
    vmin = vhat_all.min(axis=1)[:, None]
    spread = np.maximum(vmax - ref, ref - vmin)             # max_j |V^_j - O_i| per element
    denom = np.transpose(sums, (0, 2, 1))[..., None]        # [B, rows, H, 1]
    bound = 2 * 16.0 * spread / denom + 2e-3 * rms_ref
    ratio = np.abs(e) / bound
    log(f"  {name}: max |err| / (two-step bound) = {ratio.max():.3f}; "
        f"median bound / rms = {np.median(bound) / rms_ref:.3e}")
    assert ratio.max() <= 1.0, f"{name}: an element exceeds two E4M3 steps of its row ({ratio.max():.3f})"


def _lse8_close(got, ref, sums_v, sums_c):
    """lse [B, H, n_cond + n_vis] against the oracle's: a weight one E4M3 step away moves a
    row's natural-log lse by step / sum(P'), so each row may move by two of the widest steps
    (16) over its row sum, plus f32 rounding of the log."""
    sums = np.concatenate([sums_c, sums_v], axis=-1)
    bound = 2 * 16.0 / sums + 1e-5 * np.maximum(1.0, np.abs(ref))
    ratio = np.abs(got - ref) / bound
    log(f"  lse: max|err| = {np.max(np.abs(got - ref)):.3e}; max |err| / (two-step bound) = {ratio.max():.3f}")
    assert np.all(np.isfinite(got)), "lse: non-finite values"
    assert ratio.max() <= 1.0, f"lse: a row exceeds two E4M3 steps of its sum ({ratio.max():.3f})"


def _vhat(f64):
    v8v, v8c, sv = oracle.attn8_quantize_v(f64["v_vis"], f64["v_cond"])
    return np.concatenate([v8v, v8c], axis=1) * sv[:, None]


def _inputs(cfg, seed=None):
    raw = wl.attention_inputs(cfg, seed)
    dev = {k: to_dev(v, cfg.dtype) for k, v in raw.items()}
    f64 = {k: wl.to_f64(v, cfg.dtype) for k, v in raw.items()}
    return dev, f64


def _logical_v(v8t):
    """v8t [B, H, D, np] in the kernel's key order -> [B, H, D, np] in key order."""
    k = np.arange(v8t.shape[-1])
    t, kk = k // 64, k % 64
    pos = 16 * (2 * (kk >> 5) + ((kk >> 2) & 1)) + 4 * ((kk >> 3) & 3) + (kk & 3)
    return v8t[..., t * 64 + pos]


def _unpermute_v(v8t, n):
    """v8t [B, H, D, np] in the kernel's key order -> codes [B, n, H, D]."""
    return np.transpose(_logical_v(v8t)[..., :n], (0, 3, 1, 2))


def _check_operands(ops, f64, n_vis, n_cond):
    qv8, sqv, kv8, skv = oracle.attn8_quantize_stream(f64["q_vis"], f64["k_vis"])
    v8v, v8c, sv = oracle.attn8_quantize_v(f64["v_vis"], f64["v_cond"])
    parts = [(0, n_vis, qv8, sqv, kv8, skv, v8v)]
    if n_cond:
        qc8, sqc, kc8, skc = oracle.attn8_quantize_stream(f64["q_cond"], f64["k_cond"])
        parts.append((1, n_cond, qc8, sqc, kc8, skc, v8c))
    for s, n, q8, sq, k8, sk, v8 in parts:
        t = ops.t[s]
        np.testing.assert_array_equal(t["q8"].cpu().numpy().astype(np.float64), q8)
        np.testing.assert_array_equal(t["q_scale"].cpu().numpy(), np.transpose(sq, (0, 2, 1)))
        np.testing.assert_array_equal(t["k8"].cpu().numpy().astype(np.float64), k8)
        np.testing.assert_array_equal(t["k_scale"].cpu().numpy(), sk)
        got_v = _unpermute_v(t["v8t"].cpu().numpy(), n)
        np.testing.assert_array_equal(got_v, oracle.fp8_e4m3_code(v8))
        # keys past n in the last 64-key block are multiplied by P' = 0 in the FP8 MFMA: their
        # codes must be +0 (a NaN code would poison the whole row)
        tail = _logical_v(t["v8t"].cpu().numpy())[..., n:]
        assert tail.shape[-1] == (-n) % 64
        assert np.all(tail == 0), "padding keys must hold zero codes"
    np.testing.assert_array_equal(ops.v_scale.cpu().numpy(), sv)


@pytest.mark.parametrize("cfg", [
    wl.AttnConfig("a8_bf16_2x128_grid2x7x7_cond9", wl.BF16, 2, 128, (2, 7, 7), 9, seed=41),
    wl.AttnConfig("a8_bf16_3x128_grid1x8x8_cond0", wl.BF16, 3, 128, (1, 8, 8), 0, seed=42),
    wl.AttnConfig("a8_bf16_2x128_grid1x1x1_cond1_b2", wl.BF16, 2, 128, (1, 1, 1), 1, seed=43, batch=2),
    wl.ATTN_LAYER,
], ids=lambda c: c.name)
def test_attention_8bit_matches_oracle(cfg):
    dev, f64 = _inputs(cfg)
    log(f"  {cfg.name}: quantize + attention")
    ops = mm.attn8_quantize(dev["q_vis"], dev["k_vis"], dev["v_vis"],
                            dev["q_cond"] if cfg.n_cond else None, dev["k_cond"] if cfg.n_cond else None,
                            dev["v_cond"] if cfg.n_cond else None)
    ov, oc, lse = mm.joint_attention_8bit(ops, return_lse=True)
    torch.cuda.synchronize()
    _check_operands(ops, f64, cfg.n_vis, cfg.n_cond)
    log("  operand codes and scales bit-exact")
    rv, rc, rlse, sv_, sc_ = oracle.joint_attention_8bit(f64["q_vis"], f64["k_vis"], f64["v_vis"], f64["q_cond"],
                                                         f64["k_cond"], f64["v_cond"], return_lse=True,
                                                         return_row_sums=True)
    vh = _vhat(f64)
    _close8_oracle("o_vis", to_host64(ov), rv, sv_, vh)
    if cfg.n_cond:
        _close8_oracle("o_cond", to_host64(oc), rc, sc_, vh)
    _lse8_close(to_host64(lse), rlse, sv_, sc_)
    ev, ec = oracle.joint_attention(f64["q_vis"], f64["k_vis"], f64["v_vis"], f64["q_cond"], f64["k_cond"], f64["v_cond"])
    e = to_host64(ov) - ev
    log(f"  8-bit method vs exact attention: rms {np.sqrt(np.mean(e ** 2) / np.mean(ev ** 2)):.3e}, "
        f"max {oracle.rel_max_err(to_host64(ov), ev):.3e}")


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,n_rows_v,n_rows_c", [(wl.ATTN_480P, 192, 64), (wl.ATTN_720P, 96, 32)],
                         ids=lambda v: getattr(v, "name", str(v)))
def test_attention_8bit_full_size_sampled_rows(cfg, n_rows_v, n_rows_c):
    """The 480p and 720p workloads (32760 / 75600 visual + 512 conditioning tokens, 24 heads)
    in the launch the bench times (with the split-tail workspace): every operand code checked,
    and sampled query rows (the first and last 32, a band over the last query tiles, seeded
    random rows) of every head against the oracle."""
    dev, f64 = _inputs(cfg)
    ops = mm.attn8_quantize(dev["q_vis"], dev["k_vis"], dev["v_vis"], dev["q_cond"], dev["k_cond"], dev["v_cond"])
    ws = torch.empty(mm.ATTN8_SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    ov, oc = mm.joint_attention_8bit(ops, workspace=ws)
    torch.cuda.synchronize()
    log("  operands")
    _check_operands(ops, f64, cfg.n_vis, cfg.n_cond)
    rows_v = parity_rows(cfg.n_vis, n_rows_v, seed=7, bands=[(cfg.n_vis - 1536, cfg.n_vis, 97)])
    rows_c = parity_rows(cfg.n_cond, n_rows_c, seed=8)
    got_v, got_c = to_host64(ov)[:, rows_v], to_host64(oc)[:, rows_c]
    del dev, ops, ov, oc, ws
    torch.cuda.empty_cache()
    log(f"  oracle rows: {rows_v.size} visual, {rows_c.size} conditioning")
    rv, rc, sv_, sc_ = oracle.joint_attention_8bit(f64["q_vis"], f64["k_vis"], f64["v_vis"], f64["q_cond"],
                                                   f64["k_cond"], f64["v_cond"], vis_rows=rows_v, cond_rows=rows_c,
                                                   return_row_sums=True)
    vh = _vhat(f64)
    _close8_oracle("o_vis[rows]", got_v, rv, sv_, vh)
    _close8_oracle("o_cond[rows]", got_c, rc, sc_, vh)


def test_attention_8bit_zero_keys_give_mean_of_values():
    """K = 0: every weight is 2^8, so every output row is the mean of the dequantized V."""
    cfg = wl.AttnConfig("a8_zero_k", wl.BF16, 2, 128, (2, 5, 9), 20, seed=44)
    dev, f64 = _inputs(cfg)
    ops = mm.attn8_quantize(dev["q_vis"], 0 * dev["k_vis"], dev["v_vis"], dev["q_cond"], 0 * dev["k_cond"], dev["v_cond"])
    ov, oc = mm.joint_attention_8bit(ops)
    torch.cuda.synchronize()
    v8v, v8c, sv = oracle.attn8_quantize_v(f64["v_vis"], f64["v_cond"])
    mean = np.concatenate([v8v, v8c], axis=1).mean(axis=1) * sv
    assert_close("o_vis", to_host64(ov), np.broadcast_to(mean[:, None], ov.shape), 1e-4)
    assert_close("o_cond", to_host64(oc), np.broadcast_to(mean[:, None], oc.shape), 1e-4)


def test_attention_8bit_split_tail_with_workspace():
    """Batch 2, 24 heads, 1400 + 77 tokens: 288 (batch x head, query tile) items leave 32 for
    the last round, which a workspace lets the kernel cut into 8 key ranges each and merge.
    Each range takes its own integer reference, so a weight's E4M3 code is the same as in one
    pass up to the format's range at the bottom; the output is held to the same bars against
    the oracle, and against the same call without a workspace (one pass per item)."""
    cfg = wl.AttnConfig("a8_split_b2_h24_grid2x20x35_cond77", wl.BF16, 24, 128, (2, 20, 35), 77, seed=45, batch=2)
    dev, f64 = _inputs(cfg)
    ops = mm.attn8_quantize(dev["q_vis"], dev["k_vis"], dev["v_vis"], dev["q_cond"], dev["k_cond"], dev["v_cond"])
    ws = torch.empty(mm.ATTN8_SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    ov, oc = mm.joint_attention_8bit(ops, workspace=ws)
    uv, uc = mm.joint_attention_8bit(ops)
    torch.cuda.synchronize()
    _close8("o_vis split vs one pass", to_host64(ov), to_host64(uv))
    _close8("o_cond split vs one pass", to_host64(oc), to_host64(uc))
    rows_v = np.unique(np.concatenate([wl.sample_rows(cfg.n_vis, 24, seed=9), np.arange(400, cfg.n_vis, 37)]))
    rows_c = np.arange(cfg.n_cond)
    log("  oracle rows")
    rv, rc, sv_, sc_ = oracle.joint_attention_8bit(f64["q_vis"], f64["k_vis"], f64["v_vis"], f64["q_cond"],
                                                   f64["k_cond"], f64["v_cond"], vis_rows=rows_v, cond_rows=rows_c,
                                                   return_row_sums=True)
    vh = _vhat(f64)
    _close8_oracle("o_vis[rows]", to_host64(ov)[:, rows_v], rv, sv_, vh)
    _close8_oracle("o_cond[rows]", to_host64(oc)[:, rows_c], rc, sc_, vh)
