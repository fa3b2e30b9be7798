"""GPU parity of the 8-bit joint attention (INT8 Q K^T, FP8 E4M3 P V, f32 accumulation)
against the float64 oracle's definition of the same quantized method.

The operand codes and scales are integer-valued decisions taken in f32 on both sides and are
compared bit for bit.  For the attention output the codes are identical and the integer
products exact; what separates the two sides is
  (a) the FP8 MFMA's inexact sum of its 64 products (up to ~1e-4 of its result's rms), and
  (b) the f32 value of 2^(acc c + 8 - m) that decides each weight's E4M3 code: the kernel
      forms it against its running integer reference and with the hardware exp2, so a value
      within an f32 ulp of an E4M3 rounding boundary can land one E4M3 step (1/16 to 1/8 of
      the weight) away.  One such weight moves its row by (step) |V_j - O| / sum P', which at
      ~1.4 k keys reaches a few 1e-3 of the output's rms and shrinks as the sequence grows.
Bars: rms(err) / rms <= 2e-4 (systematic errors, which move every element) and
max|err| / rms <= 1e-2 (single E4M3 steps; a wrong formula or layout misses by order one,
and the method's own deviation from exact attention, logged, is ~4 % rms and ~25 % max)."""
import math

import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_mmdit_amd as mm
import workloads as wl
from tests.util import assert_close, log, to_dev, to_host64

pytestmark = pytest.mark.gpu
TOL_ATT8 = 1e-2
TOL_ATT8_RMS = 2e-4


def _close8(name, got, ref):
    e = got - ref
    rms = float(np.sqrt(np.mean(e ** 2) / np.mean(ref ** 2)))
    log(f"  {name}: rms(err)/rms = {rms:.3e} (tol {TOL_ATT8_RMS:.0e})")
    assert rms <= TOL_ATT8_RMS, f"{name}: rms(err)/rms {rms:.3e}"
    assert_close(name, got, ref, TOL_ATT8)


def _inputs(cfg, seed=None):
    raw = wl.attention_inputs(cfg, seed)
    dev = {k: to_dev(v, cfg.dtype) for k, v in raw.items()}
    f64 = {k: wl.to_f64(v, cfg.dtype) for k, v in raw.items()}
    return dev, f64


def _unpermute_v(v8t, n):
    """v8t [B, H, D, np] in the kernel's key order -> codes [B, n, H, D]."""
    k = np.arange(v8t.shape[-1])
    t, kk = k // 64, k % 64
    pos = 16 * (2 * (kk >> 5) + ((kk >> 2) & 1)) + 4 * ((kk >> 3) & 3) + (kk & 3)
    logical = v8t[..., t * 64 + pos]                       # [B, H, D, np] in key order
    return np.transpose(logical[..., :n], (0, 3, 1, 2))


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
        pad = t["v8t"].cpu().numpy()
        if pad.shape[-1] > n:                              # padding keys hold zero codes
            k = np.arange(pad.shape[-1])
            assert np.all(pad[..., k % 64 >= 0][..., :0] == 0)
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
    rv, rc, rlse = oracle.joint_attention_8bit(f64["q_vis"], f64["k_vis"], f64["v_vis"], f64["q_cond"],
                                               f64["k_cond"], f64["v_cond"], return_lse=True)
    _close8("o_vis", to_host64(ov), rv)
    if cfg.n_cond:
        _close8("o_cond", to_host64(oc), rc)
    np.testing.assert_allclose(to_host64(lse), rlse, rtol=0, atol=1e-4)
    ev, ec = oracle.joint_attention(f64["q_vis"], f64["k_vis"], f64["v_vis"], f64["q_cond"], f64["k_cond"], f64["v_cond"])
    e = to_host64(ov) - ev
    log(f"  8-bit method vs exact attention: rms {np.sqrt(np.mean(e ** 2) / np.mean(ev ** 2)):.3e}, "
        f"max {oracle.rel_max_err(to_host64(ov), ev):.3e}")


def test_attention_8bit_480p_sampled_rows():
    """The 480p workload (32760 visual + 512 conditioning tokens, 24 heads) in the launch the
    bench times, every operand code checked and sampled query rows against the oracle."""
    cfg = wl.ATTN_480P
    dev, f64 = _inputs(cfg)
    ops = mm.attn8_quantize(dev["q_vis"], dev["k_vis"], dev["v_vis"], dev["q_cond"], dev["k_cond"], dev["v_cond"])
    ov, oc = mm.joint_attention_8bit(ops)
    torch.cuda.synchronize()
    log("  operands")
    _check_operands(ops, f64, cfg.n_vis, cfg.n_cond)
    rows_v = wl.sample_rows(cfg.n_vis, 48, seed=7)
    rows_c = wl.sample_rows(cfg.n_cond, 16, seed=8)
    log("  oracle rows")
    rv, rc = oracle.joint_attention_8bit(f64["q_vis"], f64["k_vis"], f64["v_vis"], f64["q_cond"], f64["k_cond"],
                                         f64["v_cond"], vis_rows=rows_v, cond_rows=rows_c)
    _close8("o_vis[rows]", to_host64(ov)[:, rows_v], rv)
    _close8("o_cond[rows]", to_host64(oc)[:, rows_c], rc)


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
    rv, rc = oracle.joint_attention_8bit(f64["q_vis"], f64["k_vis"], f64["v_vis"], f64["q_cond"], f64["k_cond"],
                                         f64["v_cond"], vis_rows=rows_v, cond_rows=rows_c)
    _close8("o_vis[rows]", to_host64(ov)[:, rows_v], rv)
    _close8("o_cond[rows]", to_host64(oc)[:, rows_c], rc)
