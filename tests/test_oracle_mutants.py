"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins catch each.

Every mutant below is a one-line slip someone could make while writing the oracle: a
dropped term, a wrong sign, a swapped axis or index, a transposed operand.  The pin suite
in ``test_oracle_pins.py`` must fail for every one of them.
"""
import inspect
import math

import numpy as np
import pytest

import oracle
import oracle.mmdit_oracle as om
from tests import test_oracle_pins as pins

ORIG = {name: getattr(om, name) for name in
        ("rope_angles", "rope_rotate", "token_positions", "rms_norm_heads", "softmax_attention",
         "modulate", "layer_norm", "linear", "gelu", "modulation", "joint_attention",
         "timestep_sinusoid", "silu", "timestep_path", "lite_merge_gather", "lite_unpatchify",
         "fp8_e4m3_round", "quantize_fp8", "fp8_linear", "quant_scale",
         "attn8_quantize_stream", "attn8_quantize_v", "quantize_int8", "joint_attention_8bit",
         "f16_round", "fp8_weight", "fp8_linear_prequantized")}


def _rope_sign(x, angles):
    out = ORIG["rope_rotate"](x, -angles)
    return out


def _band_order(grid, split=(16, 56, 56), base=10000.0):
    a = ORIG["rope_angles"](grid, split, base)
    return np.concatenate([a[:, 8:36], a[:, :8], a[:, 36:]], axis=1)


def _positions_hw_swapped(grid):
    p = ORIG["token_positions"](grid)
    return p[:, [0, 2, 1]]


def _ladder_full_width(grid, split=(16, 56, 56), base=10000.0):
    pos = ORIG["token_positions"](grid).astype(np.float64)
    cols = []
    for axis, d_a in enumerate(split):
        j = np.arange(d_a // 2)
        cols.append(pos[:, axis:axis + 1] * (base ** (-2.0 * j / 128))[None, :])
    return np.concatenate(cols, axis=1)


def _rope_half_split(x, angles):
    d = x.shape[-1]
    x0, x1 = x[..., :d // 2], x[..., d // 2:]
    c = np.cos(angles)[None, :, None, :]
    s = np.sin(angles)[None, :, None, :]
    return np.concatenate([x0 * c - x1 * s, x0 * s + x1 * c], axis=-1)


def _rms_no_eps(x, g, eps):
    return ORIG["rms_norm_heads"](x, g, 0.0)


def _rms_sum(x, g, eps):
    return ORIG["rms_norm_heads"](x, g, eps) / math.sqrt(x.shape[-1])


def _attn_scale_d(q, k, v, scale):
    return ORIG["softmax_attention"](q, k, v, scale * scale)


def _attn_axis(q, k, v, scale):
    s = (q @ k.T) * scale
    p = np.exp(s - s.max())
    p /= p.sum(axis=0, keepdims=True)
    return p @ v


def _mod_no_shift(xn, shift, scale):
    return ORIG["modulate"](xn, 0.0 * shift, scale)


def _mod_plain_scale(xn, shift, scale):
    return xn * scale[:, None, :] + shift[:, None, :]


def _ln_unbiased(x, eps):
    mu = x.mean(axis=-1, keepdims=True)
    var = x.var(axis=-1, ddof=1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def _linear_transposed(x, w, b):
    if w.shape[0] == w.shape[1]:
        w = w.T
    return ORIG["linear"](x, w, b)


def _linear_no_bias(x, w, b):
    return ORIG["linear"](x, w, None)


def _gelu_tanh(x):
    return 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))


def _modulation_swapped(w, b, t):
    m = ORIG["modulation"](w, b, t)
    m["gate_a"], m["gate_f"] = m["gate_f"], m["gate_a"]
    return m


def _modulation_order(w, b, t):
    m = ORIG["modulation"](w, b, t)
    m["shift_a"], m["scale_a"] = m["scale_a"], m["shift_a"]
    return m


def _joint_drop_cond_keys(q_vis, k_vis, v_vis, q_cond, k_cond, v_cond, **kw):
    e = k_cond[:, :0]
    return ORIG["joint_attention"](q_vis, k_vis, v_vis, q_cond, e, v_cond[:, :0], **kw)


def _sinusoid_sin_first(t, dim=256, max_period=10000.0):
    e = ORIG["timestep_sinusoid"](t, dim, max_period)
    return np.concatenate([e[:, dim // 2:], e[:, :dim // 2]], axis=1)


def _sinusoid_half_minus_one(t, dim=256, max_period=10000.0):
    half = dim // 2
    ang = np.asarray(t, dtype=np.float64)[:, None] * max_period ** (-np.arange(half) / (half - 1))[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def _silu_sigmoid_only(x):
    return ORIG["silu"](x) / np.where(x == 0, 1.0, x) * (x != 0)


def _timestep_no_inner_silu(t, w1, b1, w2, b2, w3, b3, dim=256, max_period=10000.0):
    e = om.timestep_sinusoid(t, dim, max_period)
    hidden = om.linear(e, w1, b1)
    temb = om.linear(hidden, w2, b2)
    return {"hidden": hidden, "temb": temb, "tvec": om.linear(om.silu(temb), w3, b3)}


def _timestep_no_outer_silu(t, w1, b1, w2, b2, w3, b3, dim=256, max_period=10000.0):
    r = ORIG["timestep_path"](t, w1, b1, w2, b2, w3, b3, dim, max_period)
    r["tvec"] = om.linear(r["temb"], w3, b3)
    return r


def _merge_column_major(x, grid):
    t_n, h_n, w_n = grid
    b, n, c = x.shape
    x5 = x.reshape(b, t_n, h_n, w_n, c)
    parts = [x5[:, :, dh::2, dw::2, :] for dw in (0, 1) for dh in (0, 1)]
    return np.concatenate(parts, axis=-1).reshape(b, -1, 4 * c)


def _merge_channel_interleaved(x, grid):
    g = ORIG["lite_merge_gather"](x, grid)
    b, m, c4 = g.shape
    return g.reshape(b, m, 4, c4 // 4).transpose(0, 1, 3, 2).reshape(b, m, c4)


def _unpatchify_swapped_w(y, w, b, grid):
    out = ORIG["lite_unpatchify"](y, w, b, grid)
    t_n, h_n, w_n = grid
    o5 = out.reshape(out.shape[0], t_n, h_n, w_n, -1)
    o5 = o5.reshape(out.shape[0], t_n, h_n, w_n // 2, 2, -1)[:, :, :, :, ::-1, :]
    return o5.reshape(out.shape)


def _fp8_truncate(x):
    x = np.asarray(x, dtype=np.float64)
    r = ORIG["fp8_e4m3_round"](x)
    return np.where(np.abs(r) > np.abs(x), ORIG["fp8_e4m3_round"](x - np.sign(x) * np.abs(x) * 2.0 ** -4), r)


def _fp8_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    r = ORIG["fp8_e4m3_round"](x)
    up = ORIG["fp8_e4m3_round"](x * (1 + 2.0 ** -30))
    return np.where(up != r, up, r)


def _scale_int8_max(amax, qmax):
    return ORIG["quant_scale"](amax, 127.0)


def _fp8_linear_no_wscale(x, w, b):
    qx, sx = om.quantize_fp8(x, per_row=True)
    qw, _ = om.quantize_fp8(w, per_row=False)
    y = (qx @ qw.T) * sx.astype(np.float64)[:, None]
    return y if b is None else y + b


def _fp8_linear_per_tensor_x(x, w, b):
    qx, sx = om.quantize_fp8(x, per_row=False)
    qw, sw = om.quantize_fp8(w, per_row=False)
    y = (qx @ qw.T) * float(sx[0]) * float(sw[0])
    return y if b is None else y + b


def _att8_k_per_token(q, k):
    q8, sq, _, _ = ORIG["attn8_quantize_stream"](q, k)
    k8, skt = om.quantize_int8(k, axes=3)                 # per token, not per 64-key block
    b, n, h, _ = k.shape
    # keep the interface: one scale per block, taken from the block's first token
    nb = -(-n // 64)
    sk = np.stack([skt[:, min(j * 64, n - 1), :, 0] for j in range(nb)], axis=2)
    return q8, sq, k8, sk


def _att8_v_per_tensor(v_vis, v_cond):
    n_vis = v_vis.shape[1]
    v_all = np.concatenate([v_vis, v_cond], axis=1)
    v8, sv = om.quantize_fp8_groups(v_all, axes=(1, 3))
    return v8[:, :n_vis], v8[:, n_vis:], np.broadcast_to(sv[:, 0], (v_all.shape[0],) + v_all.shape[2:]).copy()


def _int8_truncate(x, axes):
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=axes, keepdims=True)
    s = om.quant_scale(amax, 127.0)
    y = (x32 * (np.float32(1.0) / s).astype(np.float32)).astype(np.float32)
    return np.clip(np.trunc(y), -127, 127).astype(np.float64), s


def _att8_variant(floor=False, shift=8.0, exact_sum=False):
    def f(q_vis, k_vis, v_vis, q_cond, k_cond, v_cond, scale=None, vis_rows=None, cond_rows=None,
          chunk=1024, return_lse=False):
        b, _, h, d = q_vis.shape
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        kc = float(scale) * om.LOG2E
        qa, sqa, ka, ska = om.attn8_quantize_stream(q_vis, k_vis)
        qc, sqc, kcd, skc = om.attn8_quantize_stream(q_cond, k_cond)
        v8v, v8c, sv = om.attn8_quantize_v(v_vis, v_cond)
        k8 = np.concatenate([ka, kcd], axis=1)
        v8 = np.concatenate([v8v, v8c], axis=1)
        blk = lambda s_, n: np.repeat(s_, 64, axis=2)[:, :, :n]  # noqa: E731
        skcj = np.concatenate([blk(ska, k_vis.shape[1]), blk(skc, k_cond.shape[1])], axis=2).astype(np.float64) * kc

        def run(q8, sq, rows):
            if rows is not None:
                q8, sq = q8[:, rows], sq[:, rows]
            out = np.empty(q8.shape)
            for bi in range(b):
                for hi in range(h):
                    acc = q8[bi, :, hi, :] @ k8[bi, :, hi, :].T
                    c = sq[bi, :, hi].astype(np.float64)[:, None] * skcj[bi, hi][None, :]
                    y = acc * c
                    m = (np.floor if floor else np.ceil)(y.max(axis=1, keepdims=True))
                    pe = np.exp2(y + (shift - m))
                    p = om.fp8_e4m3_round(pe)
                    ell = (pe if exact_sum else p).sum(axis=1, keepdims=True)
                    out[bi, :, hi, :] = (p @ v8[bi, :, hi, :]) * sv[bi, hi][None, :] / ell
            return out
        return run(qa, sqa, vis_rows), run(qc, sqc, cond_rows)
    return f


def _f16_not_rounded(x):
    return np.asarray(x, dtype=np.float64)


def _fp8_weight_per_row(w):
    qw, sw = om.quantize_fp8(w, per_row=True)
    return qw * sw.astype(np.float64)[:, None], 1.0


def _fp8_linear_requantize_slices(x, qw, sw, b):
    # the weight slice handed in gets its own per-tensor scale (W_qkv's q, k, v separately)
    return ORIG["fp8_linear_prequantized"](x, *ORIG["fp8_weight"](qw * sw), b)


MUTANTS = {
    "rope_sign": ("rope_rotate", _rope_sign),
    "rope_band_order": ("rope_angles", _band_order),
    "positions_hw_swapped": ("token_positions", _positions_hw_swapped),
    "rope_ladder_full_width": ("rope_angles", _ladder_full_width),
    "rope_half_split_pairs": ("rope_rotate", _rope_half_split),
    "rmsnorm_no_eps": ("rms_norm_heads", _rms_no_eps),
    "rmsnorm_sum_not_mean": ("rms_norm_heads", _rms_sum),
    "attn_scale_1_over_d": ("softmax_attention", _attn_scale_d),
    "attn_softmax_axis": ("softmax_attention", _attn_axis),
    "modulate_no_shift": ("modulate", _mod_no_shift),
    "modulate_scale_not_1p": ("modulate", _mod_plain_scale),
    "layernorm_unbiased": ("layer_norm", _ln_unbiased),
    "linear_transposed": ("linear", _linear_transposed),
    "linear_no_bias": ("linear", _linear_no_bias),
    "gelu_tanh": ("gelu", _gelu_tanh),
    "gates_swapped": ("modulation", _modulation_swapped),
    "shift_scale_swapped": ("modulation", _modulation_order),
    "cond_keys_dropped": ("joint_attention", _joint_drop_cond_keys),
    "sinusoid_sin_first": ("timestep_sinusoid", _sinusoid_sin_first),
    "sinusoid_half_minus_one": ("timestep_sinusoid", _sinusoid_half_minus_one),
    "silu_sigmoid_only": ("silu", _silu_sigmoid_only),
    "timestep_no_inner_silu": ("timestep_path", _timestep_no_inner_silu),
    "timestep_no_outer_silu": ("timestep_path", _timestep_no_outer_silu),
    "merge_column_major": ("lite_merge_gather", _merge_column_major),
    "merge_channel_interleaved": ("lite_merge_gather", _merge_channel_interleaved),
    "unpatchify_swapped_w": ("lite_unpatchify", _unpatchify_swapped_w),
    "fp8_truncate": ("fp8_e4m3_round", _fp8_truncate),
    "fp8_ties_away": ("fp8_e4m3_round", _fp8_ties_away),
    "fp8_scale_127": ("quant_scale", _scale_int8_max),
    "fp8_linear_no_wscale": ("fp8_linear", _fp8_linear_no_wscale),
    "fp8_linear_per_tensor_x": ("fp8_linear", _fp8_linear_per_tensor_x),
    "att8_k_per_token": ("attn8_quantize_stream", _att8_k_per_token),
    "att8_v_per_tensor": ("attn8_quantize_v", _att8_v_per_tensor),
    "int8_truncate": ("quantize_int8", _int8_truncate),
    "att8_floor_reference": ("joint_attention_8bit", _att8_variant(floor=True)),
    "att8_no_shift": ("joint_attention_8bit", _att8_variant(shift=0.0)),
    "att8_unquantized_row_sum": ("joint_attention_8bit", _att8_variant(exact_sum=True)),
    "block8_no_f16_storage": ("f16_round", _f16_not_rounded),
    "block8_weights_per_row": ("fp8_weight", _fp8_weight_per_row),
    "block8_qkv_slice_scales": ("fp8_linear_prequantized", _fp8_linear_requantize_slices),
}

PIN_TESTS = [f for name, f in inspect.getmembers(pins, inspect.isfunction) if name.startswith("test_")]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, monkeypatch):
    name, fn = MUTANTS[mutant]
    monkeypatch.setattr(om, name, fn)
    monkeypatch.setattr(oracle, name, fn)
    failed = []
    for t in PIN_TESTS:
        try:
            t()
        except Exception:
            failed.append(t.__name__)
    assert failed, f"no pin caught mutant {mutant}"
