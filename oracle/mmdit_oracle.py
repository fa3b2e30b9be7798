"""Float64 CPU oracle of the dual-stream MMDiT block core.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU-baseline leg
import this module.  The product path (the HIP library and its binding) never calls it,
shares no code with it, and is not imported by it.

Each function is the plain definition of one step, evaluated in float64 with numpy.
Sources (page title, then section):
- [Vimoo] "Vimoo 1.0: Video Generation for Compact, Lightweight, and High-Speed",
  section 2.2 "Dual-Stream MMDiT Backbone": per-stream Q/K/V projections, joint attention
  over the concatenated sequences, split back; per-stream output projections and FFNs;
  timestep modulation to six C-vectors (shift/scale/gate for attention and FFN) from a
  shared 1536-d bottleneck; LayerNorm before attention and FFN; per-head RMSNorm on Q and
  K with distinct learned scales; 3D RoPE split 16/56/56 over (t, h, w) on visual Q/K only.
  Section 2.4 fixes the modulation Linear's shape through its parameter counts.
- [Wan-zh] Wan 2.1 report, Chinese translation, section 4: 4.1.1 (VAE 4x8x8, 16 ch),
  4.2.1 (patchify (1,2,2), L = (1+T/4)*H/16*W/16), 4.3.1 (forward attention cost factor 4).
- [Wan-guide] reading guide to the Wan report: the DiT's attention is non-causal.

Readings where the pages leave a step open (each one is listed with its reason in the
design notes of the repository):
  r1 modulation form LN(x)*(1+scale)+shift; r2 vector order shift_a, scale_a, gate_a,
  shift_f, scale_f, gate_f; r3 tvec enters the modulation Linear as given; r4 LayerNorm
  eps 1e-6, no affine; r5 every Linear has a bias; r6 QK-norm scale [D] per stream and q/k
  (a per-head [H, D] scale is also accepted); r7 RMSNorm before RoPE; r8 RoPE rotates
  interleaved pairs (2j, 2j+1) inside each band; r9 each band has its own frequency ladder
  base^(-2j/d_band); r10 bands in t, h, w order; r11 0-based integer positions; r12 tokens
  flattened (t, h, w) row-major, w fastest; r13 no YaRN; r14 no attention mask;
  r16 exact erf GELU; r18 parity metric max|err| / rms(oracle) per output tensor;
  r20 timestep sinusoid: cosines of the first half of the frequencies, then sines,
  frequency j = max_period^(-j/half), max_period 10000, the timestep value taken as given;
  r21 the timestep MLP and the bottleneck Linear carry biases, SiLU is x*sigmoid(x);
  r22 Lite merge concatenates the 2x2 neighbours in (dh, dw) row-major order, each
  neighbour's C channels contiguous; the unpatchify output splits the same way;
  r23 Lite merge/unpatchify is defined for even H and W only (odd grids are rejected);
  r24 FP8 is OCP E4M3 (largest 448), rounding to nearest with ties to even, saturating;
  r25 8-bit scales are amax / qmax in float32 (qmax 448 for E4M3, 127 for INT8), an all-zero
  group takes scale 1, and the value to round is x * (1/s) formed in float32;
  r26 / r27 the granularity of the 8-bit attention's scales and its probability rounding
  (stated at joint_attention_8bit below).

Further sources for the Lite parts: [Vimoo] section 2.4 "Vimoo 1.0-Lite" (2x2 hidden-space
merge 4C -> C after the input projection, unpatchify C -> 4C after the backbone, time axis
untouched; the shared timestep bottleneck narrowed from 1536 to 16).

Tensor conventions: tokens [B, N, ...]; heads split as [B, N, H, D] with head-major
channels (channel c = head * D + d).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

# ------------------------------------------------------------------ 3D RoPE  [Vimoo 2.2]


def token_positions(grid: Tuple[int, int, int]) -> np.ndarray:
    """(t, h, w) of each visual token, flattened row-major with w fastest (r12).  [N, 3]."""
    t_n, h_n, w_n = grid
    n = np.arange(t_n * h_n * w_n)
    return np.stack([n // (h_n * w_n), (n // w_n) % h_n, n % w_n], axis=1)


def rope_angles(grid: Tuple[int, int, int], split: Sequence[int] = (16, 56, 56),
                base: float = 10000.0) -> np.ndarray:
    """Rotation angle of every (token, pair): [N, D/2].

    The head dims are cut into three bands, temporal / vertical / horizontal (r10).  Pair j
    of a band of width d_a turns by pos_a * base^(-2j/d_a) (r9), pos_a the token's integer
    coordinate on that axis (r11).
    """
    pos = token_positions(grid).astype(np.float64)
    cols = []
    for axis, d_a in enumerate(split):
        if d_a % 2:
            raise ValueError("RoPE band widths must be even")
        j = np.arange(d_a // 2, dtype=np.float64)
        freq = base ** (-2.0 * j / d_a)
        cols.append(pos[:, axis:axis + 1] * freq[None, :])
    return np.concatenate(cols, axis=1)


def rope_rotate(x: np.ndarray, angles: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs (x[2j], x[2j+1]) by angles[..., j] (r8).

    x: [B, N, H, D]; angles: [N, D/2] (broadcast over batch and heads)."""
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    c = np.cos(angles)[None, :, None, :]
    s = np.sin(angles)[None, :, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ------------------------------------------------------------ QK RMSNorm  [Vimoo 2.2]


def rms_norm_heads(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Per-(token, head) RMSNorm over the head dim, times the learned scale g.

    x: [B, N, H, D]; g: [D] shared by all heads, or [H, D] per head (r6)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    g = np.asarray(g, dtype=np.float64)
    g = g[None, None, None, :] if g.ndim == 1 else g[None, None, :, :]
    return x / np.sqrt(ms + eps) * g


def qk_norm_rope(q: np.ndarray, k: np.ndarray, gq: np.ndarray, gk: np.ndarray, eps: float,
                 grid: Optional[Tuple[int, int, int]] = None,
                 split: Sequence[int] = (16, 56, 56), base: float = 10000.0):
    """RMSNorm on q and k with their own scales, then 3D RoPE when ``grid`` is given
    (visual stream); the conditioning stream passes ``grid=None`` and gets no rotation (r7)."""
    qn = rms_norm_heads(q, gq, eps)
    kn = rms_norm_heads(k, gk, eps)
    if grid is not None:
        ang = rope_angles(grid, split, base)
        if ang.shape[0] != q.shape[1]:
            raise ValueError("visual token count differs from T*H*W")
        qn = rope_rotate(qn, ang)
        kn = rope_rotate(kn, ang)
    return qn, kn


# ------------------------------------------------------- joint attention  [Vimoo 2.2]


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q k^T * scale) v for one batch item and head, no mask (r14).
    q: [M, D]; k, v: [N, D]."""
    s = (q @ k.T) * scale
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ v


def joint_attention(q_vis, k_vis, v_vis, q_cond, k_cond, v_cond,
                    scale: Optional[float] = None,
                    vis_rows: Optional[np.ndarray] = None,
                    cond_rows: Optional[np.ndarray] = None,
                    chunk: int = 2048):
    """Joint non-causal attention over the concatenated conditioning and visual tokens,
    split back into the two streams.

    Inputs [B, N_s, H, D] (already normalised and rotated).  The concatenation order does not
    change any output, so the keys are taken as [cond | vis].  ``vis_rows`` / ``cond_rows``
    restrict the output to those query rows (every key is still used); queries are
    evaluated in chunks of ``chunk`` rows to bound the [chunk, N] score block.
    Returns (o_vis, o_cond), each [B, rows, H, D].
    """
    b, _, h, d = q_vis.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    k_all = np.concatenate([k_cond, k_vis], axis=1)
    v_all = np.concatenate([v_cond, v_vis], axis=1)

    def run(q, rows):
        if rows is not None:
            q = q[:, rows]
        out = np.empty(q.shape, dtype=np.float64)
        for bi in range(b):
            for hi in range(h):
                kk = k_all[bi, :, hi, :]
                vv = v_all[bi, :, hi, :]
                for r0 in range(0, q.shape[1], chunk):
                    out[bi, r0:r0 + chunk, hi, :] = softmax_attention(
                        q[bi, r0:r0 + chunk, hi, :], kk, vv, scale)
        return out

    return run(q_vis, vis_rows), run(q_cond, cond_rows)


def attention_block(inp: Dict[str, np.ndarray], grid, eps: float,
                    split=(16, 56, 56), base: float = 10000.0,
                    vis_rows=None, cond_rows=None):
    """QK-RMSNorm (+ RoPE on visual) then joint attention: the attention-only workloads.
    ``inp`` holds float64 q/k/v_{vis,cond} [B,N,H,D] and gq/gk_{vis,cond}.
    Returns dict with qh/kh for both streams and o_vis / o_cond."""
    qv, kv = qk_norm_rope(inp["q_vis"], inp["k_vis"], inp["gq_vis"], inp["gk_vis"], eps,
                          grid, split, base)
    qc, kc = qk_norm_rope(inp["q_cond"], inp["k_cond"], inp["gq_cond"], inp["gk_cond"], eps)
    o_v, o_c = joint_attention(qv, kv, inp["v_vis"], qc, kc, inp["v_cond"],
                               vis_rows=vis_rows, cond_rows=cond_rows)
    return {"qh_vis": qv, "kh_vis": kv, "qh_cond": qc, "kh_cond": kc,
            "o_vis": o_v, "o_cond": o_c}


# ------------------------------------------------- modulation, LN, FFN  [Vimoo 2.2]

MOD_ORDER = ("shift_a", "scale_a", "gate_a", "shift_f", "scale_f", "gate_f")   # r2


def modulation_param_count(width: int, t_dim: int) -> int:
    """Parameters of one per-(block, stream) modulation Linear t_dim -> 6*width, with bias."""
    return 6 * width * t_dim + 6 * width


def modulation(w_mod: np.ndarray, b_mod: np.ndarray, tvec: np.ndarray) -> Dict[str, np.ndarray]:
    """mod = W_mod @ tvec + b_mod (tvec enters as given, r3), cut into six C-vectors.
    w_mod [6C, Dt]; tvec [B, Dt] -> each vector [B, C]."""
    m = tvec @ w_mod.T + b_mod[None, :]
    c = w_mod.shape[0] // 6
    return {name: m[:, i * c:(i + 1) * c] for i, name in enumerate(MOD_ORDER)}


def layer_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last dim, biased variance, no affine (r4)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(xn: np.ndarray, shift: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Shift and scale the normalised features (r1).  xn [B, N, C]; shift/scale [B, C]."""
    return xn * (1.0 + scale[:, None, :]) + shift[:, None, :]


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """nn.Linear: x @ w^T + b, w in [out, in] layout (r5)."""
    y = x @ w.T
    return y if b is None else y + b


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU x * Phi(x) (r16)."""
    from scipy.special import erf
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def block_forward(x_vis: np.ndarray, x_cond: np.ndarray, tvec: np.ndarray,
                  w_vis: Dict[str, np.ndarray], w_cond: Dict[str, np.ndarray],
                  grid: Tuple[int, int, int], heads: int,
                  ln_eps: float = 1e-6, qk_eps: float = 1e-6,
                  split=(16, 56, 56), base: float = 10000.0,
                  vis_rows: Optional[np.ndarray] = None,
                  cond_rows: Optional[np.ndarray] = None,
                  keep: bool = True) -> Dict[str, np.ndarray]:
    """One dual-stream block forward [Vimoo 2.2].

    Per stream s: mod_s from the shared tvec; h = LN(x)*(1+scale_a)+shift_a;
    [q|k|v] = h W_qkv^T + b; QK-RMSNorm, RoPE on visual; joint attention over both streams;
    a = O W_o^T + b_o; x1 = x + gate_a*a; h2 = LN(x1)*(1+scale_f)+shift_f;
    out = x1 + gate_f * (GELU(h2 W_1^T + b_1) W_2^T + b_2).

    Every key and value is computed; ``vis_rows`` / ``cond_rows`` restrict the per-query
    work after the K/V projection to those rows.  Returns the outputs and (``keep``) the
    intermediates of the same rows, keyed ``<name>_vis`` / ``<name>_cond``.
    """
    c = x_vis.shape[-1]
    d = c // heads
    res: Dict[str, np.ndarray] = {}
    qkv = {}
    mods = {}
    for s, x, w, rows in (("vis", x_vis, w_vis, vis_rows), ("cond", x_cond, w_cond, cond_rows)):
        mods[s] = modulation(w[ "w_mod"], w["b_mod"], tvec)
        m = mods[s]
        h = modulate(layer_norm(x, ln_eps), m["shift_a"], m["scale_a"])
        b_, n_ = x.shape[:2]
        # K and V of every token; Q of the requested rows only.
        w_q, w_k, w_v = np.split(w["w_qkv"], 3, axis=0)
        b_q, b_k, b_v = np.split(w["b_qkv"], 3)
        hq = h if rows is None else h[:, rows]
        q = linear(hq, w_q, b_q).reshape(b_, hq.shape[1], heads, d)
        k = linear(h, w_k, b_k).reshape(b_, n_, heads, d)
        v = linear(h, w_v, b_v).reshape(b_, n_, heads, d)
        qkv[s] = (q, k, v)
        if keep:
            res[f"h_{s}"] = hq
            res[f"mod_{s}"] = np.concatenate([m[nm] for nm in MOD_ORDER], axis=-1)
    q_v, k_v, v_v = qkv["vis"]
    q_c, k_c, v_c = qkv["cond"]
    # RMSNorm on every k; RoPE needs each row's own position.
    k_v = rms_norm_heads(k_v, w_vis["k_norm"], qk_eps)
    k_v = rope_rotate(k_v, rope_angles(grid, split, base))
    q_v = rms_norm_heads(q_v, w_vis["q_norm"], qk_eps)
    ang = rope_angles(grid, split, base)
    q_v = rope_rotate(q_v, ang if vis_rows is None else ang[vis_rows])
    k_c = rms_norm_heads(k_c, w_cond["k_norm"], qk_eps)
    q_c = rms_norm_heads(q_c, w_cond["q_norm"], qk_eps)
    o_v, o_c = joint_attention(q_v, k_v, v_v, q_c, k_c, v_c)
    if keep:
        res["qh_vis"], res["qh_cond"] = q_v, q_c
    for s, x, w, rows, o in (("vis", x_vis, w_vis, vis_rows, o_v),
                             ("cond", x_cond, w_cond, cond_rows, o_c)):
        m = mods[s]
        xs = x if rows is None else x[:, rows]
        o = o.reshape(o.shape[0], o.shape[1], c)
        a = linear(o, w["w_o"], w["b_o"])
        x1 = xs + m["gate_a"][:, None, :] * a
        h2 = modulate(layer_norm(x1, ln_eps), m["shift_f"], m["scale_f"])
        g = gelu(linear(h2, w["w_fc1"], w["b_fc1"]))
        out = x1 + m["gate_f"][:, None, :] * linear(g, w["w_fc2"], w["b_fc2"])
        res[f"out_{s}"] = out
        if keep:
            res[f"o_{s}"] = o
            res[f"x1_{s}"] = x1
            res[f"h2_{s}"] = h2
    return res


# ------------------------------------------------------- timestep path  [Vimoo 2.2, 2.4]


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU x * sigmoid(x) (r21)."""
    from scipy.special import expit
    return x * expit(x)


def timestep_sinusoid(t: np.ndarray, dim: int = 256, max_period: float = 10000.0) -> np.ndarray:
    """Sinusoidal embedding of each timestep: [B] -> [B, dim] (r20).

    With half = dim/2 frequencies w_j = max_period^(-j/half), j = 0..half-1, the first half of
    the vector holds cos(t*w_j) and the second half sin(t*w_j)."""
    half = dim // 2
    j = np.arange(half, dtype=np.float64)
    freqs = max_period ** (-j / half)
    ang = np.asarray(t, dtype=np.float64)[:, None] * freqs[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def timestep_path(t: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray, b2: np.ndarray,
                  w3: np.ndarray, b3: np.ndarray, dim: int = 256,
                  max_period: float = 10000.0) -> Dict[str, np.ndarray]:
    """Timestep conditioning [Vimoo 2.2]: the 256-d sinusoid goes through a two-layer MLP with
    a SiLU between the layers to the 3072-d representation ``temb``; SiLU and one Linear then
    give the shared bottleneck ``tvec`` (1536-d, 16-d in Lite [Vimoo 2.4]).

    w1 [Dh, dim], w2 [Dh, Dh], w3 [Dt, Dh] in nn.Linear layout.  Returns ``hidden`` (the first
    layer's output before its SiLU), ``temb`` and ``tvec``."""
    e = timestep_sinusoid(t, dim, max_period)
    hidden = linear(e, w1, b1)
    temb = linear(silu(hidden), w2, b2)
    tvec = linear(silu(temb), w3, b3)
    return {"hidden": hidden, "temb": temb, "tvec": tvec}


# ------------------------------------------------- Lite 2x2 hidden-space merge  [Vimoo 2.4]

NEIGHBOURS = ((0, 0), (0, 1), (1, 0), (1, 1))   # r22: (dh, dw) row-major


def _check_even(grid: Tuple[int, int, int]):
    if grid[1] % 2 or grid[2] % 2:
        raise ValueError(f"Lite 2x2 merge needs an even H and W grid, got {grid} (r23)")


def lite_merge_gather(x: np.ndarray, grid: Tuple[int, int, int]) -> np.ndarray:
    """[B, T*H*W, C] visual tokens -> [B, T*(H/2)*(W/2), 4C]: for each 2x2 spatial region of
    each frame, the four neighbours' vectors side by side (r22).  Time is not merged."""
    _check_even(grid)
    t_n, h_n, w_n = grid
    b, n, c = x.shape
    x5 = x.reshape(b, t_n, h_n, w_n, c)
    parts = [x5[:, :, dh::2, dw::2, :] for dh, dw in NEIGHBOURS]     # each [B, T, H/2, W/2, C]
    return np.concatenate(parts, axis=-1).reshape(b, t_n * (h_n // 2) * (w_n // 2), 4 * c)


def lite_merge(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray],
               grid: Tuple[int, int, int]) -> np.ndarray:
    """Lite merge: concatenate each 2x2 neighbourhood, then Linear 4C -> C.  w [C, 4C]."""
    return linear(lite_merge_gather(x, grid), w, b)


def lite_unpatchify(y: np.ndarray, w: np.ndarray, b: Optional[np.ndarray],
                    grid: Tuple[int, int, int]) -> np.ndarray:
    """Lite unpatchify: Linear C -> 4C expands each merged token into four position-specific
    vectors, placed back at the 2x2 positions in the merge's order.  y [B, T*(H/2)*(W/2), C],
    w [4C, C]; ``grid`` is the full (T, H, W) grid.  Returns [B, T*H*W, C]."""
    _check_even(grid)
    t_n, h_n, w_n = grid
    z = linear(y, w, b)
    bsz, _, c4 = z.shape
    c = c4 // 4
    z5 = z.reshape(bsz, t_n, h_n // 2, w_n // 2, c4)
    out = np.zeros((bsz, t_n, h_n, w_n, c), dtype=z.dtype)
    for s, (dh, dw) in enumerate(NEIGHBOURS):
        out[:, :, dh::2, dw::2, :] = z5[..., s * c:(s + 1) * c]
    return out.reshape(bsz, t_n * h_n * w_n, c)


# ------------------------------------------------- 8-bit quantization  [Wan-zh 4.4.3]
#
# The Wan report (section 4.4.3) runs the DiT's GEMMs in FP8 with a per-tensor scale for the
# weights and a per-token scale for the activations, and its attention with INT8 for Q K^T
# and FP8 (E4M3) for P V, accumulating across blocks in FP32.  E4M3 below is the OCP FP8
# format: 1 sign, 4 exponent (bias 7), 3 mantissa bits, no infinities, largest finite 448.

FP8_E4M3_MAX = 448.0
INT8_MAX = 127.0


def _round_half_even(v: np.ndarray) -> np.ndarray:
    return np.round(v)   # numpy rounds halves to even


def fp8_e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value of each element (ties to even mantissa), saturating at +-448
    (r24).  Normal numbers are 2^e (1 + m/8), e in [-6, 8]; below 2^-6 the spacing is the
    subnormal step 2^-9."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    out = np.empty_like(a)
    sub = a < 2.0 ** -6
    out[sub] = _round_half_even(a[sub] / 2.0 ** -9) * 2.0 ** -9
    an = a[~sub]
    e = np.floor(np.log2(an))
    # guard the log2 rounding at exact powers of two
    e = np.where(2.0 ** e > an, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= an, e + 1, e)
    step = 2.0 ** (e - 3)
    out[~sub] = _round_half_even(an / step) * step
    out = np.minimum(out, FP8_E4M3_MAX)
    return np.copysign(out, x)


def fp8_e4m3_code(v: np.ndarray) -> np.ndarray:
    """Bit pattern (uint8) of E4M3 values (as returned by fp8_e4m3_round)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    code = np.zeros(a.shape, dtype=np.uint8)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.uint8)
    an = a[~sub]
    e = np.floor(np.log2(an))
    e = np.where(2.0 ** e > an, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= an, e + 1, e)
    m = np.rint((an / 2.0 ** e - 1.0) * 8).astype(np.int64)
    code[~sub] = ((e.astype(np.int64) + 7) << 3 | m).astype(np.uint8)
    return code | sign


def fp8_e4m3_decode(code: np.ndarray) -> np.ndarray:
    """Value of each E4M3 bit pattern (0x7F / 0xFF, the NaN codes, never occur here)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    return s * mag


def quant_scale(amax: np.ndarray, qmax: float) -> np.ndarray:
    """Scale s = amax / qmax evaluated in float32, with an all-zero group given s = 1 (r25)."""
    amax = np.asarray(amax, dtype=np.float32)
    s = (amax / np.float32(qmax)).astype(np.float32)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def quantize_fp8(x: np.ndarray, per_row: bool):
    """Symmetric FP8 E4M3 quantization with a scale per row (token) or one per tensor
    (r25): s = amax / 448 in float32; the code is the E4M3 rounding of x * (1/s), that
    product formed in float32.  Returns (values of the codes [same shape], scales
    [rows] or [1])."""
    x32 = np.asarray(x, dtype=np.float32)
    if per_row:
        amax = np.max(np.abs(x32), axis=-1)
    else:
        amax = np.array([np.max(np.abs(x32))], dtype=np.float32)
    s = quant_scale(amax, FP8_E4M3_MAX)
    inv = (np.float32(1.0) / s).astype(np.float32)
    inv_b = inv[..., None] if per_row else inv[0]
    y = (x32 * inv_b).astype(np.float32)
    y = np.clip(y, -FP8_E4M3_MAX, FP8_E4M3_MAX)
    return fp8_e4m3_round(y), s


def fp8_linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """The FP8 Linear of [Wan-zh] 4.4.3: x quantized per token, w per tensor, the product of
    the quantized values taken exactly, then rescaled: y = (q_x q_w^T) s_x s_w + b.
    x [M, K], w [N, K]."""
    qx, sx = quantize_fp8(x, per_row=True)
    qw, sw = quantize_fp8(w, per_row=False)
    y = (qx @ qw.T) * sx.astype(np.float64)[:, None] * float(sw[0])
    return y if b is None else y + b


# ---------------------------------------------- 8-bit joint attention  [Wan-zh 4.4.3]
#
# The Wan report (section 4.4.3) keeps S = Q K^T in INT8 and O = P V in FP8 (E4M3), with the
# cross-block accumulation in FP32.  Readings taken where the page is silent:
#   r26 Q^ has one INT8 scale per (token, head) and K^ one per (head, block of 64 consecutive
#       keys of one stream); V has one FP8 scale per (head, channel) over all keys of both
#       streams; each scale follows r25 (qmax 127 for INT8, 448 for E4M3; INT8 codes are
#       rint(x * (1/s)) clamped to +-127, ties to even);
#   r27 logits in log2 units y = acc * s_q * s_k * scale * log2(e), acc the exact integer dot
#       product of the codes and s_q, s_k the float32 scales of r25; the row reference is the
#       integer M = ceil(max_j y); each weight is the E4M3 rounding of the exact value
#       2^(y + 8 - M) (so P' <= 256); the row sum adds the same E4M3 weights:
#       O = (sum_j P'_j V^_j) / (sum_j P'_j), V^ the dequantized values.
# The codes and scales of Q, K and V are the r25 rule (an f32 product rounded); everything
# after them (logits, reference, weights, sums) is evaluated in float64.

LOG2E = 1.4426950408889634
ATT8_KEY_BLOCK = 64


def quantize_int8(x: np.ndarray, axes) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric INT8 codes of x with one scale per group (the reduced ``axes``), r25 / r26.
    Returns (codes as float64, scales float32 with the reduced axes kept as size 1)."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=axes, keepdims=True)
    s = quant_scale(amax, INT8_MAX)
    inv = (np.float32(1.0) / s).astype(np.float32)
    y = (x32 * inv).astype(np.float32)
    return np.clip(np.rint(y), -INT8_MAX, INT8_MAX).astype(np.float64), s


def quantize_fp8_groups(x: np.ndarray, axes) -> Tuple[np.ndarray, np.ndarray]:
    """FP8 E4M3 values of x with one scale per group (reduced ``axes``), r25."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=axes, keepdims=True)
    s = quant_scale(amax, FP8_E4M3_MAX)
    inv = (np.float32(1.0) / s).astype(np.float32)
    y = np.clip((x32 * inv).astype(np.float32), -FP8_E4M3_MAX, FP8_E4M3_MAX)
    return fp8_e4m3_round(y), s


def attn8_quantize_stream(q: np.ndarray, k: np.ndarray):
    """INT8 codes and scales of one stream's Q^ and K^ (r26).  q, k [B, n, H, D].
    Returns q8 [B, n, H, D], sq [B, n, H], k8 [B, n, H, D], sk [B, H, ceil(n/64)]."""
    b, _, h, d = q.shape
    n = k.shape[1]
    q8, sq = quantize_int8(q, axes=3)
    nb = -(-n // ATT8_KEY_BLOCK)
    k8 = np.empty(k.shape, dtype=np.float64)
    sk = np.empty((b, h, nb), dtype=np.float32)
    for j in range(nb):
        blk = k[:, j * ATT8_KEY_BLOCK:(j + 1) * ATT8_KEY_BLOCK]            # [B, <=64, H, D]
        codes, s = quantize_int8(blk, axes=(1, 3))                          # s [B, 1, H, 1]
        k8[:, j * ATT8_KEY_BLOCK:(j + 1) * ATT8_KEY_BLOCK] = codes
        sk[:, :, j] = s[:, 0, :, 0]
    return q8, sq[..., 0], k8, sk


def attn8_quantize_v(v_vis: np.ndarray, v_cond: np.ndarray):
    """FP8 E4M3 values of V with one scale per (batch, head, channel) over the keys of both
    streams (r26).  Returns (v8_vis, v8_cond, sv [B, H, D])."""
    n_vis = v_vis.shape[1]
    v_all = np.concatenate([v_vis, v_cond], axis=1)
    v8, sv = quantize_fp8_groups(v_all, axes=1)                             # sv [B, 1, H, D]
    return v8[:, :n_vis], v8[:, n_vis:], sv[:, 0]


def joint_attention_8bit(q_vis, k_vis, v_vis, q_cond, k_cond, v_cond,
                         scale: Optional[float] = None,
                         vis_rows: Optional[np.ndarray] = None,
                         cond_rows: Optional[np.ndarray] = None, chunk: int = 1024,
                         return_lse: bool = False, return_row_sums: bool = False):
    """The 8-bit joint attention of [Wan-zh] 4.4.3 under readings r26 / r27.  Inputs as for
    joint_attention (Q^, K^ already normalised and rotated).  Returns (o_vis, o_cond) and,
    with ``return_lse``, the natural-log row sums ln(sum_j 2^y_j) of the quantized weights,
    i.e. ln(sum_j P'_j) + (M - 8) ln 2, laid out [B, H, n_cond + n_vis] ([cond | vis]); with
    ``return_row_sums``, the sums sum_j P'_j themselves ([B, H, rows] per stream, in the
    order of the returned rows)."""
    qa, sqa, ka, ska = attn8_quantize_stream(q_vis, k_vis)
    qc, sqc, kcd, skc = attn8_quantize_stream(q_cond, k_cond)
    v8v, v8c, sv = attn8_quantize_v(v_vis, v_cond)
    return attention_8bit_from_codes(qa, sqa, ka, ska, qc, sqc, kcd, skc, v8v, v8c, sv, scale,
                                     vis_rows, cond_rows, chunk, return_lse, return_row_sums)


def attention_8bit_from_codes(qa, sqa, ka, ska, qc, sqc, kcd, skc, v8v, v8c, sv,
                              scale: Optional[float] = None,
                              vis_rows: Optional[np.ndarray] = None,
                              cond_rows: Optional[np.ndarray] = None, chunk: int = 1024,
                              return_lse: bool = False, return_row_sums: bool = False):
    """The steps of joint_attention_8bit after the quantization (r27), from the codes and
    scales of attn8_quantize_stream (per stream: Q codes [B, n, H, D], their scales [B, n, H],
    K codes, K block scales [B, H, ceil(n/64)]) and attn8_quantize_v (V values of the codes
    per stream, V scales [B, H, D]).  Options and result as for joint_attention_8bit."""
    b, _, h, d = qa.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    kc = float(scale) * LOG2E
    # keys in [vis | cond] order (any order gives the same result), each with its block scale
    k8 = np.concatenate([ka, kcd], axis=1)                                  # [B, N, H, D]
    v8 = np.concatenate([v8v, v8c], axis=1)
    blk = lambda s_, n: np.repeat(s_, ATT8_KEY_BLOCK, axis=2)[:, :, :n]    # noqa: E731
    skj = np.concatenate([blk(ska, ka.shape[1]), blk(skc, kcd.shape[1])], axis=2)   # [B, H, N]
    skcj = skj.astype(np.float64) * kc

    def run(q8, sq, rows):
        if rows is not None:
            q8, sq = q8[:, rows], sq[:, rows]
        nq = q8.shape[1]
        out = np.empty((b, nq, h, d), dtype=np.float64)
        lse = np.empty((b, h, nq), dtype=np.float64)
        sums = np.empty((b, h, nq), dtype=np.float64)
        for bi in range(b):
            for hi in range(h):
                kk = k8[bi, :, hi, :]
                for i0 in range(0, nq, chunk):
                    acc = q8[bi, i0:i0 + chunk, hi, :] @ kk.T                # exact integers
                    c = sq[bi, i0:i0 + chunk, hi].astype(np.float64)[:, None] * skcj[bi, hi][None, :]
                    y = acc * c                                              # log2 units
                    m = np.ceil(y.max(axis=1, keepdims=True))
                    p = fp8_e4m3_round(np.exp2(y + (8.0 - m)))
                    ell = p.sum(axis=1, keepdims=True)
                    out[bi, i0:i0 + chunk, hi, :] = (p @ v8[bi, :, hi, :]) * sv[bi, hi][None, :] / ell
                    lse[bi, hi, i0:i0 + chunk] = np.log(ell[:, 0]) + (m[:, 0] - 8.0) * math.log(2.0)
                    sums[bi, hi, i0:i0 + chunk] = ell[:, 0]
        return out, lse, sums

    o_vis, lse_v, sum_v = run(qa, sqa, vis_rows)
    o_cond, lse_c, sum_c = run(qc, sqc, cond_rows)
    res = (o_vis, o_cond)
    if return_lse:
        res = res + (np.concatenate([lse_c, lse_v], axis=2),)
    if return_row_sums:
        res = res + (sum_v, sum_c)
    return res


# ------------------------------------------------------- 8-bit block  [Wan-zh 4.4.3]
#
# The Wan report (section 4.4.3) serves the DiT with FP8 GEMMs (per-tensor weight scales,
# per-token activation scales) and the 8-bit attention.  The 8-bit block is the block of
# [Vimoo 2.2] (block_forward) with (reading r28):
#   - each of its four Linears (QKV, output, FFN up, FFN down) the FP8 Linear of r24 / r25,
#     the weight matrix quantized as one tensor (one scale for all of W_qkv's q, k and v
#     rows), the activation per token;
#   - the joint attention the 8-bit attention of r26 / r27;
#   - the quantizers' inputs the block's stored 16-bit intermediates h, O, h2, GELU output
#     and q^ | k^ | v, i.e. those tensors rounded to f16 (nearest even); the modulation, the
#     LayerNorm statistics, the residual x1 and the outputs are not rounded.


def f16_round(x: np.ndarray) -> np.ndarray:
    """x rounded to IEEE binary16 (nearest even), back in float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def fp8_weight(w: np.ndarray) -> Tuple[np.ndarray, float]:
    """A weight matrix quantized per tensor (r25): (E4M3 values, scale)."""
    qw, sw = quantize_fp8(w, per_row=False)
    return qw, float(sw[0])


def fp8_linear_prequantized(x: np.ndarray, qw: np.ndarray, sw: float, b: Optional[np.ndarray]) -> np.ndarray:
    """The FP8 Linear with an already quantized weight: x [..., K] quantized per token (r25),
    the product of the quantized values exact, y = (q_x q_w^T) s_x s_w + b."""
    qx, sx = quantize_fp8(x, per_row=True)
    y = (qx @ qw.T) * sx.astype(np.float64)[..., None] * sw
    return y if b is None else y + b


def block_forward_8bit(x_vis: np.ndarray, x_cond: np.ndarray, tvec: np.ndarray,
                       w_vis: Dict[str, np.ndarray], w_cond: Dict[str, np.ndarray],
                       grid: Tuple[int, int, int], heads: int,
                       ln_eps: float = 1e-6, qk_eps: float = 1e-6,
                       split=(16, 56, 56), base: float = 10000.0,
                       vis_rows: Optional[np.ndarray] = None,
                       cond_rows: Optional[np.ndarray] = None,
                       keep: bool = True) -> Dict[str, np.ndarray]:
    """The 8-bit dual-stream block (r28): block_forward's steps with FP8 Linears and the
    8-bit joint attention, each quantizer fed the f16 rounding of its input.  Arguments and
    result as for block_forward (``*_rows`` restrict the query-side work to those rows)."""
    c = x_vis.shape[-1]
    d = c // heads
    res: Dict[str, np.ndarray] = {}
    mods, qkv, wq = {}, {}, {}
    for s, x, w, rows in (("vis", x_vis, w_vis, vis_rows), ("cond", x_cond, w_cond, cond_rows)):
        wq[s] = {k: fp8_weight(w[k]) for k in ("w_qkv", "w_o", "w_fc1", "w_fc2")}
        mods[s] = modulation(w["w_mod"], w["b_mod"], tvec)
        m = mods[s]
        h = f16_round(modulate(layer_norm(x, ln_eps), m["shift_a"], m["scale_a"]))
        b_, n_ = x.shape[:2]
        qw, sw = wq[s]["w_qkv"]
        qw_q, qw_k, qw_v = np.split(qw, 3, axis=0)
        b_q, b_k, b_v = np.split(w["b_qkv"], 3)
        hq = h if rows is None else h[:, rows]
        # the stored projections are f16; q^ and k^ are normalised and rotated from them
        q = f16_round(fp8_linear_prequantized(hq, qw_q, sw, b_q)).reshape(b_, hq.shape[1], heads, d)
        k = f16_round(fp8_linear_prequantized(h, qw_k, sw, b_k)).reshape(b_, n_, heads, d)
        v = f16_round(fp8_linear_prequantized(h, qw_v, sw, b_v)).reshape(b_, n_, heads, d)
        qkv[s] = (q, k, v)
        if keep:
            res[f"h_{s}"] = hq
            res[f"mod_{s}"] = np.concatenate([m[nm] for nm in MOD_ORDER], axis=-1)
    q_v, k_v, v_v = qkv["vis"]
    q_c, k_c, v_c = qkv["cond"]
    ang = rope_angles(grid, split, base)
    k_v = f16_round(rope_rotate(rms_norm_heads(k_v, w_vis["k_norm"], qk_eps), ang))
    q_v = f16_round(rope_rotate(rms_norm_heads(q_v, w_vis["q_norm"], qk_eps),
                                ang if vis_rows is None else ang[vis_rows]))
    k_c = f16_round(rms_norm_heads(k_c, w_cond["k_norm"], qk_eps))
    q_c = f16_round(rms_norm_heads(q_c, w_cond["q_norm"], qk_eps))
    o_v, o_c = joint_attention_8bit(q_v, k_v, v_v, q_c, k_c, v_c)
    if keep:
        res["qh_vis"], res["qh_cond"] = q_v, q_c
    for s, x, w, rows, o in (("vis", x_vis, w_vis, vis_rows, o_v),
                             ("cond", x_cond, w_cond, cond_rows, o_c)):
        m = mods[s]
        xs = x if rows is None else x[:, rows]
        o = f16_round(o.reshape(o.shape[0], o.shape[1], c))
        a = fp8_linear_prequantized(o, *wq[s]["w_o"], w["b_o"])
        x1 = xs + m["gate_a"][:, None, :] * a
        h2 = f16_round(modulate(layer_norm(x1, ln_eps), m["shift_f"], m["scale_f"]))
        g = f16_round(gelu(fp8_linear_prequantized(h2, *wq[s]["w_fc1"], w["b_fc1"])))
        out = x1 + m["gate_f"][:, None, :] * fp8_linear_prequantized(g, *wq[s]["w_fc2"], w["b_fc2"])
        res[f"out_{s}"] = out
        if keep:
            res[f"o_{s}"] = o
            res[f"x1_{s}"] = x1
            res[f"h2_{s}"] = h2
    return res


# ------------------------------------------------------------------ parity metric (r18)


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / sqrt(mean(ref^2)), in float64."""
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / rms if rms > 0 else float(np.max(np.abs(got - ref)))


# ------------------------------------------------------------------ FLOP accounting


def attention_flops(n_tokens: int, head_dim: int, heads: int, batch: int = 1) -> float:
    """Forward non-causal attention cost with factor 4 on s^2*h ([Wan-zh] 4.3.1):
    two N x N x D products per head, 2 FLOP per multiply-add."""
    return 4.0 * n_tokens * n_tokens * head_dim * heads * batch
