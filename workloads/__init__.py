"""Seeded synthetic workloads for the dual-stream MMDiT block core.

This module is shared test/bench infrastructure.  It holds shapes and random draws
only; it contains no step of the block's arithmetic.  Both the float64 oracle and the
HIP path take their inputs from the generators below, so the two see the same values.

Shapes follow the pages:
- visual tokens come from Wan-VAE latents (4x8x8 compression, 16 channels; Wan 2.1
  report, Chinese translation, section 4.1.1) patchified by a (1,2,2) kernel (same
  report, section 4.2.1), flattened in (t, h, w) order with w fastest;
- 24 heads of 128 dims (width 3072) and the 1536-d shared timestep bottleneck are the
  Vimoo 1.0 notes' backbone (section 2.2);
- 512 conditioning tokens match the umT5 text length of the Wan report (section 4.2.2).

Storage convention: bf16 tensors are numpy ``uint16`` arrays holding bf16 bit patterns,
rounded once from float32 with round-to-nearest-even; fp32 tensors are ``float32``.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

F32 = "f32"
BF16 = "bf16"
F16 = "f16"


# --------------------------------------------------------------------------- shapes
@dataclasses.dataclass(frozen=True)
class AttnConfig:
    """One joint-attention workload: QK-RMSNorm (+3D RoPE on visual) then attention."""
    name: str
    dtype: str                      # storage dtype of Q/K/V and of the norm scales
    heads: int
    head_dim: int
    grid: Tuple[int, int, int]      # latent (T, H, W) grid of visual tokens
    n_cond: int
    rope_split: Tuple[int, int, int] = (16, 56, 56)
    rope_base: float = 10000.0
    qk_eps: float = 1e-6
    batch: int = 1
    seed: int = 0

    @property
    def n_vis(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def n_tokens(self) -> int:
        return self.n_vis + self.n_cond

    @property
    def attn_flops(self) -> float:
        """Forward attention FLOPs, 4*N^2*D*H per batch item (non-causal, two GEMMs)."""
        return 4.0 * self.n_tokens ** 2 * self.head_dim * self.heads * self.batch


@dataclasses.dataclass(frozen=True)
class BlockConfig:
    """One full dual-stream block forward."""
    name: str
    width: int                      # C = heads * head_dim
    heads: int
    head_dim: int
    ffn: int                        # F
    t_dim: int                      # shared timestep bottleneck width
    grid: Tuple[int, int, int]
    n_cond: int
    rope_split: Tuple[int, int, int] = (16, 56, 56)
    rope_base: float = 10000.0
    ln_eps: float = 1e-6
    qk_eps: float = 1e-6
    batch: int = 1
    seed: int = 0

    @property
    def n_vis(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def n_tokens(self) -> int:
        return self.n_vis + self.n_cond

    @property
    def attn_flops(self) -> float:
        return 4.0 * self.n_tokens ** 2 * self.head_dim * self.heads * self.batch

    @property
    def linear_flops(self) -> float:
        """QKV (3C^2) + out (C^2) + FFN (2CF) multiply-adds, x2 FLOP, per token."""
        c, f = self.width, self.ffn
        per_tok = 2.0 * (3 * c * c + c * c + 2 * c * f)
        return per_tok * self.n_tokens * self.batch

    @property
    def total_flops(self) -> float:
        return self.attn_flops + self.linear_flops


# The five measured workloads.  1 is the tiny fp32 case, 2 one layer-sized case,
# 3 and 4 the 81-frame 480p / 720p latent grids, 5 the full block at 480p.
ATTN_TINY = AttnConfig("tiny_fp32_2x128_grid2x4x4_cond8", F32, 2, 128, (2, 4, 4), 8, seed=1)
ATTN_LAYER = AttnConfig("layer_bf16_24x128_grid5x16x16_cond77", BF16, 24, 128, (5, 16, 16), 77, seed=2)
ATTN_480P = AttnConfig("480p_bf16_24x128_grid21x30x52_cond512", BF16, 24, 128, (21, 30, 52), 512, seed=3)
ATTN_720P = AttnConfig("720p_bf16_24x128_grid21x45x80_cond512", BF16, 24, 128, (21, 45, 80), 512, seed=4)
BLOCK_480P = BlockConfig("block480p_bf16_c3072_h24_f12288_grid21x30x52_cond512",
                         3072, 24, 128, 12288, 1536, (21, 30, 52), 512, seed=5)

# Smaller cases used by parity tests: several tiles plus ragged tails.
BLOCK_TINY = BlockConfig("block_tiny_c256_h2_f1024_grid2x4x4_cond8",
                         256, 2, 128, 1024, 64, (2, 4, 4), 8, seed=11)
BLOCK_SMALL = BlockConfig("block_small_c3072_h24_f12288_grid3x8x9_cond77",
                          3072, 24, 128, 12288, 1536, (3, 8, 9), 77, seed=12)

CONFIGS: Dict[int, object] = {1: ATTN_TINY, 2: ATTN_LAYER, 3: ATTN_480P, 4: ATTN_720P, 5: BLOCK_480P}


def latent_grid(frames: int, height: int, width: int,
                vae_stride=(4, 8, 8), patch=(1, 2, 2)) -> Tuple[int, int, int]:
    """Token grid of a (1+T)-frame video: causal VAE keeps the first frame, then patchify."""
    st, sh, sw = vae_stride
    pt, ph, pw = patch
    t = (1 + (frames - 1) // st) // pt
    return t, height // sh // ph, width // sw // pw


# --------------------------------------------------------------------------- draws
def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return ((bits + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Widen a stored tensor (see module doc) to float64 exactly."""
    if dtype == BF16:
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float64)


def _normal(rng: np.random.Generator, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return round_to_bf16_bits(x)
    if dtype == F32:
        return x.astype(np.float32)
    raise ValueError(dtype)


def attention_inputs(cfg: AttnConfig, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Q/K/V ~ N(0,1) for both streams, norm scales 1 + 0.1*N(0,1).

    Draw order: q_vis, k_vis, v_vis, q_cond, k_cond, v_cond, gq_vis, gk_vis, gq_cond, gk_cond.
    Shapes: tokens [B, N_s, H, D]; scales [D] (one per stream and per q/k).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    b, h, d = cfg.batch, cfg.heads, cfg.head_dim
    out = {}
    for s, n in (("vis", cfg.n_vis), ("cond", cfg.n_cond)):
        for nm in ("q", "k", "v"):
            out[f"{nm}_{s}"] = _store(_normal(rng, (b, n, h, d)), cfg.dtype)
    for s in ("vis", "cond"):
        for nm in ("gq", "gk"):
            out[f"{nm}_{s}"] = _store(_normal(rng, (d,), std=0.1, mean=1.0), cfg.dtype)
    return out


STREAM_WEIGHTS = ("w_mod", "b_mod", "w_qkv", "b_qkv", "q_norm", "k_norm",
                  "w_o", "b_o", "w_fc1", "b_fc1", "w_fc2", "b_fc2")


def stream_weight_shapes(cfg: BlockConfig) -> Dict[str, Tuple[int, ...]]:
    """nn.Linear layout [out, in].  The modulation Linear maps the shared bottleneck to six
    C-vectors (shift, scale, gate for the attention and FFN branches)."""
    c, f, dt, d = cfg.width, cfg.ffn, cfg.t_dim, cfg.head_dim
    return {"w_mod": (6 * c, dt), "b_mod": (6 * c,), "w_qkv": (3 * c, c), "b_qkv": (3 * c,),
            "q_norm": (d,), "k_norm": (d,), "w_o": (c, c), "b_o": (c,),
            "w_fc1": (f, c), "b_fc1": (f,), "w_fc2": (c, f), "b_fc2": (c,)}


def block_inputs(cfg: BlockConfig, seed: Optional[int] = None,
                 weight_std: float = 0.02) -> Dict[str, np.ndarray]:
    """Activations x ~ N(0,1), tvec ~ N(0,1); weights and biases ~ N(0, 0.02);
    QK-norm scales 1 + 0.1*N(0,1).  All bf16.

    Draw order: x_vis, x_cond, tvec, then per stream (vis, cond) the weights in
    STREAM_WEIGHTS order.  Keys of the result: ``x_vis``, ``x_cond``, ``tvec`` and
    ``vis.<w>`` / ``cond.<w>``.
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    b, c = cfg.batch, cfg.width
    out = {"x_vis": round_to_bf16_bits(_normal(rng, (b, cfg.n_vis, c))),
           "x_cond": round_to_bf16_bits(_normal(rng, (b, cfg.n_cond, c))),
           "tvec": round_to_bf16_bits(_normal(rng, (b, cfg.t_dim)))}
    shapes = stream_weight_shapes(cfg)
    for s in ("vis", "cond"):
        for nm in STREAM_WEIGHTS:
            if nm in ("q_norm", "k_norm"):
                x = _normal(rng, shapes[nm], std=0.1, mean=1.0)
            else:
                x = _normal(rng, shapes[nm], std=weight_std)
            out[f"{s}.{nm}"] = round_to_bf16_bits(x)
    return out


# --------------------------------------------------------------------------- timestep path
@dataclasses.dataclass(frozen=True)
class TimestepConfig:
    """Timestep conditioning: 256-d sinusoid -> MLP(SiLU) -> hidden -> SiLU -> Linear t_dim
    (Vimoo 1.0 notes, section 2.2; t_dim 16 in Lite, section 2.4)."""
    name: str
    batch: int
    freq_dim: int = 256
    hidden: int = 3072
    t_dim: int = 1536
    max_period: float = 10000.0
    seed: int = 0


TIMESTEP_FULL = TimestepConfig("timestep_b2_f256_h3072_dt1536", 2, t_dim=1536, seed=21)
TIMESTEP_LITE = TimestepConfig("timestep_b2_f256_h3072_dt16", 2, t_dim=16, seed=22)
TIMESTEP_WEIGHTS = ("w1", "b1", "w2", "b2", "w3", "b3")


def timestep_inputs(cfg: TimestepConfig, seed: Optional[int] = None, weight_std: float = 0.02,
                    weight_dtype: str = BF16) -> Dict[str, np.ndarray]:
    """Timesteps t = 1000 * sigmoid(N(0, 1)) (logit-normal, the training distribution the Wan
    report's reading guide gives for flow matching), stored f32; weights and biases
    ~ N(0, weight_std).  Draw order: t, then w1, b1, w2, b2, w3, b3."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    z = _normal(rng, (cfg.batch,)).astype(np.float64)
    out = {"t": (1000.0 / (1.0 + np.exp(-z))).astype(np.float32)}
    shapes = {"w1": (cfg.hidden, cfg.freq_dim), "b1": (cfg.hidden,), "w2": (cfg.hidden, cfg.hidden),
              "b2": (cfg.hidden,), "w3": (cfg.t_dim, cfg.hidden), "b3": (cfg.t_dim,)}
    for nm in TIMESTEP_WEIGHTS:
        out[nm] = _store(_normal(rng, shapes[nm], std=weight_std), weight_dtype)
    return out


# --------------------------------------------------------------------------- Lite 2x2 merge
@dataclasses.dataclass(frozen=True)
class LiteConfig:
    """Lite hidden-space 2x2 merge before the backbone and unpatchify after it (Vimoo 1.0
    notes, section 2.4) on a (T, H, W) grid of visual tokens of width C."""
    name: str
    width: int
    grid: Tuple[int, int, int]
    batch: int = 1
    seed: int = 0

    @property
    def n_full(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def merged_grid(self) -> Tuple[int, int, int]:
        t, h, w = self.grid
        return t, h // 2, w // 2

    @property
    def n_merged(self) -> int:
        t, h, w = self.merged_grid
        return t * h * w

    @property
    def flops(self) -> float:
        """Merge and unpatchify each: 2 * merged tokens * C * 4C."""
        return 2 * 2.0 * self.batch * self.n_merged * self.width * 4 * self.width


LITE_480P = LiteConfig("lite480p_c3072_grid21x30x52", 3072, (21, 30, 52), seed=31)
LITE_SMALL = LiteConfig("lite_small_c512_grid3x6x10_b2", 512, (3, 6, 10), batch=2, seed=32)


def lite_inputs(cfg: LiteConfig, seed: Optional[int] = None, weight_std: float = 0.02) -> Dict[str, np.ndarray]:
    """Hidden states x ~ N(0, 1) [B, T*H*W, C] and merged-grid states y ~ N(0, 1)
    [B, T*(H/2)*(W/2), C]; merge weights [C, 4C] + [C] and unpatchify weights [4C, C] + [4C]
    ~ N(0, weight_std).  All bf16.  Draw order: x, y, w_merge, b_merge, w_unpatch, b_unpatch."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    b, c = cfg.batch, cfg.width
    return {"x": round_to_bf16_bits(_normal(rng, (b, cfg.n_full, c))),
            "y": round_to_bf16_bits(_normal(rng, (b, cfg.n_merged, c))),
            "w_merge": round_to_bf16_bits(_normal(rng, (c, 4 * c), std=weight_std)),
            "b_merge": round_to_bf16_bits(_normal(rng, (c,), std=weight_std)),
            "w_unpatch": round_to_bf16_bits(_normal(rng, (4 * c, c), std=weight_std)),
            "b_unpatch": round_to_bf16_bits(_normal(rng, (4 * c,), std=weight_std))}


def sample_rows(n: int, k: int, seed: int) -> np.ndarray:
    """Sorted distinct row indices for sampled comparisons; always keeps the first and the
    last row (tile edges and the ragged tail)."""
    if k >= n:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    idx = rng.choice(n, size=k, replace=False)
    idx[0], idx[-1] = 0, n - 1
    return np.unique(idx)
