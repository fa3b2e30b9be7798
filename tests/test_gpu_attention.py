"""GPU parity of QK-RMSNorm + 3D RoPE and joint attention against the float64 oracle.

Workloads 1 (fp32) and 2 (bf16) are compared element by element; the 480p and 720p
workloads are compared on sampled query rows (every key is used), in the same launch
configuration the bench times.  Tolerance: max|err| / rms(oracle) <= 1e-4 (fp32) and
<= 2e-2 (bf16) per output tensor.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import video_diffusion_transformer_mmdit_amd as mm
import workloads as wl
from tests.util import TOL, assert_close, assert_close_stored, log, parity_rows, to_dev, to_host64

pytestmark = pytest.mark.gpu


def _inputs(cfg):
    raw = wl.attention_inputs(cfg)
    dev = {k: to_dev(v, cfg.dtype) for k, v in raw.items()}
    return raw, dev


def _gpu_attention(cfg, dev, out_dtype=torch.float32, qk_dtype=None, return_lse=False):
    """QK-norm/RoPE then attention.  bf16 workloads keep Q^/K^ in f16 (their range is
    bounded by the RMSNorm), fp32 workloads in f32."""
    if qk_dtype is None:
        qk_dtype = torch.float32 if cfg.dtype == wl.F32 else torch.float16
    rope = mm.Rope3D.make(cfg.grid, cfg.rope_split, cfg.rope_base)
    qv, kv = mm.qk_norm_rope(dev["q_vis"], dev["k_vis"], dev["gq_vis"], dev["gk_vis"], rope=rope,
                             eps=cfg.qk_eps, out_dtype=qk_dtype)
    qc, kc = mm.qk_norm_rope(dev["q_cond"], dev["k_cond"], dev["gq_cond"], dev["gk_cond"],
                             eps=cfg.qk_eps, out_dtype=qk_dtype)
    res = mm.joint_attention(qv, kv, dev["v_vis"], qc, kc, dev["v_cond"], out_dtype=out_dtype,
                             return_lse=return_lse)
    torch.cuda.synchronize()
    return (qv, kv, qc, kc) + tuple(res)


@pytest.mark.parametrize("cfg", [wl.ATTN_TINY, wl.ATTN_LAYER], ids=lambda c: c.name)
def test_attention_full_parity(cfg):
    log(f"attention full parity {cfg.name}")
    raw, dev = _inputs(cfg)
    f64 = {k: wl.to_f64(v, cfg.dtype) for k, v in raw.items()}
    ref = oracle.attention_block(f64, cfg.grid, cfg.qk_eps, cfg.rope_split, cfg.rope_base)
    qv, kv, qc, kc, o_v, o_c, lse = _gpu_attention(cfg, dev, return_lse=True)
    tol = TOL[cfg.dtype]
    for nm, got in (("qh_vis", qv), ("kh_vis", kv), ("qh_cond", qc), ("kh_cond", kc)):
        assert_close(nm, to_host64(got), ref[nm], tol if cfg.dtype == wl.F32 else 4e-3)
    assert_close("o_vis", to_host64(o_v), ref["o_vis"], tol)
    assert_close("o_cond", to_host64(o_c), ref["o_cond"], tol)
    # log-sum-exp of every query row, [cond | vis] order, against the oracle's normalised
    # inputs: lse = log sum_j exp(q.k_j / sqrt(D))
    kall = np.concatenate([ref["kh_cond"], ref["kh_vis"]], axis=1)[0]
    qall = np.concatenate([ref["qh_cond"], ref["qh_vis"]], axis=1)[0]
    lse_ref = np.empty((cfg.heads, qall.shape[0]))
    for h in range(cfg.heads):
        s = qall[:, h] @ kall[:, h].T / math.sqrt(cfg.head_dim)
        m = s.max(axis=1, keepdims=True)
        lse_ref[h] = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]
    got = to_host64(lse)[0]
    err = np.max(np.abs(got - lse_ref))
    log(f"  lse: max abs err {err:.3e}")
    assert err < (1e-4 if cfg.dtype == wl.F32 else 3e-2)


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg", [wl.ATTN_480P, wl.ATTN_720P], ids=lambda c: c.name)
def test_attention_sampled_parity_full_size(cfg):
    """4096 query rows of every head against the oracle: every conditioning row, and visual
    rows that include the first and last 32, a band over the last 1536 (at 480p the last
    round's items, query tiles 124-129 of heads 16-23, are split over key ranges by the
    workspace, as in the block the bench times) and seeded random rows.  Every key is used."""
    log(f"attention sampled parity {cfg.name}: generating inputs")
    raw, dev = _inputs(cfg)
    log("  GPU qk_norm_rope + joint_attention (with the split-tail workspace)")
    rope = mm.Rope3D.make(cfg.grid, cfg.rope_split, cfg.rope_base)
    qv, kv = mm.qk_norm_rope(dev["q_vis"], dev["k_vis"], dev["gq_vis"], dev["gk_vis"], rope=rope,
                             eps=cfg.qk_eps, out_dtype=torch.float16)
    qc, kc = mm.qk_norm_rope(dev["q_cond"], dev["k_cond"], dev["gq_cond"], dev["gk_cond"],
                             eps=cfg.qk_eps, out_dtype=torch.float16)
    ws = torch.empty(mm.ATTN_SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    o_v, o_c = mm.joint_attention(qv, kv, dev["v_vis"], qc, kc, dev["v_cond"], workspace=ws)
    torch.cuda.synchronize()
    rc = np.arange(cfg.n_cond)
    rv = parity_rows(cfg.n_vis, 4096 - rc.size, seed=cfg.seed + 100,
                     bands=[(cfg.n_vis - 1536, cfg.n_vis, 3)])
    log(f"  {rv.size} visual + {rc.size} conditioning rows")
    o_v_s = to_host64(o_v[:, torch.from_numpy(rv).cuda()])
    o_c_s = to_host64(o_c[:, torch.from_numpy(rc).cuda()])
    kv_h, qv_s = to_host64(kv), to_host64(qv[:, torch.from_numpy(rv).cuda()])
    del dev, qv, kv, qc, kc, o_v, o_c, ws
    torch.cuda.empty_cache()
    log("  oracle (float64) on sampled rows")
    f64 = {k: wl.to_f64(v, cfg.dtype) for k, v in raw.items()}
    del raw
    ref = oracle.attention_block(f64, cfg.grid, cfg.qk_eps, cfg.rope_split, cfg.rope_base,
                                 vis_rows=rv, cond_rows=rc)
    tol = TOL[cfg.dtype]
    assert_close("kh_vis(all rows)", kv_h, ref["kh_vis"], 4e-3)
    assert_close("qh_vis(sampled)", qv_s, ref["qh_vis"][:, rv], 4e-3)
    assert_close("o_vis(sampled)", o_v_s, ref["o_vis"], tol)
    assert_close("o_cond(all rows)", o_c_s, ref["o_cond"], tol)


def _rand(shape, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype).cuda()


def _oracle_attn(qv, kv, vv, qc, kc, vc):
    f = lambda t: to_host64(t) if t is not None else np.zeros((qv.shape[0], 0) + tuple(qv.shape[2:]))  # noqa: E731
    return oracle.joint_attention(f(qv), f(kv), f(vv), f(qc), f(kc), f(vc))


@pytest.mark.parametrize("n_vis,n_cond", [(1, 0), (0, 5), (63, 1), (64, 64), (129, 77), (200, 0), (300, 130)])
def test_attention_ragged_edges(n_vis, n_cond):
    """Tails of the 64-key and 128-query tiles, empty streams, a single token."""
    H, D = 3, 128
    qv, kv, vv = (_rand((1, n_vis, H, D), s) for s in (1, 2, 3))
    qc, kc, vc = (_rand((1, n_cond, H, D), s) for s in (4, 5, 6))
    o_v, o_c = mm.joint_attention(qv, kv, vv, qc if n_cond else None, kc if n_cond else None,
                                  vc if n_cond else None)
    torch.cuda.synchronize()
    r_v, r_c = _oracle_attn(qv, kv, vv, qc, kc, vc)
    if n_vis:
        assert_close("o_vis", to_host64(o_v), r_v, 2e-2)
    if n_cond:
        assert_close("o_cond", to_host64(o_c), r_c, 2e-2)


def test_attention_batch_and_strided_packed_rows():
    """B = 2 and Q/K/V read as views of one packed [B, N, 3, H, D] buffer."""
    B, nv, nc, H, D = 2, 150, 20, 2, 128
    pv = _rand((B, nv, 3, H, D), 7)
    pc = _rand((B, nc, 3, H, D), 8)
    o_v, o_c = mm.joint_attention(pv[:, :, 0], pv[:, :, 1], pv[:, :, 2], pc[:, :, 0], pc[:, :, 1], pc[:, :, 2])
    torch.cuda.synchronize()
    for b in range(B):
        r_v, r_c = _oracle_attn(*(t[b:b + 1].contiguous() for t in (pv[:, :, 0], pv[:, :, 1], pv[:, :, 2],
                                                                     pc[:, :, 0], pc[:, :, 1], pc[:, :, 2])))
        assert_close(f"o_vis[b={b}]", to_host64(o_v[b:b + 1]), r_v, 2e-2)
        assert_close(f"o_cond[b={b}]", to_host64(o_c[b:b + 1]), r_c, 2e-2)


def test_attention_identical_keys_give_mean_of_values_and_is_deterministic():
    nv, nc, H, D = 333, 21, 2, 128
    qv, vv = _rand((1, nv, H, D), 11), _rand((1, nv, H, D), 12)
    qc, vc = _rand((1, nc, H, D), 13), _rand((1, nc, H, D), 14)
    kv = torch.full((1, nv, H, D), 0.25, dtype=torch.bfloat16, device="cuda")
    kc = torch.full((1, nc, H, D), 0.25, dtype=torch.bfloat16, device="cuda")
    o_v, o_c = mm.joint_attention(qv, kv, vv, qc, kc, vc)
    o_v2, o_c2 = mm.joint_attention(qv, kv, vv, qc, kc, vc)
    torch.cuda.synchronize()
    mean = torch.cat([vv, vc], dim=1).double().mean(dim=1, keepdim=True).cpu().numpy()
    assert_close("o_vis vs mean(V)", to_host64(o_v), np.broadcast_to(mean, o_v.shape), 2e-2)
    assert_close("o_cond vs mean(V)", to_host64(o_c), np.broadcast_to(mean, o_c.shape), 2e-2)
    assert torch.equal(o_v, o_v2) and torch.equal(o_c, o_c2), "attention is not bitwise deterministic"


def test_attention_bf16_output_and_cond_permutation():
    nv, nc, H, D = 260, 40, 2, 128
    qv, kv, vv = (_rand((1, nv, H, D), s) for s in (21, 22, 23))
    qc, kc, vc = (_rand((1, nc, H, D), s) for s in (24, 25, 26))
    o_v, o_c = mm.joint_attention(qv, kv, vv, qc, kc, vc, out_dtype=torch.bfloat16)
    perm = torch.randperm(nc, generator=torch.Generator().manual_seed(3)).cuda()
    o_v2, o_c2 = mm.joint_attention(qv, kv, vv, qc[:, perm].contiguous(), kc[:, perm].contiguous(),
                                    vc[:, perm].contiguous(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    r_v, r_c = _oracle_attn(qv, kv, vv, qc, kc, vc)
    assert_close("o_vis bf16", to_host64(o_v), r_v, 2e-2)
    assert_close("o_cond bf16", to_host64(o_c), r_c, 2e-2)
    assert_close("o_vis permuted cond", to_host64(o_v2), r_v, 2e-2)
    assert_close("o_cond permuted", to_host64(o_c2), r_c[:, perm.cpu().numpy()], 2e-2)


def test_qk_norm_rope_in_place_matches_out_of_place_and_per_head_scales():
    cfg = wl.ATTN_LAYER
    raw, dev = _inputs(cfg)
    H = cfg.heads
    rope = mm.Rope3D.make(cfg.grid)
    qkv = torch.stack([dev["q_vis"], dev["k_vis"], dev["v_vis"]], dim=2)   # [1, N, 3, H, D]
    gq = _rand((H, 128), 31, torch.float32) * 0.1 + 1
    gk = _rand((H, 128), 32, torch.float32) * 0.1 + 1
    qo, ko = mm.qk_norm_rope(qkv[:, :, 0], qkv[:, :, 1], gq, gk, rope=rope)   # bf16 out
    mm.qk_norm_rope(qkv[:, :, 0], qkv[:, :, 1], gq, gk, rope=rope, q_out=qkv[:, :, 0], k_out=qkv[:, :, 1])
    torch.cuda.synchronize()
    assert torch.equal(qo, qkv[:, :, 0]) and torch.equal(ko, qkv[:, :, 1])
    assert torch.equal(qkv[:, :, 2], dev["v_vis"]), "V must be untouched"
    f64 = lambda k: wl.to_f64(raw[k], cfg.dtype)  # noqa: E731
    rq, rk = oracle.qk_norm_rope(f64("q_vis"), f64("k_vis"), to_host64(gq), to_host64(gk), cfg.qk_eps, cfg.grid)
    assert_close_stored("q^ per-head scales", to_host64(qo), rq, torch.bfloat16, 1e-4)
    assert_close_stored("k^ per-head scales", to_host64(ko), rk, torch.bfloat16, 1e-4)


def test_qk_norm_rope_f32_out_tight():
    """bf16 in, f32 out: only the fp32 arithmetic separates it from the oracle."""
    cfg = wl.ATTN_LAYER
    raw, dev = _inputs(cfg)
    rope = mm.Rope3D.make(cfg.grid)
    qo, ko = mm.qk_norm_rope(dev["q_vis"], dev["k_vis"], dev["gq_vis"], dev["gk_vis"], rope=rope,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    f64 = lambda k: wl.to_f64(raw[k], cfg.dtype)  # noqa: E731
    rq, rk = oracle.qk_norm_rope(f64("q_vis"), f64("k_vis"), f64("gq_vis"), f64("gk_vis"), cfg.qk_eps, cfg.grid)
    assert_close("q^ f32", to_host64(qo), rq, 1e-5)
    assert_close("k^ f32", to_host64(ko), rk, 1e-5)


def test_invalid_arguments_raise_before_launch():
    q = _rand((1, 8, 2, 128), 1)
    g = torch.ones(128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mm.MmditError, match="N != T"):
        mm.qk_norm_rope(q, q.clone(), g, g, rope=mm.Rope3D.make((2, 2, 3)))
    with pytest.raises(mm.MmditError, match="d_t"):
        mm.qk_norm_rope(q, q.clone(), g, g, rope=mm.Rope3D.make((2, 2, 2), (16, 56, 54)))
    with pytest.raises(mm.MmditError, match="overlap"):
        mm.joint_attention(q, q, q, out_dtype=torch.bfloat16, o_vis=q)
    with pytest.raises(mm.MmditError, match="f16 / bf16"):
        mm.joint_attention(q, q, q.float())


@pytest.mark.parametrize("qk,v", [(torch.float16, torch.float16), (torch.bfloat16, torch.bfloat16),
                                  (torch.bfloat16, torch.float16), (torch.float16, torch.bfloat16)])
def test_attention_operand_dtype_combinations(qk, v):
    """Every Q/K x V operand type pair on ragged sizes (V in bf16 is converted to f16 on its
    way into LDS; P V always runs on f16)."""
    nv, nc, H, D = 190, 33, 2, 128
    qv, kv = _rand((1, nv, H, D), 41, qk), _rand((1, nv, H, D), 42, qk)
    qc, kc = _rand((1, nc, H, D), 43, qk), _rand((1, nc, H, D), 44, qk)
    vv, vc = _rand((1, nv, H, D), 45, v), _rand((1, nc, H, D), 46, v)
    o_v, o_c = mm.joint_attention(qv, kv, vv, qc, kc, vc)
    torch.cuda.synchronize()
    r_v, r_c = _oracle_attn(qv, kv, vv, qc, kc, vc)
    assert_close("o_vis", to_host64(o_v), r_v, 1e-2)
    assert_close("o_cond", to_host64(o_c), r_c, 1e-2)


def test_attention_split_tail_with_workspace():
    """B = 2, 24 heads, 1400 + 77 tokens: 288 (batch x head, query tile) items leave 32 for the
    last round, which a workspace lets the kernel cut into 8 key ranges each and merge.  The
    output matches the oracle at the 16-bit bar and the same call without a workspace to
    within the f16 rounding of P (each range rounds exp2 against its own running max)."""
    B, nv, nc, H, D = 2, 1400, 77, 24, 128
    qv, kv, vv = (_rand((B, nv, H, D), s) for s in (11, 12, 13))
    qc, kc, vc = (_rand((B, nc, H, D), s) for s in (14, 15, 16))
    ws = torch.empty(mm.ATTN_SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    o_v, o_c = mm.joint_attention(qv, kv, vv, qc, kc, vc, workspace=ws)
    u_v, u_c = mm.joint_attention(qv, kv, vv, qc, kc, vc)
    torch.cuda.synchronize()
    assert_close("o_vis split vs one pass", to_host64(o_v), to_host64(u_v), 5e-3)
    assert_close("o_cond split vs one pass", to_host64(o_c), to_host64(u_c), 5e-3)
    for b in range(B):
        r_v, r_c = _oracle_attn(*(t[b:b + 1].contiguous() for t in (qv, kv, vv, qc, kc, vc)))
        assert_close(f"o_vis[b={b}]", to_host64(o_v[b:b + 1]), r_v, 2e-2)
        assert_close(f"o_cond[b={b}]", to_host64(o_c[b:b + 1]), r_c, 2e-2)


@pytest.mark.parametrize("dt", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("split", [False, True], ids=["one_pass", "split_tail"])
def test_logits_far_above_the_running_max(dt, split):
    """Keys in later tiles whose logits lie far above everything before them: about 10 log2
    units (weights up to ~2^8 above the first tile's max, kept without raising it), then about
    20, 40 and 69 (in a middle visual tile, the partial last visual tile and the conditioning
    segment), each of which passes the f16-safe bound of its tile.  A tile
    whose weights would pass that bound raises the running max and is weighed again;
    the output stays finite and matches the oracle, for f16 Q (scaled before the product)
    and bf16 Q (scaled at the exponential), in one pass and with the split tail's key ranges
    (B = 2, 24 heads, 1400 + 77 tokens: 32 items of the last round in 8 ranges each)."""
    B, nv, nc, H, D = 2, 1400, 77, 24, 128
    g = torch.Generator().manual_seed(71)
    u = torch.randn((H, D), generator=g)
    q = lambda n: u + 0.5 * torch.randn((B, n, H, D), generator=g)  # noqa: E731
    k = lambda n: 0.5 * torch.randn((B, n, H, D), generator=g)  # noqa: E731
    qv, qc, kv, kc = q(nv), q(nc), k(nv), k(nc)
    unit = u / math.sqrt(D)   # q . (lam * unit) / sqrt(D) is about lam nats
    for rows, at, lam in ((kv, 150, 7.0), (kv, 300, 14.0), (kv, 1395, 28.0), (kc, 40, 48.0)):
        rows[:, at] = lam * unit
    vv = torch.randn((B, nv, H, D), generator=g)
    vc = torch.randn((B, nc, H, D), generator=g)
    qv, kv, vv, qc, kc, vc = (t.to(dt).cuda() for t in (qv, kv, vv, qc, kc, vc))
    ws = torch.empty(mm.ATTN_SPLIT_BYTES, dtype=torch.uint8, device="cuda") if split else None
    o_v, o_c = mm.joint_attention(qv, kv, vv, qc, kc, vc, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o_v).all() and torch.isfinite(o_c).all()
    for b in range(B):
        r_v, r_c = _oracle_attn(*(t[b:b + 1].contiguous() for t in (qv, kv, vv, qc, kc, vc)))
        assert_close(f"o_vis[b={b}]", to_host64(o_v[b:b + 1]), r_v, 2e-2)
        assert_close(f"o_cond[b={b}]", to_host64(o_c[b:b + 1]), r_c, 2e-2)


def test_host_workspace_or_output_raises_before_launch():
    """GPU inputs with a host workspace (or a host output) are refused by the binding."""
    q = _rand((1, 300, 2, 128), 51)
    host_ws = torch.empty(mm.ATTN_SPLIT_BYTES, dtype=torch.uint8)
    with pytest.raises(mm.MmditError, match="workspace must be a GPU tensor"):
        mm.joint_attention(q, q, q, workspace=host_ws)
    with pytest.raises(mm.MmditError, match="o_vis must be a GPU tensor"):
        mm.joint_attention(q, q, q, o_vis=torch.empty((1, 300, 2, 128)))
    ops = mm.attn8_quantize(q, q, q)
    with pytest.raises(mm.MmditError, match="workspace must be a GPU tensor"):
        mm.joint_attention_8bit(ops, workspace=host_ws)
    with pytest.raises(mm.MmditError, match="o_vis must be a GPU tensor"):
        mm.joint_attention_8bit(ops, o_vis=torch.empty((1, 300, 2, 128)))
    torch.cuda.synchronize()


@pytest.mark.parametrize("B,n_vis,n_cond", [(1, 1000, 77), (2, 333, 5), (1, 64, 0)])
def test_nan_rows_past_each_segment_are_never_read(B, n_vis, n_cond):
    """Q/K/V of each stream are views of buffers whose rows past the segment (and past the last
    batch item) are NaN: the kernels' partial tiles must take zeros there (their loads stop at
    the segment's end), so every output is finite and matches the oracle.  The 8-bit path's
    quantizer and attention read the same views."""
    H, D, pad = 3, 128, 300
    def padded(n, seed):
        full = torch.full((B * n + pad, 3, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
        full[:B * n] = _rand((B * n, 3, H, D), seed)
        return full[:B * n].view(B, n, 3, H, D)
    pv, pc = padded(n_vis, 61), padded(n_cond, 62)
    qv, kv, vv = pv[:, :, 0], pv[:, :, 1], pv[:, :, 2]
    qc, kc, vc = (pc[:, :, 0], pc[:, :, 1], pc[:, :, 2]) if n_cond else (None, None, None)
    ws = torch.empty(mm.ATTN_SPLIT_BYTES, dtype=torch.uint8, device="cuda")
    o_v, o_c = mm.joint_attention(qv, kv, vv, qc, kc, vc, workspace=ws)
    ops = mm.attn8_quantize(qv, kv, vv, qc, kc, vc)
    e_v, e_c = mm.joint_attention_8bit(ops, workspace=ws)
    torch.cuda.synchronize()
    for nm, t in (("o_vis", o_v), ("o_cond", o_c), ("o8_vis", e_v), ("o8_cond", e_c)):
        if t is not None and t.numel():
            assert torch.isfinite(t).all(), f"{nm}: non-finite output (a padding row was read)"
    for b in range(B):
        f = lambda t: to_host64(t[b:b + 1]) if t is not None else np.zeros((1, 0, H, D))  # noqa: E731
        r_v, r_c = oracle.joint_attention(f(qv), f(kv), f(vv), f(qc), f(kc), f(vc))
        assert_close(f"o_vis[b={b}]", f(o_v), r_v, 2e-2)
        if n_cond:
            assert_close(f"o_cond[b={b}]", f(o_c), r_c, 2e-2)
