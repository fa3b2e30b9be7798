"""Loop-based pure-Python recomputation of the block for tiny inputs.

Independent of ``oracle/``: written from the definitions in the Vimoo 1.0 notes
(section 2.2) with plain Python floats and the ``math`` module only (no numpy), so a
mistake in the vectorised oracle (a wrong axis, a transposed weight, a swapped band)
shows up as a mismatch.  Tensors are nested lists.
"""
import math


def decode_position(n, grid):
    """Visual token index -> (t, h, w), w fastest."""
    _, hh, ww = grid
    t = n // (hh * ww)
    rem = n - t * hh * ww
    return t, rem // ww, rem % ww


def pair_angle(pair, pos, split, base):
    """Angle of rotation pair ``pair`` (0 .. D/2-1) for a token at ``pos`` = (t, h, w)."""
    start = 0
    for axis in range(3):
        width = split[axis]
        if 2 * pair < start + width:
            j = pair - start // 2
            return pos[axis] * base ** (-(2.0 * j) / width)
        start += width
    raise ValueError("pair out of range")


def rmsnorm_vec(x, g, eps):
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r * gg for v, gg in zip(x, g)]


def rope_vec(x, pos, split, base):
    out = list(x)
    for p in range(len(x) // 2):
        a = pair_angle(p, pos, split, base)
        c, s = math.cos(a), math.sin(a)
        x0, x1 = x[2 * p], x[2 * p + 1]
        out[2 * p] = x0 * c - x1 * s
        out[2 * p + 1] = x0 * s + x1 * c
    return out


def attention_rows(qs, ks, vs, scale):
    """qs: list of query vectors; ks, vs: lists of key / value vectors (one head)."""
    outs = []
    for q in qs:
        logits = [scale * sum(a * b for a, b in zip(q, k)) for k in ks]
        m = max(logits)
        w = [math.exp(l - m) for l in logits]
        z = sum(w)
        d = len(vs[0])
        outs.append([sum(w[j] * vs[j][i] for j in range(len(vs))) / z for i in range(d)])
    return outs


def attention_block(q_vis, k_vis, v_vis, q_cond, k_cond, v_cond, gq_vis, gk_vis, gq_cond, gk_cond,
                    grid, eps, split=(16, 56, 56), base=10000.0):
    """Per-head lists: x[n][h] is a D-vector.  Returns (o_vis, o_cond) as nested lists."""
    n_vis, n_cond = len(q_vis), len(q_cond)
    heads = len(q_vis[0]) if n_vis else len(q_cond[0])
    d = len(q_vis[0][0]) if n_vis else len(q_cond[0][0])
    scale = 1.0 / math.sqrt(d)
    o_vis = [[None] * heads for _ in range(n_vis)]
    o_cond = [[None] * heads for _ in range(n_cond)]
    for h in range(heads):
        qv, kv, qc, kc = [], [], [], []
        for n in range(n_vis):
            pos = decode_position(n, grid)
            qv.append(rope_vec(rmsnorm_vec(q_vis[n][h], gq_vis, eps), pos, split, base))
            kv.append(rope_vec(rmsnorm_vec(k_vis[n][h], gk_vis, eps), pos, split, base))
        for n in range(n_cond):
            qc.append(rmsnorm_vec(q_cond[n][h], gq_cond, eps))
            kc.append(rmsnorm_vec(k_cond[n][h], gk_cond, eps))
        # keys in visual-then-conditioning order (the opposite of the oracle's choice)
        keys = kv + kc
        vals = [v_vis[n][h] for n in range(n_vis)] + [v_cond[n][h] for n in range(n_cond)]
        for n, o in enumerate(attention_rows(qv, keys, vals, scale)):
            o_vis[n][h] = o
        for n, o in enumerate(attention_rows(qc, keys, vals, scale)):
            o_cond[n][h] = o
    return o_vis, o_cond


def matvec(w, x, b):
    """w: list of rows [out][in]; returns w x + b."""
    return [sum(wi * xi for wi, xi in zip(row, x)) + bb for row, bb in zip(w, b)]


def layernorm_vec(x, eps):
    mu = sum(x) / len(x)
    var = sum((v - mu) ** 2 for v in x) / len(x)
    r = 1.0 / math.sqrt(var + eps)
    return [(v - mu) * r for v in x]


def gelu(x):
    return 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))


def block_forward(x_vis, x_cond, tvec, w_vis, w_cond, grid, heads, ln_eps, qk_eps,
                  split=(16, 56, 56), base=10000.0):
    """x_*: [N][C] lists; tvec: [Dt] list; w_*: dict of nested lists (nn.Linear [out][in])."""
    c = len(x_vis[0]) if x_vis else len(x_cond[0])
    d = c // heads
    streams = {"vis": (x_vis, w_vis), "cond": (x_cond, w_cond)}
    mod, qkv = {}, {}
    for s, (x, w) in streams.items():
        m = matvec(w["w_mod"], tvec, w["b_mod"])
        mod[s] = [m[i * c:(i + 1) * c] for i in range(6)]
        shift_a, scale_a = mod[s][0], mod[s][1]
        rows = []
        for xt in x:
            hn = layernorm_vec(xt, ln_eps)
            hm = [v * (1.0 + sc) + sh for v, sc, sh in zip(hn, scale_a, shift_a)]
            rows.append(matvec(w["w_qkv"], hm, w["b_qkv"]))
        qkv[s] = rows

    def split_heads(rows, part):
        return [[r[part * c + h * d: part * c + (h + 1) * d] for h in range(heads)] for r in rows]

    o_vis, o_cond = attention_block(
        split_heads(qkv["vis"], 0), split_heads(qkv["vis"], 1), split_heads(qkv["vis"], 2),
        split_heads(qkv["cond"], 0), split_heads(qkv["cond"], 1), split_heads(qkv["cond"], 2),
        w_vis["q_norm"], w_vis["k_norm"], w_cond["q_norm"], w_cond["k_norm"],
        grid, qk_eps, split, base)
    outs = {}
    for s, o_s in (("vis", o_vis), ("cond", o_cond)):
        x, w = streams[s]
        _, _, gate_a, shift_f, scale_f, gate_f = mod[s]
        res = []
        for xt, oh in zip(x, o_s):
            o = [v for head in oh for v in head]
            a = matvec(w["w_o"], o, w["b_o"])
            x1 = [xv + g * av for xv, g, av in zip(xt, gate_a, a)]
            hn = layernorm_vec(x1, ln_eps)
            h2 = [v * (1.0 + sc) + sh for v, sc, sh in zip(hn, scale_f, shift_f)]
            f = [gelu(v) for v in matvec(w["w_fc1"], h2, w["b_fc1"])]
            y = matvec(w["w_fc2"], f, w["b_fc2"])
            res.append([xv + g * yv for xv, g, yv in zip(x1, gate_f, y)])
        outs[s] = res
    return outs["vis"], outs["cond"]


# ------------------------------------------------------------------ timestep path, Lite merge
def sinusoid_vec(t, dim, max_period=10000.0):
    """One timestep's embedding: entry i < dim/2 is cos(t * f_i), entry dim/2 + i is
    sin(t * f_i), with f_i = max_period ** (-i / (dim/2))."""
    half = dim // 2
    out = [0.0] * dim
    for i in range(half):
        f = max_period ** (-i / half)
        out[i] = math.cos(t * f)
        out[half + i] = math.sin(t * f)
    return out


def silu_scalar(x):
    return x / (1.0 + math.exp(-x)) if x > -700 else 0.0


def timestep_path(t, w1, b1, w2, b2, w3, b3, dim, max_period=10000.0):
    """Returns (hidden, temb, tvec) lists for one timestep value."""
    hidden = matvec(w1, sinusoid_vec(t, dim, max_period), b1)
    temb = matvec(w2, [silu_scalar(v) for v in hidden], b2)
    tvec = matvec(w3, [silu_scalar(v) for v in temb], b3)
    return hidden, temb, tvec


def lite_merge(x, w, b, grid):
    """x: [T*H*W][C] lists (w fastest).  Merged token (t, i, j) reads the four tokens
    (t, 2i+dh, 2j+dw), (dh, dw) in row-major order, side by side, then w [C][4C] + b."""
    tt, hh, ww = grid
    out = []
    for t in range(tt):
        for i in range(hh // 2):
            for j in range(ww // 2):
                cat = []
                for dh in range(2):
                    for dw in range(2):
                        cat += x[(t * hh + 2 * i + dh) * ww + 2 * j + dw]
                out.append(matvec(w, cat, b))
    return out


def lite_unpatchify(y, w, b, grid):
    """y: [T*(H/2)*(W/2)][C]; w [4C][C].  Token (t, h, w) of the output takes part
    (h % 2) * 2 + (w % 2) of merged token (t, h // 2, w // 2)'s expansion."""
    tt, hh, ww = grid
    c = len(y[0])
    out = []
    for t in range(tt):
        for h in range(hh):
            for x_ in range(ww):
                m = (t * (hh // 2) + h // 2) * (ww // 2) + x_ // 2
                z = matvec(w, y[m], b)
                part = (h % 2) * 2 + (x_ % 2)
                out.append(z[part * c:(part + 1) * c])
    return out


# ------------------------------------------------------------------ FP8 linear
def fp8_linear(x, w, b, round_fp8):
    """x: [M][K], w: [N][K] lists; ``round_fp8`` rounds one float to E4M3 (an independent
    routine is passed in).  Per-row scales of x and one scale of w: amax / 448 in float32,
    values scaled by the float32 reciprocal, rounded, multiplied exactly, rescaled."""
    import numpy as np
    f32 = np.float32

    def quant(rows):
        amax = f32(max(abs(f32(v)) for r in rows for v in r))
        s = f32(amax / f32(448.0)) if amax > 0 else f32(1.0)
        inv = f32(f32(1.0) / s)
        return [[round_fp8(float(min(max(f32(f32(v) * inv), f32(-448.0)), f32(448.0)))) for v in r] for r in rows], float(s)

    qw, sw = quant(w)
    out = []
    for r in x:
        (qr,), sr = quant([r])
        out.append([sum(a * c for a, c in zip(qr, wr)) * sr * sw + bb for wr, bb in zip(qw, b)])
    return out


# ------------------------------------------------------------------ 8-bit joint attention
def attention_8bit(q_rows, k_rows, v_rows, seg_of_key, scale, round_fp8):
    """One head, loops only.  q_rows: list of (vector, stream) queries; k_rows / v_rows: key
    and value vectors in any order, seg_of_key[j] = (stream, position in that stream).
    INT8: one scale per query row, one per 64-key block of a stream; V: one E4M3 scale per
    channel over all keys.  Scales amax / qmax in float32, codes from x * (1/s) in float32.
    Logits in log2 units acc * s_q * s_k * scale * log2(e) as python floats; reference M =
    ceil of the row's max; weights 2^(logit - M + 8) rounded to E4M3; O = sum P V / sum P."""
    import numpy as np
    f32 = np.float32

    def scale_of(vals, qmax):
        amax = f32(max(abs(f32(v)) for v in vals))
        return f32(amax / f32(qmax)) if amax > 0 else f32(1.0)

    def int8(v, s):
        inv = f32(f32(1.0) / s)
        return [int(max(-127.0, min(127.0, float(np.rint(f32(f32(x) * inv)))))) for x in v]

    # key block scales per (stream, block)
    blocks = {}
    for j, (sg, pos) in enumerate(seg_of_key):
        blocks.setdefault((sg, pos // 64), []).extend(k_rows[j])
    ks = {key: scale_of(vals, 127.0) for key, vals in blocks.items()}
    k8 = [int8(k_rows[j], ks[(sg, pos // 64)]) for j, (sg, pos) in enumerate(seg_of_key)]
    d = len(v_rows[0])
    sv = [scale_of([v_rows[j][c] for j in range(len(v_rows))], 448.0) for c in range(d)]
    v8 = [[round_fp8(float(min(max(f32(f32(v_rows[j][c]) * f32(f32(1.0) / sv[c])), f32(-448)), f32(448))))
           for c in range(d)] for j in range(len(v_rows))]
    kc = float(scale) * math.log2(math.e)
    outs = []
    for qv, _ in q_rows:
        sq = scale_of(qv, 127.0)
        q8 = int8(qv, sq)
        y = []
        for j, (sg, pos) in enumerate(seg_of_key):
            acc = sum(a * b for a, b in zip(q8, k8[j]))                  # python int, exact
            y.append(acc * float(sq) * float(ks[(sg, pos // 64)]) * kc)
        m = math.ceil(max(y))
        p = [round_fp8(2.0 ** (yj + 8 - m)) for yj in y]
        ell = sum(p)
        outs.append([sum(p[j] * v8[j][c] for j in range(len(p))) * float(sv[c]) / ell for c in range(d)])
    return outs


# ------------------------------------------------------------------ 8-bit block
def f16_scalar(v):
    """v rounded to IEEE binary16 through the struct module's half-precision packing."""
    import struct
    return struct.unpack("<e", struct.pack("<e", v))[0]


def block_forward_8bit(x_vis, x_cond, tvec, w_vis, w_cond, grid, heads, ln_eps, qk_eps, round_fp8,
                       split=(16, 56, 56), base=10000.0):
    """The 8-bit block with loops: the block's steps with every Linear the FP8 Linear above
    (weights quantized once per matrix, activations per row) and the attention the 8-bit
    attention above, per head; h, q^ / k^ / v, O, h2 and the GELU output rounded to binary16
    before they are quantized.  Same arguments as block_forward plus ``round_fp8``."""
    c = len(x_vis[0]) if x_vis else len(x_cond[0])
    d = c // heads
    h16 = lambda rows: [[f16_scalar(v) for v in r] for r in rows]  # noqa: E731
    streams = {"vis": (x_vis, w_vis), "cond": (x_cond, w_cond)}
    mod, heads_qkv = {}, {}
    for s, (x, w) in streams.items():
        m = matvec(w["w_mod"], tvec, w["b_mod"])
        mod[s] = [m[i * c:(i + 1) * c] for i in range(6)]
        shift_a, scale_a = mod[s][0], mod[s][1]
        hrows = [[v * (1.0 + sc) + sh for v, sc, sh in zip(layernorm_vec(xt, ln_eps), scale_a, shift_a)] for xt in x]
        qkv = h16(fp8_linear(h16(hrows), w["w_qkv"], w["b_qkv"], round_fp8)) if x else []
        heads_qkv[s] = qkv
    per_head = {}
    for hd in range(heads):
        qs, keys, vals, seg = [], [], [], []
        for s, gq, gk in (("vis", w_vis["q_norm"], w_vis["k_norm"]), ("cond", w_cond["q_norm"], w_cond["k_norm"])):
            for n, r in enumerate(heads_qkv[s]):
                q = rmsnorm_vec(r[hd * d:(hd + 1) * d], gq, qk_eps)
                k = rmsnorm_vec(r[c + hd * d:c + (hd + 1) * d], gk, qk_eps)
                if s == "vis":
                    pos = decode_position(n, grid)
                    q, k = rope_vec(q, pos, split, base), rope_vec(k, pos, split, base)
                qs.append(([f16_scalar(v) for v in q], 0 if s == "vis" else 1))
                keys.append([f16_scalar(v) for v in k])
                vals.append(r[2 * c + hd * d:2 * c + (hd + 1) * d])
                seg.append((0 if s == "vis" else 1, n))
        per_head[hd] = attention_8bit(qs, keys, vals, seg, 1.0 / math.sqrt(d), round_fp8)
    outs = {}
    base_row = {"vis": 0, "cond": len(x_vis)}
    for s, (x, w) in streams.items():
        _, _, gate_a, shift_f, scale_f, gate_f = mod[s]
        if not x:
            outs[s] = []
            continue
        o_rows = h16([[v for hd in range(heads) for v in per_head[hd][base_row[s] + n]] for n in range(len(x))])
        a = fp8_linear(o_rows, w["w_o"], w["b_o"], round_fp8)
        x1 = [[xv + g * av for xv, g, av in zip(xt, gate_a, ar)] for xt, ar in zip(x, a)]
        h2 = h16([[v * (1.0 + sc) + sh for v, sc, sh in zip(layernorm_vec(r, ln_eps), scale_f, shift_f)] for r in x1])
        g = h16([[gelu(v) for v in r] for r in fp8_linear(h2, w["w_fc1"], w["b_fc1"], round_fp8)])
        y = fp8_linear(g, w["w_fc2"], w["b_fc2"], round_fp8)
        outs[s] = [[xv + gg * yv for xv, gg, yv in zip(r, gate_f, yr)] for r, yr in zip(x1, y)]
    return outs["vis"], outs["cond"]
