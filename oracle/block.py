"""Oracle: one dual-stream NR-MMDiT block and its conditioning (test
infrastructure only).  float64 throughout; a matmul is the only library
primitive used for contractions.

What the pages fix: the backbone is a multimodal diffusion transformer in
which text and image tokens keep their own projections and norms but attend
jointly (blog close-reading, 5 "MMDiT"); attention is confined to each packed
sample (blog close-reading, 2.2(2)); each sample keeps its own 2D RoPE and
editing adds a frame axis (hyper.ai 2607.19064, 方法; blog close-reading,
2.2(2)); the fused chains are norm, RoPE, gating and residual, and fusion must
not change the model function (blog close-reading, 2.2(3)).

Everything else is a reading where the pages are silent:
  R7   RoPE: theta = 10000, bands (frame, row, col) of widths (d/4, 3d/8,
       3d/8), adjacent dimensions (2j, 2j+1) form a pair, angle of pair j in
       a band of width d_a is pos * theta**(-2j/d_a), rotation
       (x, y) -> (x cos - y sin, x sin + y cos).
  R8   pre-norm is RMSNorm without gain, eps = 1e-6.
  R9   QK-norm is RMSNorm over head_dim with a per-stream gain, before RoPE.
  R10  adaLN: W_mod maps SiLU(c) to six H-vectors in the order (shift1,
       scale1, gate1, shift2, scale2, gate2); modulate(n) = n*(1+scale)+shift.
  R11  timestep embedding: 256 dims, [cos(1000 t f_k), sin(1000 t f_k)],
       f_k = 10000**(-k/128); c = W_t2 SiLU(W_t1 emb).
  R12  all linear maps are bias-free and use y = x W^T with W [out, in].
  R13  GELU is the exact erf form.
  R14  attention: scale 1/sqrt(d), non-causal, joint over [text; image] of a
       sample; QKV columns are [Q | K | V], each head-contiguous.
  R15  final layer: adaLN (shift, scale) + RMSNorm + W_out on target rows.
  R24  image tokens enter through W_in [H, C]; text features through
       W_txt [H, H].
"""

import math

import numpy as np
from scipy.special import erf as _sp_erf

EPS = 1e-6
THETA = 10000.0
T_DIM = 256


# ---------------------------------------------------------------- primitives

def rms_norm(x, eps=EPS):
    """x / sqrt(mean(x^2) + eps) over the last axis (R8)."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def modulate(n, shift, scale):
    """adaLN modulation n*(1+scale)+shift (R10)."""
    return n * (1.0 + scale) + shift


def silu(x):
    return x / (1.0 + np.exp(-x))


def gelu(x):
    """Exact GELU, 0.5 x (1 + erf(x / sqrt 2)) (R13); erf from scipy.special."""
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + _sp_erf(x / math.sqrt(2.0)))


def linear(x, w):
    """y = x W^T with W stored [out, in] (R12)."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


# ------------------------------------------------------------- conditioning

def timestep_embedding(t, dim=T_DIM):
    """Sinusoidal embedding of t in [0, 1] (R11): [cos(1000 t f), sin(1000 t f)]."""
    t = np.asarray(t, np.float64).reshape(-1)
    half = dim // 2
    freqs = np.array([THETA ** (-k / half) for k in range(half)])
    arg = 1000.0 * t[:, None] * freqs[None, :]
    return np.concatenate([np.cos(arg), np.sin(arg)], axis=1)


def cond(t, w_t1, w_t2):
    """Per-sample conditioning vector c [B, H] = W_t2 SiLU(W_t1 emb(t)) (R11)."""
    return linear(silu(linear(timestep_embedding(t, np.asarray(w_t1).shape[1]), w_t1)), w_t2)


def modulation(c, w_mod, chunks=6):
    """adaLN vectors from c (R10): returns a list of `chunks` arrays [B, H]."""
    m = linear(silu(c), w_mod)
    return np.split(m, chunks, axis=1)


# ---------------------------------------------------------------------- RoPE

def rope_bands(head_dim):
    """Band widths (frame, row, col) of R7."""
    if head_dim % 8:
        raise ValueError("head_dim must be a multiple of 8")
    return (head_dim // 4, 3 * head_dim // 8, 3 * head_dim // 8)


def rope_angles(pos, head_dim, theta=THETA, bands=None):
    """Angle of every rotation pair [n, head_dim/2] for positions pos [n, 3] (R7).

    bands: the (frame, row, col) band widths, default R7's.
    """
    pos = np.asarray(pos, np.float64).reshape(-1, 3)
    bands = rope_bands(head_dim) if bands is None else tuple(bands)
    if sum(bands) != head_dim or any(b % 2 for b in bands):
        raise ValueError("band widths must be even and sum to head_dim")
    cols = []
    for axis, width in enumerate(bands):
        for j in range(width // 2):
            cols.append(pos[:, axis] * theta ** (-2.0 * j / width))
    return np.stack(cols, axis=1)


def apply_rope(x, pos, theta=THETA, bands=None):
    """Rotate pairs (2j, 2j+1) of every head of x [n, heads, d] (R7)."""
    x = np.asarray(x, np.float64)
    ang = rope_angles(pos, x.shape[-1], theta, bands)[:, None, :]      # [n, 1, d/2]
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * np.cos(ang) - xo * np.sin(ang)
    out[..., 1::2] = xe * np.sin(ang) + xo * np.cos(ang)
    return out


# ----------------------------------------------------------------- attention

def attention(q, k, v, q_chunk=1024):
    """softmax(q k^T / sqrt(d)) v over one sample, per head (R14).

    q [Lq, heads, d], k and v [L, heads, d].  Queries are processed in chunks so
    a long sample never holds an Lq x L score matrix; each chunk is the plain
    definition.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    d = q.shape[-1]
    out = np.empty((q.shape[0], q.shape[1], v.shape[2]))
    kh = k.transpose(1, 2, 0)                                    # [heads, d, L]
    vh = v.transpose(1, 0, 2)                                    # [heads, L, d]
    for s in range(0, q.shape[0], q_chunk):
        qh = q[s:s + q_chunk].transpose(1, 0, 2)                 # [heads, c, d]
        logits = (qh @ kh) / math.sqrt(d)
        logits -= logits.max(axis=-1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=-1, keepdims=True)
        out[s:s + q_chunk] = (p @ vh).transpose(1, 0, 2)
    return out


def packed_attention(q_txt, k_txt, v_txt, q_img, k_img, v_img, pk):
    """Block-diagonal joint attention over a pack (blog close-reading, 2.2(2)).

    Every sample b attends over its own [text_b; image_b] tokens only.  Inputs
    are modality-major [n, heads, d]; outputs are (o_txt, o_img) likewise.
    """
    o_txt = np.zeros(np.shape(q_txt))
    o_img = np.zeros(np.shape(q_img))
    for b in range(pk["B"]):
        t0, t1 = pk["cu_txt"][b], pk["cu_txt"][b + 1]
        i0, i1 = pk["cu_img"][b], pk["cu_img"][b + 1]
        q = np.concatenate([q_txt[t0:t1], q_img[i0:i1]])
        k = np.concatenate([k_txt[t0:t1], k_img[i0:i1]])
        v = np.concatenate([v_txt[t0:t1], v_img[i0:i1]])
        o = attention(q, k, v)
        o_txt[t0:t1] = o[:t1 - t0]
        o_img[i0:i1] = o[t1 - t0:]
    return o_txt, o_img


# --------------------------------------------------------------------- block

STREAM_KEYS = ("w_mod", "w_qkv", "g_q", "g_k", "w_o", "w_up", "w_down")


def _stream_pre_attn(x, seg, mod, w, heads, pos):
    """Per-token work before attention for one stream: (h, qkv, q, k, v)."""
    shift1, scale1 = mod[0][seg], mod[1][seg]
    h = modulate(rms_norm(x), shift1, scale1)
    qkv = linear(h, w["w_qkv"])
    H = x.shape[1]
    d = H // heads
    q = qkv[:, :H].reshape(-1, heads, d)
    k = qkv[:, H:2 * H].reshape(-1, heads, d)
    v = qkv[:, 2 * H:].reshape(-1, heads, d)
    q = rms_norm(q) * np.asarray(w["g_q"], np.float64)
    k = rms_norm(k) * np.asarray(w["g_k"], np.float64)
    q = apply_rope(q, pos)
    k = apply_rope(k, pos)
    return h, qkv, q, k, v


def _stream_post_attn(x, o, seg, mod, w):
    """Per-token work after attention for one stream (gated residuals, MLP)."""
    gate1, shift2, scale2, gate2 = mod[2][seg], mod[3][seg], mod[4][seg], mod[5][seg]
    attn_out = linear(o.reshape(o.shape[0], o.shape[1] * o.shape[2]), w["w_o"])
    x_mid = x + gate1 * attn_out
    h2 = modulate(rms_norm(x_mid), shift2, scale2)
    u = gelu(linear(h2, w["w_up"]))
    mlp_out = linear(u, w["w_down"])
    x_out = x_mid + gate2 * mlp_out
    return attn_out, x_mid, h2, u, mlp_out, x_out


def block_forward(x_img, x_txt, c, wb, pk, heads):
    """One dual-stream joint-attention block over a pack (R8-R14).

    x_img [n_img, H], x_txt [n_txt, H]: residual streams; c [B, H];
    wb = {"img": {...}, "txt": {...}} with the STREAM_KEYS weights.
    Returns a dict with every intermediate, keyed "<name>_img"/"<name>_txt":
      h (pre-attn modulated norm), qkv (raw projection), q, k (after QK-norm
      and RoPE), v, o (attention), attn_out (o W_o^T), x_mid, h2, u (GELU
      output), mlp_out (u W_down^T), x_out.
    """
    x_img = np.asarray(x_img, np.float64)
    x_txt = np.asarray(x_txt, np.float64)
    mods = {s: modulation(c, wb[s]["w_mod"]) for s in ("img", "txt")}
    pos_txt = np.zeros((x_txt.shape[0], 3))
    out = {}
    pre = {
        "img": _stream_pre_attn(x_img, pk["seg_img"], mods["img"], wb["img"], heads, pk["pos_img"]),
        "txt": _stream_pre_attn(x_txt, pk["seg_txt"], mods["txt"], wb["txt"], heads, pos_txt),
    }
    o_txt, o_img = packed_attention(pre["txt"][2], pre["txt"][3], pre["txt"][4],
                                    pre["img"][2], pre["img"][3], pre["img"][4], pk)
    o = {"img": o_img, "txt": o_txt}
    for s, x, seg in (("img", x_img, pk["seg_img"]), ("txt", x_txt, pk["seg_txt"])):
        h, qkv, q, k, v = pre[s]
        attn_out, x_mid, h2, u, mlp_out, x_out = _stream_post_attn(x, o[s], seg, mods[s], wb[s])
        for name, val in (("h", h), ("qkv", qkv), ("q", q), ("k", k), ("v", v), ("o", o[s]),
                          ("attn_out", attn_out), ("x_mid", x_mid), ("h2", h2), ("u", u),
                          ("mlp_out", mlp_out), ("x_out", x_out)):
            out[f"{name}_{s}"] = val
    return out


def block_forward_rows(x_img, x_txt, c, wb, pk, heads, b, img_rows, txt_rows):
    """The block's outputs for selected rows of sample b only.

    Rows are indices local to sample b (image rows from 0 at cu_img[b], text
    rows from 0 at cu_txt[b]).  Keys and values of the whole sample are
    computed (attention needs them); queries and every later step only for the
    selected rows.  Same definition as block_forward, restricted to fewer
    outputs, so full-size packs can be checked on a sample of rows.
    Returns {"x_mid_img", "x_out_img", "o_img", "x_mid_txt", ...} for the rows.
    """
    t0, t1 = pk["cu_txt"][b], pk["cu_txt"][b + 1]
    i0, i1 = pk["cu_img"][b], pk["cu_img"][b + 1]
    cb = np.asarray(c, np.float64)[b:b + 1]
    parts = {}
    for s, x, pos in (("txt", np.asarray(x_txt[t0:t1], np.float64), np.zeros((t1 - t0, 3))),
                      ("img", np.asarray(x_img[i0:i1], np.float64), pk["pos_img"][i0:i1])):
        seg = np.zeros(x.shape[0], np.int64)
        mod = modulation(cb, wb[s]["w_mod"])
        parts[s] = (x, seg, mod) + _stream_pre_attn(x, seg, mod, wb[s], heads, pos)
    k = np.concatenate([parts["txt"][6], parts["img"][6]])
    v = np.concatenate([parts["txt"][7], parts["img"][7]])
    out = {}
    for s, rows in (("txt", np.asarray(txt_rows, np.int64)), ("img", np.asarray(img_rows, np.int64))):
        x, seg, mod = parts[s][:3]
        q = parts[s][5][rows]
        o = attention(q, k, v)
        attn_out, x_mid, h2, u, mlp_out, x_out = _stream_post_attn(x[rows], o, seg[rows], mod, wb[s])
        out.update({f"o_{s}": o, f"attn_out_{s}": attn_out, f"x_mid_{s}": x_mid,
                    f"mlp_out_{s}": mlp_out, f"x_out_{s}": x_out, f"h_{s}": parts[s][3][rows]})
    return out


# ------------------------------------------------------------ embed / final

def embed(zt, tau, w_in, w_txt):
    """x_img = z_t W_in^T, x_txt = tau W_txt^T (R24)."""
    return linear(zt, w_in), linear(tau, w_txt)


def final_layer(x_img, c, w_fmod, w_out, pk):
    """v on target rows only (R15): (rms(x)(1+scale)+shift) W_out^T.

    Returns v [n_tgt, C] in target-row order (sample by sample, raster order).
    """
    shift, scale = modulation(c, w_fmod, chunks=2)
    rows = pk["tgt_rows"]
    seg = pk["seg_img"][rows]
    x = np.asarray(x_img, np.float64)[rows]
    return linear(modulate(rms_norm(x), shift[seg], scale[seg]), w_out)
