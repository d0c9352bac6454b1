"""Oracle: gradients of one dual-stream block (test infrastructure only).
float64 throughout; a matmul is the only library primitive for contractions.

The pages train the backbone with the rectified-flow objective on packed
native-resolution samples (hyper.ai 2607.19064, 方法; blog close-reading,
2.2(2)) and report the whole training step, forward and backward, as their
headline systems figure (blog close-reading, 证据二, Table 4).  They print no
backward pass: what a block's gradients are follows from the block's own
definition (the forward in block.py) by the chain rule, written here step by
step in the reverse order of the forward:

  x_out = x_mid + g2 * (GELU(h2 W_up^T) W_down^T),  h2 = rms(x_mid)(1+sc2)+sh2
  x_mid = x_in  + g1 * (o W_o^T),                    o  = attention(q', k', v)
  q' = RoPE(g_q * rms_head(q)), k' likewise, [q|k|v] = h1 W_qkv^T,
  h1 = rms(x_in)(1+sc1)+sh1,  [sh1,sc1,g1,sh2,sc2,g2] = W_mod SiLU(c).

Given dy = dL/dx_out for both streams it returns dL/dx_in, dL/dc and every
weight gradient.  Per-sample modulation vectors collect their gradient as a
sum over that sample's rows.  Pinned against central finite differences of
the forward (tests/test_oracle_grad.py).
"""

import math

import numpy as np
from scipy.special import erf as _sp_erf

from . import block as _blk


def seg_sum(x, seg, B):
    """Sum of the rows of x [n, H] per sample: [B, H]."""
    out = np.zeros((B, x.shape[1]))
    np.add.at(out, np.asarray(seg, np.int64), x)
    return out


def rms_backward(x, dn, eps=_blk.EPS):
    """Gradient through n = x / sqrt(mean(x^2) + eps) over the last axis:
    dx = (dn - n mean(dn n)) / r."""
    x = np.asarray(x, np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    n = x / r
    return (dn - n * np.mean(dn * n, axis=-1, keepdims=True)) / r


def gelu_grad(x):
    """d/dx of x Phi(x): Phi(x) + x phi(x)."""
    x = np.asarray(x, np.float64)
    return 0.5 * (1.0 + _sp_erf(x / math.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def silu_grad(x):
    s = 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))
    return s * (1.0 + x * (1.0 - s))


def rope_backward(dy, pos, theta=_blk.THETA):
    """The transpose of the pair rotation: rotate the gradient by -angle."""
    dy = np.asarray(dy, np.float64)
    ang = _blk.rope_angles(pos, dy.shape[-1], theta)[:, None, :]
    de, do = dy[..., 0::2], dy[..., 1::2]
    out = np.empty_like(dy)
    out[..., 0::2] = de * np.cos(ang) + do * np.sin(ang)
    out[..., 1::2] = -de * np.sin(ang) + do * np.cos(ang)
    return out


def attention_backward(q, k, v, do):
    """One sample: o = softmax(q k^T / sqrt(d)) v per head.
    With P the softmax, dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(dP P)),
    dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d).  Arrays [L, heads, d]."""
    q, k, v, do = (np.asarray(a, np.float64).transpose(1, 0, 2) for a in (q, k, v, do))
    d = q.shape[-1]
    s = q @ k.transpose(0, 2, 1) / math.sqrt(d)
    s -= s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    dv = p.transpose(0, 2, 1) @ do
    dp = do @ v.transpose(0, 2, 1)
    ds = p * (dp - np.sum(dp * p, axis=-1, keepdims=True))
    dq = ds @ k / math.sqrt(d)
    dk = ds.transpose(0, 2, 1) @ q / math.sqrt(d)
    return tuple(a.transpose(1, 0, 2) for a in (dq, dk, dv))


def packed_attention_backward(fw, d_o, pk):
    """Per-sample attention gradients over a pack; fw holds the forward's
    q, k, v per stream ([n, heads, d]), d_o = {"img": .., "txt": ..}."""
    g = {s: {n: np.zeros_like(fw[f"{n}_{s}"]) for n in ("q", "k", "v")} for s in ("img", "txt")}
    for b in range(pk["B"]):
        t0, t1 = pk["cu_txt"][b], pk["cu_txt"][b + 1]
        i0, i1 = pk["cu_img"][b], pk["cu_img"][b + 1]
        cat = {n: np.concatenate([fw[f"{n}_txt"][t0:t1], fw[f"{n}_img"][i0:i1]]) for n in ("q", "k", "v")}
        dob = np.concatenate([d_o["txt"][t0:t1], d_o["img"][i0:i1]])
        dq, dk, dv = attention_backward(cat["q"], cat["k"], cat["v"], dob)
        for n, val in (("q", dq), ("k", dk), ("v", dv)):
            g["txt"][n][t0:t1] = val[:t1 - t0]
            g["img"][n][i0:i1] = val[t1 - t0:]
    return g


def block_backward(x_img, x_txt, c, wb, pk, heads, dy_img, dy_txt):
    """Gradients of L = <dy_img, x_out_img> + <dy_txt, x_out_txt> for one block.

    Returns {"dx_img", "dx_txt", "dc", "img": {...}, "txt": {...}} where each
    stream dict holds d<w> for every key of block.STREAM_KEYS (w_mod [6H, H],
    w_qkv [3H, H], g_q [d], g_k [d], w_o [H, H], w_up [M, H], w_down [H, M])
    and "d_mod" [B, 6H] (the per-sample modulation gradient).
    """
    c = np.asarray(c, np.float64)
    B = c.shape[0]
    fw = _blk.block_forward(x_img, x_txt, c, wb, pk, heads)
    x_in = {"img": np.asarray(x_img, np.float64), "txt": np.asarray(x_txt, np.float64)}
    dy = {"img": np.asarray(dy_img, np.float64), "txt": np.asarray(dy_txt, np.float64)}
    seg = {"img": pk["seg_img"], "txt": pk["seg_txt"]}
    pos = {"img": pk["pos_img"], "txt": np.zeros((x_in["txt"].shape[0], 3))}
    H = c.shape[1]
    out = {"dc": np.zeros_like(c)}
    post = {}
    d_o = {}
    for s in ("img", "txt"):
        w = {k: np.asarray(v, np.float64) for k, v in wb[s].items()}
        sh1, sc1, g1, sh2, sc2, g2 = (m[seg[s]] for m in _blk.modulation(c, w["w_mod"]))
        # MLP branch and its gated residual
        d_xmid = dy[s].copy()
        d_g2 = seg_sum(dy[s] * fw[f"mlp_out_{s}"], seg[s], B)
        d_mlp = g2 * dy[s]
        dw_down = d_mlp.T @ fw[f"u_{s}"]
        u_pre = _blk.linear(fw[f"h2_{s}"], w["w_up"])
        d_upre = (d_mlp @ w["w_down"]) * gelu_grad(u_pre)
        dw_up = d_upre.T @ fw[f"h2_{s}"]
        d_h2 = d_upre @ w["w_up"]
        n2 = _blk.rms_norm(fw[f"x_mid_{s}"])
        d_sh2, d_sc2 = seg_sum(d_h2, seg[s], B), seg_sum(d_h2 * n2, seg[s], B)
        d_xmid += rms_backward(fw[f"x_mid_{s}"], d_h2 * (1.0 + sc2))
        # attention output projection and its gated residual
        d_g1 = seg_sum(d_xmid * fw[f"attn_out_{s}"], seg[s], B)
        d_a = g1 * d_xmid
        o = fw[f"o_{s}"].reshape(d_a.shape[0], H)
        dw_o = d_a.T @ o
        d_o[s] = (d_a @ w["w_o"]).reshape(fw[f"o_{s}"].shape)
        post[s] = dict(w=w, sh1=sh1, sc1=sc1, d_xmid=d_xmid, d_g1=d_g1, d_sh2=d_sh2, d_sc2=d_sc2, d_g2=d_g2,
                       dw_down=dw_down, dw_up=dw_up, dw_o=dw_o)
    ga = packed_attention_backward(fw, d_o, pk)
    for s in ("img", "txt"):
        p = post[s]
        w = p["w"]
        qkv = fw[f"qkv_{s}"]
        n_rows = qkv.shape[0]
        d = H // heads
        dqkv = []
        grads = {}
        for name, col, gname in (("q", 0, "g_q"), ("k", 1, "g_k")):
            raw = qkv[:, col * H:(col + 1) * H].reshape(n_rows, heads, d)
            nrm = _blk.rms_norm(raw)
            d_t = rope_backward(ga[s][name], pos[s])              # gradient of g * rms(raw)
            grads["d" + gname] = np.sum(d_t * nrm, axis=(0, 1))
            dqkv.append(rms_backward(raw, d_t * w[gname]).reshape(n_rows, H))
        dqkv.append(ga[s]["v"].reshape(n_rows, H))
        dqkv = np.concatenate(dqkv, axis=1)
        grads["dw_qkv"] = dqkv.T @ fw[f"h_{s}"]
        d_h = dqkv @ w["w_qkv"]
        n1 = _blk.rms_norm(x_in[s])
        d_sh1, d_sc1 = seg_sum(d_h, seg[s], B), seg_sum(d_h * n1, seg[s], B)
        out[f"dx_{s}"] = p["d_xmid"] + rms_backward(x_in[s], d_h * (1.0 + p["sc1"]))
        d_mod = np.concatenate([d_sh1, d_sc1, p["d_g1"], p["d_sh2"], p["d_sc2"], p["d_g2"]], axis=1)
        grads["dw_mod"] = d_mod.T @ _blk.silu(c)
        out["dc"] += (d_mod @ w["w_mod"]) * silu_grad(c)
        grads.update(dw_o=p["dw_o"], dw_up=p["dw_up"], dw_down=p["dw_down"], d_mod=d_mod)
        out[s] = grads
    return out


# ------------------------------------------------------ the whole training step

def final_layer_backward(x_img, c, w_fmod, w_out, pk, dv):
    """Gradients through v = (rms(x)(1 + sc) + sh) W_out^T on the target rows,
    [sh, sc] = W_fmod SiLU(c).  Returns (dx_img [n_img, H] (zero on rows that
    are not targets), dc [B, H], dw_fmod, dw_out)."""
    x_img = np.asarray(x_img, np.float64)
    c = np.asarray(c, np.float64)
    w_fmod = np.asarray(w_fmod, np.float64)
    w_out = np.asarray(w_out, np.float64)
    B = c.shape[0]
    rows = pk["tgt_rows"]
    seg = pk["seg_img"][rows]
    sh, sc = _blk.modulation(c, w_fmod, chunks=2)
    x = x_img[rows]
    n = _blk.rms_norm(x)
    h = _blk.modulate(n, sh[seg], sc[seg])
    dw_out = dv.T @ h
    dh = dv @ w_out
    d_mod = np.concatenate([seg_sum(dh, seg, B), seg_sum(dh * n, seg, B)], axis=1)
    dx = np.zeros_like(x_img)
    dx[rows] = rms_backward(x, dh * (1.0 + sc[seg]))
    dw_fmod = d_mod.T @ _blk.silu(c)
    dc = (d_mod @ w_fmod) * silu_grad(c)
    return dx, dc, dw_fmod, dw_out


def cond_backward(t, w_t1, w_t2, dc):
    """Gradients of c = W_t2 SiLU(W_t1 emb(t)) for the two weights."""
    w_t1 = np.asarray(w_t1, np.float64)
    w_t2 = np.asarray(w_t2, np.float64)
    emb = _blk.timestep_embedding(t, w_t1.shape[1])
    hid = _blk.linear(emb, w_t1)
    dw_t2 = dc.T @ _blk.silu(hid)
    dhid = (dc @ w_t2) * silu_grad(hid)
    return dhid.T @ emb, dw_t2


def training_step_grads(zt_img, tau, t, W, pk, heads, z, eps):
    """Every gradient of the flow-matching loss of one pack (hyper.ai
    2607.19064, 方法, the objective; blog close-reading, 2.2(2)): the model is
    cond -> embed -> blocks -> final layer on target rows; the loss is
    mean_b SSE_b / (tgt_len_b C) with SSE_b = sum (v - (z - eps))^2 over the
    target rows of sample b.  W as for flow.velocity_model.  Returns
    {"loss", "dv", "w_t1", "w_t2", "w_in", "w_txt", "w_fmod", "w_out",
    "blocks": [block_backward's stream dicts per block]}."""
    from . import flow as _flow

    c = _blk.cond(t, W["w_t1"], W["w_t2"])
    x_img, x_txt = _blk.embed(zt_img, tau, W["w_in"], W["w_txt"])
    xs = []
    for wb in W["blocks"]:
        xs.append((x_img, x_txt))
        o = _blk.block_forward(x_img, x_txt, c, wb, pk, heads)
        x_img, x_txt = o["x_out_img"], o["x_out_txt"]
    v = _blk.final_layer(x_img, c, W["w_fmod"], W["w_out"], pk)
    _, loss = _flow.loss(v, z, eps, pk)
    C = v.shape[1]
    scale = np.asarray(pk["tgt_len"], np.float64)[pk["seg_img"][pk["tgt_rows"]]] * C * pk["B"]
    dv = 2.0 * (v - _flow.velocity_target(z, eps, pk)) / scale[:, None]
    out = {"loss": loss, "dv": dv}
    dx_img, dc, out["w_fmod"], out["w_out"] = final_layer_backward(x_img, c, W["w_fmod"], W["w_out"], pk, dv)
    dx_txt = np.zeros_like(x_txt)
    out["blocks"] = [None] * len(W["blocks"])
    for i in range(len(W["blocks"]) - 1, -1, -1):
        g = block_backward(xs[i][0], xs[i][1], c, W["blocks"][i], pk, heads, dx_img, dx_txt)
        dx_img, dx_txt = g["dx_img"], g["dx_txt"]
        dc = dc + g["dc"]
        out["blocks"][i] = {"img": g["img"], "txt": g["txt"]}
    out["w_in"] = dx_img.T @ np.asarray(zt_img, np.float64)
    out["w_txt"] = dx_txt.T @ np.asarray(tau, np.float64)
    out["w_t1"], out["w_t2"] = cond_backward(t, W["w_t1"], W["w_t2"], dc)
    return out
