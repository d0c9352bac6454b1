"""Pins for the oracle block: library routines, brute force and invariants."""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from oracle import block as K
from oracle import pack as P


# ------------------------------------------------------------------ norms

def test_rms_norm_unit_rms_and_scale_invariance():
    r = np.random.default_rng(0)
    x = r.standard_normal((50, 96)) * 3.0
    n = K.rms_norm(x)
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, -1)), 1.0, atol=1e-6)
    np.testing.assert_allclose(K.rms_norm(7.5 * x), n, atol=1e-9)
    # zero shift and scale reduce adaLN to the plain norm
    np.testing.assert_array_equal(K.modulate(n, 0.0, 0.0), n)


def test_rms_norm_matches_torch():
    r = np.random.default_rng(1)
    x = r.standard_normal((20, 64))
    want = TF.rms_norm(torch.from_numpy(x), (64,), eps=1e-6).numpy()
    np.testing.assert_allclose(K.rms_norm(x), want, rtol=1e-12, atol=1e-14)


def test_gelu_is_exact_erf_form():
    x = np.linspace(-6, 6, 2001)
    want = TF.gelu(torch.from_numpy(x)).numpy()                 # erf form
    np.testing.assert_allclose(K.gelu(x), want, rtol=1e-12, atol=1e-15)
    tanh = TF.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.max(np.abs(K.gelu(x) - tanh)) > 1e-4             # would catch the tanh form


# ------------------------------------------------------------------- RoPE

def test_rope_bands_and_pair_zero_rotates_by_position():
    assert K.rope_bands(128) == (32, 48, 48)
    assert K.rope_bands(64) == (16, 24, 24)
    pos = np.array([[3, 5, 11]])
    a = K.rope_angles(pos, 128)[0]
    # pair 0 of each band has frequency theta**0 = 1, so it turns by the raw position
    assert a[0] == 3 and a[16] == 5 and a[16 + 24] == 11
    # consecutive pairs inside a band are a geometric sequence of ratio theta**(-2/width)
    np.testing.assert_allclose(a[1:16] / a[:15], 10000 ** (-2 / 32), rtol=1e-13)
    np.testing.assert_allclose(a[17:40] / a[16:39], 10000 ** (-2 / 48), rtol=1e-13)
    np.testing.assert_allclose(a[41:64] / a[40:63], 10000 ** (-2 / 48), rtol=1e-13)


def test_rope_is_complex_multiplication():
    # RoPE of a pair (x, y) is (x + i y) * exp(i angle) (RoFormer's definition)
    r = np.random.default_rng(2)
    x = r.standard_normal((7, 3, 64))
    pos = r.integers(0, 40, (7, 3))
    ang = K.rope_angles(pos, 64)[:, None, :]
    zc = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)
    out = K.apply_rope(x, pos)
    np.testing.assert_allclose(out[..., 0::2], zc.real, atol=1e-13)
    np.testing.assert_allclose(out[..., 1::2], zc.imag, atol=1e-13)


def test_rope_norm_preservation_and_identity():
    r = np.random.default_rng(3)
    x = r.standard_normal((9, 2, 128))
    pos = r.integers(0, 128, (9, 3))
    out = K.apply_rope(x, pos)
    np.testing.assert_allclose(out[..., 0::2] ** 2 + out[..., 1::2] ** 2,
                               x[..., 0::2] ** 2 + x[..., 1::2] ** 2, rtol=1e-12)
    np.testing.assert_array_equal(K.apply_rope(x, np.zeros((9, 3))), x)
    # frame 0 leaves the frame band untouched: 3D with f = 0 is 2D RoPE
    pos[:, 0] = 0
    np.testing.assert_array_equal(K.apply_rope(x, pos)[..., :32], x[..., :32])


def test_rope_relative_position_property():
    r = np.random.default_rng(4)
    q, k = r.standard_normal((2, 6, 1, 64))
    pq = r.integers(0, 30, (6, 3))
    pk_ = r.integers(0, 30, (6, 3))
    shift = np.array([[1, 7, -4]])
    s0 = np.einsum("ihd,jhd->ij", K.apply_rope(q, pq), K.apply_rope(k, pk_))
    s1 = np.einsum("ihd,jhd->ij", K.apply_rope(q, pq + shift), K.apply_rope(k, pk_ + shift))
    np.testing.assert_allclose(s0, s1, atol=1e-11)


# -------------------------------------------------------------- attention

def _brute_attention(q, k, v):
    L, Hh, d = k.shape
    out = np.zeros((q.shape[0], Hh, d))
    for h in range(Hh):
        for i in range(q.shape[0]):
            s = [sum(q[i, h, e] * k[j, h, e] for e in range(d)) / math.sqrt(d) for j in range(L)]
            m = max(s)
            p = [math.exp(x - m) for x in s]
            z = sum(p)
            for e in range(d):
                out[i, h, e] = sum(p[j] * v[j, h, e] for j in range(L)) / z
    return out


def test_attention_brute_force():
    r = np.random.default_rng(5)
    q, k, v = r.standard_normal((3, 9, 2, 8)) * 2
    np.testing.assert_allclose(K.attention(q, k, v), _brute_attention(q, k, v), atol=1e-12)
    # query chunking does not change the result
    np.testing.assert_allclose(K.attention(q, k, v, q_chunk=4), K.attention(q, k, v), atol=1e-15)


def test_attention_matches_torch_sdpa():
    r = np.random.default_rng(6)
    q, k, v = r.standard_normal((3, 40, 3, 16))
    t = [torch.from_numpy(a).transpose(0, 1).contiguous() for a in (q, k, v)]
    want = TF.scaled_dot_product_attention(*t).transpose(0, 1).numpy()
    np.testing.assert_allclose(K.attention(q, k, v), want, atol=1e-12)


def _packed_qkv(pk, heads=2, d=8, seed=7):
    r = np.random.default_rng(seed)
    nt, ni = pk["cu_txt"][-1], pk["cu_img"][-1]
    return [r.standard_normal((n, heads, d)) for n in (nt, nt, nt, ni, ni, ni)]


def test_packed_equals_per_sample_unpacked():
    samples = [(3, 4, 1, 2), (2, 2, 2, 5), (1, 3, 1, 0)]
    pk = P.pack(samples)
    arrs = _packed_qkv(pk)
    o_txt, o_img = K.packed_attention(*arrs, pk)
    for b, s in enumerate(samples):
        one = P.pack([s])
        sl_t = slice(pk["cu_txt"][b], pk["cu_txt"][b + 1])
        sl_i = slice(pk["cu_img"][b], pk["cu_img"][b + 1])
        sub = [a[sl_t] for a in arrs[:3]] + [a[sl_i] for a in arrs[3:]]
        t1, i1 = K.packed_attention(*sub, one)
        np.testing.assert_array_equal(o_txt[sl_t], t1)
        np.testing.assert_array_equal(o_img[sl_i], i1)


def test_sample_order_invariance():
    samples = [(3, 4, 1, 2), (2, 2, 2, 5), (1, 3, 1, 1)]
    pk = P.pack(samples)
    arrs = _packed_qkv(pk)
    o_txt, o_img = K.packed_attention(*arrs, pk)
    perm = [2, 0, 1]
    pk2 = P.pack([samples[p] for p in perm])

    def cat(a, cu):
        return np.concatenate([a[cu[p]:cu[p + 1]] for p in perm])

    arrs2 = [cat(a, pk["cu_txt"]) for a in arrs[:3]] + [cat(a, pk["cu_img"]) for a in arrs[3:]]
    t2, i2 = K.packed_attention(*arrs2, pk2)
    np.testing.assert_array_equal(t2, cat(o_txt, pk["cu_txt"]))
    np.testing.assert_array_equal(i2, cat(o_img, pk["cu_img"]))


def test_uniform_logits_give_per_sample_mean_no_leak():
    pk = P.pack([(3, 4, 1, 2), (2, 2, 2, 5), (1, 3, 1, 1)])
    arrs = _packed_qkv(pk)
    arrs[0][:] = 0.0
    arrs[3][:] = 0.0                       # q = 0: every logit equal
    o_txt, o_img = K.packed_attention(*arrs, pk)
    for b in range(pk["B"]):
        sl_t = slice(pk["cu_txt"][b], pk["cu_txt"][b + 1])
        sl_i = slice(pk["cu_img"][b], pk["cu_img"][b + 1])
        mean = np.concatenate([arrs[2][sl_t], arrs[5][sl_i]]).mean(0)
        np.testing.assert_allclose(o_img[sl_i], np.broadcast_to(mean, o_img[sl_i].shape), atol=1e-14)
        np.testing.assert_allclose(o_txt[sl_t], np.broadcast_to(mean, o_txt[sl_t].shape), atol=1e-14)


def test_in_sample_permutation_equivariance():
    r = np.random.default_rng(8)
    q, k, v = r.standard_normal((3, 11, 2, 8))
    p = r.permutation(11)
    np.testing.assert_allclose(K.attention(q[p], k[p], v[p]), K.attention(q, k, v)[p], atol=1e-13)


# ------------------------------------------------------------------ block

def _weights(H, heads, r, std=None, mlp=None):
    mlp = mlp or 4 * H

    def w(o, i):
        return r.standard_normal((o, i)) * (std if std is not None else 1 / np.sqrt(i))

    return {s: {"w_mod": w(6 * H, H), "w_qkv": w(3 * H, H), "g_q": 1 + 0.1 * r.standard_normal(H // heads),
                "g_k": 1 + 0.1 * r.standard_normal(H // heads), "w_o": w(H, H), "w_up": w(mlp, H),
                "w_down": w(H, mlp)} for s in ("img", "txt")}


def test_adaln_zero_block_is_identity():
    r = np.random.default_rng(9)
    pk = P.pack([(3, 3, 1, 2), (2, 2, 2, 3)])
    wb = _weights(32, 2, r)
    for s in wb:
        wb[s]["w_mod"][:] = 0.0
    x_img = r.standard_normal((pk["cu_img"][-1], 32))
    x_txt = r.standard_normal((pk["cu_txt"][-1], 32))
    c = r.standard_normal((2, 32))
    o = K.block_forward(x_img, x_txt, c, wb, pk, 2)
    np.testing.assert_array_equal(o["x_out_img"], x_img)
    np.testing.assert_array_equal(o["x_out_txt"], x_txt)


def _torch_block(x_img, x_txt, c, wb, pos_img, heads):
    """The same block written with torch.nn.functional primitives and complex
    RoPE, for one sample, as an independent composition check."""
    T = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    xi, xt, c = T(x_img), T(x_txt), T(c)
    H = xi.shape[1]
    d = H // heads
    out = {}
    pre = {}
    for s, x, pos in (("txt", xt, np.zeros((xt.shape[0], 3))), ("img", xi, pos_img)):
        w = {k: T(v) for k, v in wb[s].items()}
        mod = TF.linear(TF.silu(c), w["w_mod"]).chunk(6, dim=-1)
        h = TF.rms_norm(x, (H,), eps=1e-6) * (1 + mod[1]) + mod[0]
        q, k, v = TF.linear(h, w["w_qkv"]).chunk(3, dim=-1)
        q = TF.rms_norm(q.view(-1, heads, d), (d,), weight=w["g_q"], eps=1e-6)
        k = TF.rms_norm(k.view(-1, heads, d), (d,), weight=w["g_k"], eps=1e-6)
        ang = torch.from_numpy(K.rope_angles(pos, d))[:, None, :]
        rot = torch.polar(torch.ones_like(ang), ang)
        q = torch.view_as_real(torch.view_as_complex(q.reshape(-1, heads, d // 2, 2).contiguous()) * rot)
        k = torch.view_as_real(torch.view_as_complex(k.reshape(-1, heads, d // 2, 2).contiguous()) * rot)
        pre[s] = (x, w, mod, q.reshape(-1, heads, d), k.reshape(-1, heads, d), v.reshape(-1, heads, d))
    q = torch.cat([pre["txt"][3], pre["img"][3]]).transpose(0, 1)
    k = torch.cat([pre["txt"][4], pre["img"][4]]).transpose(0, 1)
    v = torch.cat([pre["txt"][5], pre["img"][5]]).transpose(0, 1)
    o = TF.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(-1, H)
    nt = xt.shape[0]
    for s, os_ in (("txt", o[:nt]), ("img", o[nt:])):
        x, w, mod = pre[s][:3]
        x = x + mod[2] * TF.linear(os_, w["w_o"])
        h2 = TF.rms_norm(x, (H,), eps=1e-6) * (1 + mod[4]) + mod[3]
        x = x + mod[5] * TF.linear(TF.gelu(TF.linear(h2, w["w_up"])), w["w_down"])
        out[s] = x.numpy()
    return out


def test_block_matches_torch_functional_composition():
    r = np.random.default_rng(10)
    pk = P.pack([(4, 5, 2, 6)])
    H, heads = 64, 2
    wb = _weights(H, heads, r)
    x_img = r.standard_normal((pk["cu_img"][-1], H))
    x_txt = r.standard_normal((pk["cu_txt"][-1], H))
    c = r.standard_normal((1, H))
    o = K.block_forward(x_img, x_txt, c, wb, pk, heads)
    want = _torch_block(x_img, x_txt, c, wb, pk["pos_img"], heads)
    np.testing.assert_allclose(o["x_out_img"], want["img"], atol=1e-10)
    np.testing.assert_allclose(o["x_out_txt"], want["txt"], atol=1e-10)


def test_block_translation_invariance_of_rope():
    # shifting every (row, col) id of a sample leaves the block output unchanged
    r = np.random.default_rng(11)
    # (text tokens sit at the fixed origin, so the sample here has none)
    pk = P.pack([(3, 4, 2, 0)])
    H, heads = 32, 2
    wb = _weights(H, heads, r)
    x_img = r.standard_normal((pk["cu_img"][-1], H))
    x_txt = np.zeros((0, H))
    c = r.standard_normal((1, H))
    o0 = K.block_forward(x_img, x_txt, c, wb, pk, heads)
    pk2 = dict(pk)
    pk2["pos_img"] = pk["pos_img"] + np.array([[0, 5, 9]])
    o1 = K.block_forward(x_img, x_txt, c, wb, pk2, heads)
    np.testing.assert_allclose(o1["x_out_img"], o0["x_out_img"], atol=1e-11)


def test_block_rows_equals_full_block():
    r = np.random.default_rng(12)
    pk = P.pack([(3, 3, 1, 2), (2, 3, 2, 4)])
    H, heads = 32, 2
    wb = _weights(H, heads, r)
    x_img = r.standard_normal((pk["cu_img"][-1], H))
    x_txt = r.standard_normal((pk["cu_txt"][-1], H))
    c = r.standard_normal((2, H))
    full = K.block_forward(x_img, x_txt, c, wb, pk, heads)
    rows = K.block_forward_rows(x_img, x_txt, c, wb, pk, heads, 1, [0, 5, 11], [1, 3])
    i0, t0 = pk["cu_img"][1], pk["cu_txt"][1]
    for name in ("o", "x_mid", "x_out", "attn_out", "mlp_out", "h"):
        np.testing.assert_allclose(rows[f"{name}_img"].reshape(3, -1),
                                   full[f"{name}_img"][i0 + np.array([0, 5, 11])].reshape(3, -1), atol=1e-12)
        np.testing.assert_allclose(rows[f"{name}_txt"].reshape(2, -1),
                                   full[f"{name}_txt"][t0 + np.array([1, 3])].reshape(2, -1), atol=1e-12)


def test_final_layer_only_target_rows():
    r = np.random.default_rng(13)
    pk = P.pack([(2, 2, 2, 1), (1, 3, 1, 2)])
    H, C = 16, 4
    x = r.standard_normal((pk["cu_img"][-1], H))
    c = r.standard_normal((2, H))
    wf, wo = r.standard_normal((2 * H, H)), r.standard_normal((C, H))
    v = K.final_layer(x, c, wf, wo, pk)
    assert v.shape == (pk["cu_tgt"][-1], C)
    x2 = x.copy()
    x2[4:8] += 50.0                                          # source rows of sample 0
    np.testing.assert_array_equal(K.final_layer(x2, c, wf, wo, pk), v)


@pytest.mark.parametrize("H,heads", [(256, 4)])
def test_cond_shapes(H, heads):
    r = np.random.default_rng(14)
    c = K.cond(np.array([0.2, 0.7]), r.standard_normal((H, 256)), r.standard_normal((H, H)))
    assert c.shape == (2, H)
    m = K.modulation(c, r.standard_normal((6 * H, H)))
    assert len(m) == 6 and m[0].shape == (2, H)


# ------------------------------------------ conditioning and final layer pins
#
# Hand-derivable values.  SiLU(1) = 1 / (1 + e^-1) = 0.7310585786300049 and
# SiLU(0) = 0; the timestep embedding of R11 at t = 0 is cos(0) = 1 on its
# first half and sin(0) = 0 on its second half.

SILU1 = 0.7310585786300049


def _selector(rows, cols, picks):
    w = np.zeros((rows, cols))
    for i, j in enumerate(picks):
        w[i, j] = 1.0
    return w


def test_cond_closed_form_at_t0():
    # W_t1 picks embedding entries 0..3 (cos half) and 128..131 (sin half),
    # scaled by 3; W_t2 = 2 I.  c = W_t2 SiLU(W_t1 emb(0)) = 2 SiLU(3) on the
    # cos picks and 2 SiLU(0) = 0 on the sin picks.
    H = 8
    w1 = 3.0 * _selector(H, 256, [0, 1, 2, 3, 128, 129, 130, 131])
    w2 = 2.0 * np.eye(H)
    c = K.cond(np.array([0.0]), w1, w2)
    silu3 = 3.0 / (1.0 + math.exp(-3.0))                     # 2.857722...
    np.testing.assert_allclose(c[0], [2 * silu3] * 4 + [0.0] * 4, rtol=0, atol=1e-15)
    # SiLU after W_t2 instead (silu(6) = 5.985...) or before W_t1 would differ:
    assert abs(2 * silu3 - 6.0 / (1.0 + math.exp(-6.0))) > 0.1


def test_cond_closed_form_factor_1000():
    # t = pi / 2000: the first frequency turns by 1000 t = pi / 2, so the
    # embedding's entry 0 is cos(pi/2) = 0 and entry 128 is sin(pi/2) = 1.
    H = 4
    w1 = _selector(H, 256, [0, 128, 0, 128])
    w2 = np.eye(H)
    c = K.cond(np.array([math.pi / 2000.0]), w1, w2)
    np.testing.assert_allclose(c[0], [0.0, SILU1, 0.0, SILU1], rtol=0, atol=1e-12)


def test_cond_per_sample_and_modulation_chunk_order():
    # two samples keep their own t; modulation splits W SiLU(c) into six
    # H-chunks in order: chunk k of row b is rows k*H..(k+1)*H of W applied
    # to SiLU(c_b)
    H = 4
    w1 = _selector(H, 256, [0, 1, 128, 129])
    c = K.cond(np.array([0.0, math.pi / 2000.0]), w1, np.eye(H))
    np.testing.assert_allclose(c[0], [SILU1, SILU1, 0.0, 0.0], atol=1e-15)
    assert abs(c[1][0]) < 1e-12 and abs(c[1][2] - SILU1) < 1e-12
    w_mod = np.zeros((6 * H, H))
    for k in range(6):
        w_mod[k * H, 0] = k + 1.0                             # chunk k, entry 0: (k + 1) SiLU(c[0])
    m = K.modulation(np.array([[1.0, 0, 0, 0]]), w_mod)
    assert [float(x[0, 0]) for x in m] == pytest.approx([(k + 1) * SILU1 for k in range(6)], abs=1e-15)


def _final_pack():
    # one sample, 1 x 2 grid, no text: target rows 0 and 1
    return P.pack([(1, 2, 1, 0)])


def test_final_layer_zero_modulation_is_plain_norm():
    # W_fmod = 0: shift = scale = 0, so v = rms(x) W_out^T.  Row 0 is
    # (2, -2, ...): mean square 4, so rms(x) = x / sqrt(4 + eps).
    pk = _final_pack()
    H = 8
    x = np.array([[2.0, -2.0] * 4, [1.0, 0, 0, 0, 0, 0, 0, 0]])
    w_out = _selector(2, H, [0, 1])
    v = K.final_layer(x, np.ones((1, H)), np.zeros((2 * H, H)), w_out, pk)
    n0 = 2.0 / math.sqrt(4.0 + 1e-6)
    n1 = 1.0 / math.sqrt(1.0 / 8.0 + 1e-6)                    # row 1: mean square 1/8
    np.testing.assert_allclose(v, [[n0, -n0], [n1, 0.0]], rtol=0, atol=1e-14)


def test_final_layer_modulation_closed_form():
    # c = (1, 0, ...) so SiLU(c) = (SiLU(1), 0, ...); W_fmod's first column
    # = (shift; scale) / SiLU(1) with shift = 0.5 and scale = 2 everywhere.
    # v = (rms(x)(1 + 2) + 0.5) W_out^T = 3 n + 0.5.  A dropped (1 + scale)
    # gives 2 n + 0.5, swapped chunks 1.5 n + 2, a missing RMS 3 x + 0.5.
    pk = _final_pack()
    H = 8
    x = np.array([[2.0, -2.0] * 4, [4.0] * 8])
    c = np.zeros((1, H))
    c[0, 0] = 1.0
    w_fmod = np.zeros((2 * H, H))
    w_fmod[:H, 0] = 0.5 / SILU1
    w_fmod[H:, 0] = 2.0 / SILU1
    w_out = _selector(2, H, [0, 1])
    v = K.final_layer(x, c, w_fmod, w_out, pk)
    n0 = 2.0 / math.sqrt(4.0 + 1e-6)
    n1 = 4.0 / math.sqrt(16.0 + 1e-6)
    np.testing.assert_allclose(v, [[3 * n0 + 0.5, -3 * n0 + 0.5], [3 * n1 + 0.5, 3 * n1 + 0.5]],
                               rtol=0, atol=1e-13)


def test_final_layer_uses_each_samples_modulation():
    # two samples with different c: each target row takes its own sample's
    # (shift, scale); sample 1's c is 0, so SiLU(c) = 0 and v is the plain norm
    pk = P.pack([(1, 1, 1, 0), (1, 1, 1, 0)])
    H = 8
    x = np.array([[2.0, -2.0] * 4, [2.0, -2.0] * 4])
    c = np.zeros((2, H))
    c[0, 0] = 1.0
    w_fmod = np.zeros((2 * H, H))
    w_fmod[:H, 0] = 0.5 / SILU1
    w_fmod[H:, 0] = 2.0 / SILU1
    v = K.final_layer(x, c, w_fmod, _selector(1, H, [0]), pk)
    n0 = 2.0 / math.sqrt(4.0 + 1e-6)
    np.testing.assert_allclose(v[:, 0], [3 * n0 + 0.5, n0], rtol=0, atol=1e-13)


def test_rope_other_band_widths():
    # a frame band of width 0 leaves the frame id unused (2D RoPE); the row
    # band's pair 0 turns by the raw row id whatever the split
    pos = np.array([[3, 5, 7]])
    a = K.rope_angles(pos, 8, bands=(0, 4, 4))
    np.testing.assert_allclose(a[0], [5, 5 * 100.0 ** -1, 7, 7 * 100.0 ** -1], rtol=1e-14)
    b = K.rope_angles(pos, 8, bands=(2, 2, 4))
    np.testing.assert_allclose(b[0], [3, 5, 7, 7 * 100.0 ** -1], rtol=1e-14)
    with pytest.raises(ValueError):
        K.rope_angles(pos, 8, bands=(2, 2, 2))
    with pytest.raises(ValueError):
        K.rope_angles(pos, 8, bands=(1, 3, 4))


def test_row_wise_metric_catches_a_wrong_small_row():
    from helpers import rel_err, rel_err_rows

    r = np.random.default_rng(30)
    ref = r.standard_normal((8, 16))
    ref[3] *= 0.02                          # a small-magnitude row
    got = ref.copy()
    got[3] *= 1.5                           # 50% off on that row only
    assert rel_err(got, ref) < 2e-2 < rel_err_rows(got, ref)
    assert rel_err_rows(ref, ref) == 0.0
