"""Pins for the oracle's block gradients: central finite differences of the
oracle forward, closed forms of the elementwise derivatives, and the
softmax-attention gradient against an explicit Jacobian."""

import math

import numpy as np
import pytest

from oracle import block as K
from oracle import grad as G
from oracle import pack as P

H, HEADS, MLP = 32, 2, 64
SAMPLES = [(2, 3, 1, 3), (3, 2, 2, 2)]          # a generation and an editing sample


def _setup(seed=0, scale=0.3):
    r = np.random.default_rng(seed)
    pk = P.pack(SAMPLES)
    n_img, n_txt, B = pk["cu_img"][-1], pk["cu_txt"][-1], len(SAMPLES)

    def w(o, i):
        return r.standard_normal((o, i)) * scale / math.sqrt(i)

    wb = {s: {"w_mod": w(6 * H, H) * 3.0, "w_qkv": w(3 * H, H) * 2.0,
              "g_q": 1.0 + 0.3 * r.standard_normal(H // HEADS), "g_k": 1.0 + 0.3 * r.standard_normal(H // HEADS),
              "w_o": w(H, H) * 3.0, "w_up": w(MLP, H) * 3.0, "w_down": w(H, MLP) * 3.0} for s in ("img", "txt")}
    x_img, x_txt = r.standard_normal((n_img, H)), r.standard_normal((n_txt, H))
    c = r.standard_normal((B, H))
    dy_img, dy_txt = r.standard_normal((n_img, H)), r.standard_normal((n_txt, H))
    return pk, wb, x_img, x_txt, c, dy_img, dy_txt


def _loss(pk, wb, x_img, x_txt, c, dy_img, dy_txt):
    o = K.block_forward(x_img, x_txt, c, wb, pk, HEADS)
    return float(np.sum(dy_img * o["x_out_img"]) + np.sum(dy_txt * o["x_out_txt"]))


def _fd(f, x, u, eps=1e-4):
    """Central difference along u with one Richardson step (error O(eps^4))."""
    c1 = (f(x + eps * u) - f(x - eps * u)) / (2 * eps)
    c2 = (f(x + 0.5 * eps * u) - f(x - 0.5 * eps * u)) / eps
    return (4 * c2 - c1) / 3


@pytest.fixture(scope="module")
def case():
    pk, wb, x_img, x_txt, c, dy_img, dy_txt = _setup()
    g = G.block_backward(x_img, x_txt, c, wb, pk, HEADS, dy_img, dy_txt)
    return pk, wb, x_img, x_txt, c, dy_img, dy_txt, g


@pytest.mark.parametrize("what", ["x_img", "x_txt", "c"])
def test_input_gradients_match_finite_differences(case, what):
    pk, wb, x_img, x_txt, c, dy_img, dy_txt, g = case
    args = {"x_img": x_img, "x_txt": x_txt, "c": c}
    grad = {"x_img": g["dx_img"], "x_txt": g["dx_txt"], "c": g["dc"]}[what]
    r = np.random.default_rng(hash(what) % 1000)
    for _ in range(2):
        u = r.standard_normal(args[what].shape)

        def f(v):
            a = dict(args)
            a[what] = v
            return _loss(pk, wb, a["x_img"], a["x_txt"], a["c"], dy_img, dy_txt)

        fd = _fd(f, args[what], u)
        an = float(np.sum(grad * u))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (what, fd, an)


@pytest.mark.parametrize("stream", ["img", "txt"])
@pytest.mark.parametrize("key", list(K.STREAM_KEYS))
def test_weight_gradients_match_finite_differences(case, stream, key):
    pk, wb, x_img, x_txt, c, dy_img, dy_txt, g = case
    r = np.random.default_rng(len(key) * 7 + len(stream))
    for _ in range(2):
        u = r.standard_normal(np.shape(wb[stream][key]))

        def f(v):
            w2 = {s: dict(wb[s]) for s in wb}
            w2[stream][key] = v
            return _loss(pk, w2, x_img, x_txt, c, dy_img, dy_txt)

        fd = _fd(f, np.asarray(wb[stream][key], np.float64), u)
        an = float(np.sum(g[stream]["d" + key] * u))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (stream, key, fd, an)


def test_single_entries_of_the_weight_gradients(case):
    # element-wise spot checks (a transposed gradient passes few of these)
    pk, wb, x_img, x_txt, c, dy_img, dy_txt, g = case
    for stream, key, idx in (("img", "w_qkv", (5, 17)), ("img", "w_qkv", (40, 3)), ("txt", "w_up", (60, 1)),
                             ("img", "w_down", (2, 50)), ("txt", "w_mod", (100, 9)), ("img", "w_o", (3, 30))):
        e = np.zeros(np.shape(wb[stream][key]))
        e[idx] = 1.0

        def f(v):
            w2 = {s: dict(wb[s]) for s in wb}
            w2[stream][key] = v
            return _loss(pk, w2, x_img, x_txt, c, dy_img, dy_txt)

        fd = _fd(f, np.asarray(wb[stream][key], np.float64), e)
        assert abs(fd - g[stream]["d" + key][idx]) <= 1e-7 * max(1.0, abs(fd)), (stream, key, idx)


def test_elementwise_derivatives_closed_forms():
    x = np.linspace(-5, 5, 1001)
    h = 1e-6
    np.testing.assert_allclose(G.gelu_grad(x), (K.gelu(x + h) - K.gelu(x - h)) / (2 * h), atol=1e-8)
    np.testing.assert_allclose(G.silu_grad(x), (K.silu(x + h) - K.silu(x - h)) / (2 * h), atol=1e-8)
    # GELU'(0) = 1/2, GELU' -> 1 and -> 0 far from 0; SiLU'(0) = 1/2
    assert G.gelu_grad(0.0) == 0.5 and abs(G.gelu_grad(8.0) - 1) < 1e-12 and abs(G.gelu_grad(-8.0)) < 1e-12
    assert G.silu_grad(0.0) == 0.5


def test_rope_backward_is_the_inverse_rotation():
    r = np.random.default_rng(5)
    y = r.standard_normal((6, 2, 16))
    pos = r.integers(0, 30, (6, 3))
    # the rotation is orthogonal: its transpose is its inverse
    np.testing.assert_allclose(G.rope_backward(K.apply_rope(y, pos), pos), y, atol=1e-12)
    u = r.standard_normal(y.shape)
    np.testing.assert_allclose(np.sum(K.apply_rope(y, pos) * u), np.sum(y * G.rope_backward(u, pos)), rtol=1e-12)


def test_attention_backward_against_explicit_jacobian():
    # brute force: the full Jacobian of o with respect to q, k, v by finite differences
    r = np.random.default_rng(6)
    L, hd, d = 5, 1, 4
    q, k, v = (r.standard_normal((L, hd, d)) for _ in range(3))
    do = r.standard_normal((L, hd, d))
    dq, dk, dv = G.attention_backward(q, k, v, do)
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            e = np.zeros_like(arr)
            e[idx] = 1e-6
            a1, a2 = arr + e, arr - e
            args = lambda a: (a, k, v) if arr is q else (q, a, v) if arr is k else (q, k, a)  # noqa: E731
            num[idx] = np.sum(do * (K.attention(*args(a1)) - K.attention(*args(a2)))) / 2e-6
        np.testing.assert_allclose(grad, num, atol=1e-8)


def test_zero_gates_pass_the_gradient_straight_through():
    # adaLN-Zero: W_mod = 0 makes every gate 0, the block the identity, and dx = dy exactly
    pk, wb, x_img, x_txt, c, dy_img, dy_txt = _setup(seed=7)
    for s in wb:
        wb[s]["w_mod"] = np.zeros_like(wb[s]["w_mod"])
    g = G.block_backward(x_img, x_txt, c, wb, pk, HEADS, dy_img, dy_txt)
    # the only path left for dx is the residual; modulation gradients stay nonzero (gates receive gradient)
    np.testing.assert_allclose(g["dx_img"], dy_img, atol=1e-14)
    np.testing.assert_allclose(g["dx_txt"], dy_txt, atol=1e-14)
    assert np.max(np.abs(g["img"]["d_mod"][:, 2 * H:3 * H])) > 0


def _tiny_model(seed=11, depth=2, C=8, t_dim=16):
    r = np.random.default_rng(seed)

    def w(o, i, s=1.0):
        return r.standard_normal((o, i)) * s / math.sqrt(i)

    blocks = []
    for _ in range(depth):
        blocks.append({s: {"w_mod": w(6 * H, H), "w_qkv": w(3 * H, H), "g_q": 1 + 0.2 * r.standard_normal(H // HEADS),
                           "g_k": 1 + 0.2 * r.standard_normal(H // HEADS), "w_o": w(H, H), "w_up": w(MLP, H),
                           "w_down": w(H, MLP)} for s in ("img", "txt")})
    return {"w_t1": w(H, t_dim), "w_t2": w(H, H), "w_in": w(H, C), "w_txt": w(H, H), "blocks": blocks,
            "w_fmod": w(2 * H, H), "w_out": w(C, H)}


def test_training_step_gradients_match_finite_differences():
    # the whole loss of one pack (generation + editing sample) against central
    # differences along random directions, for every weight of the model
    from oracle import flow as F

    pk = P.pack(SAMPLES)
    r = np.random.default_rng(12)
    W = _tiny_model()
    n_img, n_txt = pk["cu_img"][-1], pk["cu_txt"][-1]
    z, eps = r.standard_normal((n_img, 8)), r.standard_normal((n_img, 8))
    tau = r.standard_normal((n_txt, H))
    t = np.array([0.3, 0.8])
    zt = F.make_xt(z, eps, t, pk)
    g = G.training_step_grads(zt, tau, t, W, pk, HEADS, z, eps)

    def loss_of(Wm):
        v = F.velocity_model(zt, tau, t, Wm, pk, HEADS)
        return F.loss(v, z, eps, pk)[1]

    assert abs(loss_of(W) - g["loss"]) < 1e-12
    checks = [(k, None, None) for k in ("w_t1", "w_t2", "w_in", "w_txt", "w_fmod", "w_out")]
    checks += [(k, i, s) for i in range(2) for s in ("img", "txt") for k in ("w_mod", "w_qkv", "g_q", "w_down")]
    for key, bi, s in checks:
        base = W[key] if bi is None else W["blocks"][bi][s][key]
        grad = g[key] if bi is None else g["blocks"][bi][s]["d" + key]
        u = r.standard_normal(np.shape(base))

        def f(v):
            W2 = dict(W)
            if bi is None:
                W2[key] = v
            else:
                W2["blocks"] = [{ss: dict(b[ss]) for ss in b} for b in W["blocks"]]
                W2["blocks"][bi][s][key] = v
            return loss_of(W2)

        fd = _fd(f, np.asarray(base, np.float64), u)
        an = float(np.sum(grad * u))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(fd)), (key, bi, s, fd, an)
    # dv is the loss gradient with respect to the velocity, per target row
    v = F.velocity_model(zt, tau, t, W, pk, HEADS)
    du = r.standard_normal(v.shape)
    fd = (F.loss(v + 1e-5 * du, z, eps, pk)[1] - F.loss(v - 1e-5 * du, z, eps, pk)[1]) / 2e-5
    assert abs(fd - np.sum(g["dv"] * du)) < 1e-9
