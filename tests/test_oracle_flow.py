"""Pins for the oracle's rectified-flow wrapper: closed forms and exactness."""

import numpy as np
import pytest

from oracle import block as K
from oracle import flow as F
from oracle import pack as P


def _pk():
    return P.pack([(3, 4, 1, 2), (2, 2, 2, 3), (1, 5, 1, 0)])


def test_make_xt_endpoints_bitwise():
    pk = _pk()
    r = np.random.default_rng(1)
    z, eps = r.standard_normal((2, pk["cu_img"][-1], 8))
    np.testing.assert_array_equal(F.make_xt(z, eps, np.zeros(3), pk), z)
    zt1 = F.make_xt(z, eps, np.ones(3), pk)
    rows = pk["tgt_rows"]
    np.testing.assert_array_equal(zt1[rows], eps[rows])
    src = np.setdiff1d(np.arange(len(z)), rows)
    assert len(src) == 4
    np.testing.assert_array_equal(zt1[src], z[src])          # source rows stay clean


def test_make_xt_is_affine_in_t():
    pk = _pk()
    r = np.random.default_rng(2)
    z, eps = r.standard_normal((2, pk["cu_img"][-1], 8))
    t0, t1 = np.array([0.1, 0.4, 0.9]), np.array([0.3, 0.2, 0.5])
    a = F.make_xt(z, eps, t0, pk)
    b = F.make_xt(z, eps, t1, pk)
    m = F.make_xt(z, eps, 0.5 * (t0 + t1), pk)
    np.testing.assert_allclose(m, 0.5 * (a + b), rtol=0, atol=1e-14)


def test_loss_zero_at_target_velocity_and_source_eps_ignored():
    pk = _pk()
    r = np.random.default_rng(3)
    z, eps = r.standard_normal((2, pk["cu_img"][-1], 8))
    v = F.velocity_target(z, eps, pk)
    sse, loss = F.loss(v, z, eps, pk)
    assert np.all(sse == 0) and loss == 0.0
    eps2 = eps.copy()
    src = np.setdiff1d(np.arange(len(z)), pk["tgt_rows"])
    eps2[src] += 100.0
    v2 = v + r.standard_normal(v.shape)
    np.testing.assert_array_equal(F.loss(v2, z, eps, pk)[0], F.loss(v2, z, eps2, pk)[0])


def test_loss_brute_force():
    pk = _pk()
    r = np.random.default_rng(4)
    z, eps = r.standard_normal((2, pk["cu_img"][-1], 3))
    v = r.standard_normal((pk["cu_tgt"][-1], 3))
    want = np.zeros(3)
    for b in range(3):
        i0 = pk["cu_img"][b]
        for i in range(pk["tgt_len"][b]):
            for c in range(3):
                d = v[pk["cu_tgt"][b] + i, c] - (z[i0 + i, c] - eps[i0 + i, c])
                want[b] += d * d
    sse, loss = F.loss(v, z, eps, pk)
    np.testing.assert_allclose(sse, want, rtol=1e-13)
    np.testing.assert_allclose(loss, np.mean(want / (pk["tgt_len"] * 3)), rtol=1e-13)


def test_euler_exact_on_linear_flow():
    # v == z* - eps is the exact velocity of the straight path z_t = (1-t) z* + t eps;
    # four Euler steps from z_1 = eps land on z*.
    r = np.random.default_rng(5)
    zs, eps = r.standard_normal((2, 64, 16))
    z = eps.copy()
    for i in range(4):
        z = F.euler_step(z, zs - eps, F.SCHEDULE[i], F.SCHEDULE[i + 1])
    np.testing.assert_allclose(z, zs, rtol=0, atol=1e-14)


def test_cfg_special_cases():
    r = np.random.default_rng(6)
    vc, vu = r.standard_normal((2, 32, 4))
    np.testing.assert_array_equal(F.cfg_combine(vu, vu, 4.0), vu)
    np.testing.assert_array_equal(F.cfg_combine(vc, vu, 0.0), vu)
    np.testing.assert_allclose(F.cfg_combine(vc, vu, 1.0), vc, atol=1e-15)


def _tiny_model(H=32, heads=2, C=8, depth=2, seed=7):
    r = np.random.default_rng(seed)

    def w(o, i):
        return r.standard_normal((o, i)) / np.sqrt(i)

    blocks = []
    for _ in range(depth):
        blocks.append({s: {"w_mod": w(6 * H, H), "w_qkv": w(3 * H, H), "g_q": np.ones(H // heads),
                           "g_k": np.ones(H // heads), "w_o": w(H, H), "w_up": w(4 * H, H),
                           "w_down": w(H, 4 * H)} for s in ("img", "txt")})
    return {"w_t1": w(H, 256), "w_t2": w(H, H), "w_in": w(H, C), "w_txt": w(H, H),
            "blocks": blocks, "w_fmod": w(2 * H, H), "w_out": w(C, H)}


def test_packed_cfg_equals_two_pass():
    # packing cond and uncond into one forward does not change the trajectory
    W = _tiny_model()
    r = np.random.default_rng(8)
    eps = r.standard_normal((12, 8))
    tc, tu = r.standard_normal((5, 32)), r.standard_normal((5, 32))
    zp, vp = F.sample_packed_cfg(eps, tc, tu, W, (3, 4), heads=2, g=4.0)
    z2, v2 = F.sample_two_pass_cfg(eps, tc, tu, W, (3, 4), heads=2, g=4.0)
    np.testing.assert_allclose(zp, z2, rtol=0, atol=1e-11)
    for a, b in zip(vp, v2):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def test_edit_sampler_packed_equals_two_pass():
    # editing packs (target + clean source per sample): packing the two CFG
    # branches still leaves the trajectory unchanged
    W = _tiny_model()
    r = np.random.default_rng(9)
    eps, src = r.standard_normal((12, 8)), r.standard_normal((12, 8))
    tc, tu = r.standard_normal((5, 32)), r.standard_normal((3, 32))
    zp, vp = F.sample_packed_cfg(eps, tc, tu, W, (3, 4), heads=2, g=4.0, src=src)
    z2, v2 = F.sample_two_pass_cfg(eps, tc, tu, W, (3, 4), heads=2, g=4.0, src=src)
    np.testing.assert_allclose(zp, z2, rtol=0, atol=1e-11)
    for a, b in zip(vp, v2):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def test_edit_sampler_source_enters_only_through_attention():
    # with every block gate at zero (adaLN-Zero) each block is the identity,
    # so a target row's velocity depends on that row alone: the edit sampler
    # then follows the generation sampler whatever the source holds.  With
    # live gates the source must steer the target through joint attention.
    W = _tiny_model()
    r = np.random.default_rng(10)
    eps = r.standard_normal((12, 8))
    src1, src2 = r.standard_normal((12, 8)), 3.0 * r.standard_normal((12, 8))
    tc, tu = r.standard_normal((5, 32)), r.standard_normal((5, 32))
    live1, _ = F.sample_packed_cfg(eps, tc, tu, W, (3, 4), heads=2, g=4.0, src=src1)
    live2, _ = F.sample_packed_cfg(eps, tc, tu, W, (3, 4), heads=2, g=4.0, src=src2)
    assert np.max(np.abs(live1 - live2)) > 1e-3
    Z = dict(W, blocks=[{s: dict(b[s], w_mod=np.zeros_like(b[s]["w_mod"])) for s in b} for b in W["blocks"]])
    gen, _ = F.sample_packed_cfg(eps, tc, tu, Z, (3, 4), heads=2, g=4.0)
    for src in (src1, src2):
        ed, _ = F.sample_packed_cfg(eps, tc, tu, Z, (3, 4), heads=2, g=4.0, src=src)
        np.testing.assert_allclose(ed, gen, rtol=0, atol=1e-12)


def test_timestep_embedding_closed_forms():
    e0 = K.timestep_embedding([0.0])
    np.testing.assert_array_equal(e0[0, :128], 1.0)
    np.testing.assert_array_equal(e0[0, 128:], 0.0)
    t = np.array([0.37, 0.9])
    e = K.timestep_embedding(t)
    np.testing.assert_allclose(e[:, :128] ** 2 + e[:, 128:] ** 2, 1.0, atol=1e-14)
    # first frequency is 1: pair 0 is (cos 1000t, sin 1000t); last is 10000**(-127/128)
    np.testing.assert_allclose(e[:, 0], np.cos(1000 * t), atol=1e-14)
    np.testing.assert_allclose(np.arctan2(e[:, 128 + 127], e[:, 127]),
                               1000 * t * 10000 ** (-127 / 128), atol=1e-12)


# ------------------------------------------------- negative-aware loss (R26)

def test_nft_loss_hand_value():
    # one sample, one 1x1 target row, C = 2: v+ - (z - eps) = (1, 0) and
    # v- - (z - eps) = (0, 2), so SSE = r * 1 + (1 - r) * 4 and the loss is
    # SSE / (1 * 2)
    pk = P.pack([(1, 1, 1, 0)])
    z, eps = np.array([[0.5, 0.5]]), np.array([[0.25, 0.5]])          # z - eps = (0.25, 0)
    vp, vn = np.array([[1.25, 0.0]]), np.array([[0.25, 2.0]])
    for r in (0.0, 0.3, 1.0):
        sse, loss = F.nft_loss(vp, vn, z, eps, np.array([r]), pk)
        assert sse[0] == pytest.approx(r + 4.0 * (1 - r), abs=1e-15)
        assert loss == pytest.approx((r + 4.0 * (1 - r)) / 2.0, abs=1e-15)


def test_nft_loss_reduces_to_the_base_loss_at_r_0_and_1():
    pk = _pk()
    r = np.random.default_rng(21)
    z, eps = r.standard_normal((2, pk["cu_img"][-1], 8))
    vp, vn = r.standard_normal((2, pk["cu_tgt"][-1], 8))
    base_p, base_n = F.loss(vp, z, eps, pk), F.loss(vn, z, eps, pk)
    one = F.nft_loss(vp, vn, z, eps, np.ones(3), pk)
    zero = F.nft_loss(vp, vn, z, eps, np.zeros(3), pk)
    np.testing.assert_array_equal(one[0], base_p[0])
    np.testing.assert_array_equal(zero[0], base_n[0])
    # mixed rewards pick per sample; v+ = v- makes r irrelevant
    mix = F.nft_loss(vp, vn, z, eps, np.array([1.0, 0.0, 1.0]), pk)[0]
    np.testing.assert_array_equal(mix, [base_p[0][0], base_n[0][1], base_p[0][2]])
    same = F.nft_loss(vp, vp, z, eps, np.array([0.2, 0.9, 0.5]), pk)
    np.testing.assert_allclose(same[0], base_p[0], rtol=1e-14)


def test_nft_loss_brute_force_and_source_rows_ignored():
    pk = _pk()
    r = np.random.default_rng(22)
    C = 3
    z, eps = r.standard_normal((2, pk["cu_img"][-1], C))
    vp, vn = r.standard_normal((2, pk["cu_tgt"][-1], C))
    rw = np.array([0.25, 0.6, 0.9])
    want = np.zeros(3)
    for b in range(3):
        i0, t0 = pk["cu_img"][b], pk["cu_tgt"][b]
        for i in range(pk["tgt_len"][b]):
            for ch in range(C):
                tgt = z[i0 + i, ch] - eps[i0 + i, ch]
                want[b] += rw[b] * (vp[t0 + i, ch] - tgt) ** 2 + (1 - rw[b]) * (vn[t0 + i, ch] - tgt) ** 2
    sse, loss = F.nft_loss(vp, vn, z, eps, rw, pk)
    np.testing.assert_allclose(sse, want, rtol=1e-13)
    assert loss == pytest.approx(np.mean(want / (pk["tgt_len"] * C)), rel=1e-13)
    eps2 = eps.copy()
    eps2[np.setdiff1d(np.arange(len(z)), pk["tgt_rows"])] += 50.0   # source rows of the edit sample
    np.testing.assert_array_equal(F.nft_loss(vp, vn, z, eps2, rw, pk)[0], sse)


# --------------------------------------------------- the sampler's step loop

def test_sampler_loop_hand_unrolled(monkeypatch):
    # Replace the network by a stub that records what it is called with and
    # returns a constant velocity per branch: a for the cond sample (first in
    # the pack), b for the uncond sample.  The guided velocity is then
    # b + g (a - b) at every step and the four steps, whose lengths sum to 1,
    # land on z_0 = eps + b + g (a - b).  The stub also checks that step i
    # runs at t = schedule[i], on z_t = the current latent for both samples.
    h, w, C, g = 2, 3, 4, 4.0
    n = h * w
    r = np.random.default_rng(23)
    eps = r.standard_normal((n, C))
    tau_c, tau_u = r.standard_normal((2, 5, 8))
    a, b = r.standard_normal((2, C))
    calls = []

    def stub(zt, tau, t, W, pk, heads):
        calls.append((np.array(zt), np.array(t), pk["B"]))
        np.testing.assert_array_equal(tau, np.concatenate([tau_c, tau_u]))
        return np.concatenate([np.tile(a, (n, 1)), np.tile(b, (n, 1))])

    monkeypatch.setattr(F, "velocity_model", stub)
    z, vs = F.sample_packed_cfg(eps, tau_c, tau_u, {}, (h, w), 1, g)
    vhat = b + g * (a - b)
    np.testing.assert_allclose(z, eps + vhat, rtol=0, atol=1e-14)
    assert [float(c[1][0]) for c in calls] == [1.0, 0.75, 0.5, 0.25]
    assert all(c[2] == 2 and c[1][0] == c[1][1] for c in calls)
    for i, (zt, _, _) in enumerate(calls):          # z_1 = eps, then one quarter step of vhat each
        want = eps + 0.25 * i * vhat
        np.testing.assert_allclose(zt[:n], want, atol=1e-14)
        np.testing.assert_allclose(zt[n:], want, atol=1e-14)
    for v in vs:
        np.testing.assert_allclose(v, np.tile(vhat, (n, 1)), atol=1e-15)
