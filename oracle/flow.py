"""Oracle: the rectified-flow wrapper around the block (test infrastructure
only).  float64 throughout.

What the pages fix (hyper.ai 2607.19064, 方法, the flow-matching objective and
the line under it; blog close-reading, 2.2(2), same equation):
  z_t = (1 - t) z + t eps,  eps ~ N(0, I),
  loss = E || v_theta(z_t, t, tau) - (z - eps) ||_2^2.
Editing: the condition holds the clean source latent and the loss is taken on
the target latent only (blog close-reading, 2.2(2)).  Sampling integrates the
learned velocity ODE from noise to data (blog close-reading, 5 "Rectified flow
matching"); classifier-free guidance combines conditional and unconditional
predictions, and packed CFG runs both branches in one packed forward without
changing the trajectory (hyper.ai 2607.19064, 实验; blog close-reading, 2.2(3)
and 5 "CFG").

Readings:
  R17  loss reported per sample as the sum of squares SSE_b, and as the scalar
       mean_b SSE_b / (tgt_len_b * C).
  R19  with target z - eps, dz/dt = eps - z = -v, so one Euler step from t to
       t' is z_{t'} = z_t + (t - t') v; z_1 = eps; schedule 1, .75, .5, .25 -> 0.
  R20  guided velocity v_u + g (v_c - v_u); cond and uncond share z_t and t.
  R25  in an editing pack only target rows are noised and scored; source rows
       carry the clean source latent.
  R26  the negative-aware loss of the post-training stage (blog close-reading,
       2.2(4), the Diffusion-NFT objective): per sample a reward r_b in [0, 1]
       weighs the squared error of a positive-policy velocity v+ against
       the target velocity and 1 - r_b weighs that of a negative-policy
       velocity v-.  The target velocity is the base objective's z - eps on
       the sample's target rows (same straight path); v+ and v- are inputs
       (the pages do not say how the two policies are formed); the
       normalisation is R17's.
"""

import numpy as np

from . import block as _blk


def make_xt(z, eps, t, pk):
    """Noised latent of every image row (R25).

    z, eps [n_img, C]: target rows hold the clean target latent, source rows
    the clean source latent.  t [B].  Target rows become (1-t_b) z + t_b eps;
    source rows keep z.
    """
    z = np.asarray(z, np.float64)
    eps = np.asarray(eps, np.float64)
    t = np.asarray(t, np.float64)
    zt = z.copy()
    rows = pk["tgt_rows"]
    tb = t[pk["seg_img"][rows]][:, None]
    zt[rows] = (1.0 - tb) * z[rows] + tb * eps[rows]
    return zt


def velocity_target(z, eps, pk):
    """z - eps on target rows, in target-row order [n_tgt, C]."""
    rows = pk["tgt_rows"]
    return np.asarray(z, np.float64)[rows] - np.asarray(eps, np.float64)[rows]


def loss(v, z, eps, pk):
    """RF matching loss (R17).  v [n_tgt, C] in target-row order.

    Returns (sse [B], scalar loss).
    """
    diff = np.asarray(v, np.float64) - velocity_target(z, eps, pk)
    C = diff.shape[1]
    sse = np.zeros(pk["B"])
    for b in range(pk["B"]):
        r0, r1 = pk["cu_tgt"][b], pk["cu_tgt"][b + 1]
        sse[b] = np.sum(diff[r0:r1] ** 2)
    per_elem = sse / (pk["tgt_len"].astype(np.float64) * C)
    return sse, float(np.mean(per_elem)) if pk["B"] else 0.0


def nft_loss(v_pos, v_neg, z, eps, r, pk):
    """Negative-aware flow-matching loss (R26).  v_pos, v_neg [n_tgt, C] in
    target-row order; r [B] rewards in [0, 1].

    SSE_b = r_b ||v+ - (z - eps)||^2 + (1 - r_b) ||v- - (z - eps)||^2 over the
    target rows of sample b; returns (sse [B], mean_b SSE_b / (tgt_len_b C)).
    """
    target = velocity_target(z, eps, pk)
    dp = np.asarray(v_pos, np.float64) - target
    dn = np.asarray(v_neg, np.float64) - target
    r = np.asarray(r, np.float64)
    C = target.shape[1]
    sse = np.zeros(pk["B"])
    for b in range(pk["B"]):
        r0, r1 = pk["cu_tgt"][b], pk["cu_tgt"][b + 1]
        sse[b] = r[b] * np.sum(dp[r0:r1] ** 2) + (1.0 - r[b]) * np.sum(dn[r0:r1] ** 2)
    per_elem = sse / (pk["tgt_len"].astype(np.float64) * C)
    return sse, float(np.mean(per_elem)) if pk["B"] else 0.0


def cfg_combine(v_cond, v_uncond, g):
    """Guided velocity v_u + g (v_c - v_u) (R20)."""
    v_cond = np.asarray(v_cond, np.float64)
    v_uncond = np.asarray(v_uncond, np.float64)
    return v_uncond + g * (v_cond - v_uncond)


def euler_step(z, v, t_cur, t_next):
    """z_{t'} = z_t + (t - t') v (R19)."""
    return np.asarray(z, np.float64) + (t_cur - t_next) * np.asarray(v, np.float64)


SCHEDULE = (1.0, 0.75, 0.5, 0.25, 0.0)


def velocity_model(zt_img, tau, t, W, pk, heads):
    """Full forward v_theta(z_t, t, tau) of a stack of blocks over a pack.

    W holds w_t1, w_t2, w_in, w_txt, blocks (list of {"img", "txt"} dicts),
    w_fmod, w_out.  Returns v [n_tgt, C].
    """
    c = _blk.cond(t, W["w_t1"], W["w_t2"])
    x_img, x_txt = _blk.embed(zt_img, tau, W["w_in"], W["w_txt"])
    for wb in W["blocks"]:
        o = _blk.block_forward(x_img, x_txt, c, wb, pk, heads)
        x_img, x_txt = o["x_out_img"], o["x_out_txt"]
    return _blk.final_layer(x_img, c, W["w_fmod"], W["w_out"], pk)


def _image_rows(z, src):
    """A sample's image rows: the target latent, then (editing) the clean
    source latent (R6, R25: slot 0 target, slot 1 source)."""
    return z if src is None else np.concatenate([z, np.asarray(src, np.float64)])


def sample_packed_cfg(eps, tau_c, tau_u, W, grid, heads, g, schedule=SCHEDULE, src=None):
    """Euler sampling with packed CFG (R19, R20).

    One pack holds [cond, uncond], both with the same image grid (h, w) and
    latent z; each step runs one packed forward, combines the two velocities
    and takes an Euler step.  With src (the clean source latent of an edit,
    [h*w, C]) both samples are editing samples: target rows noised, then the
    source rows, unchanged through the steps (R25); only the target moves.
    Returns (z_final, list of guided velocities).
    """
    from . import pack as _pack

    h, w = grid
    f = 1 if src is None else 2
    pk = _pack.pack([(h, w, f, len(tau_c)), (h, w, f, len(tau_u))])
    z = np.asarray(eps, np.float64).copy()
    tau = np.concatenate([np.asarray(tau_c, np.float64), np.asarray(tau_u, np.float64)])
    vs = []
    n = h * w
    for i in range(len(schedule) - 1):
        t = np.full(2, schedule[i])
        rows = _image_rows(z, src)
        v = velocity_model(np.concatenate([rows, rows]), tau, t, W, pk, heads)
        vhat = cfg_combine(v[:n], v[n:], g)
        vs.append(vhat)
        z = euler_step(z, vhat, schedule[i], schedule[i + 1])
    return z, vs


def sample_two_pass_cfg(eps, tau_c, tau_u, W, grid, heads, g, schedule=SCHEDULE, src=None):
    """The same sampler with cond and uncond run as two separate forwards."""
    from . import pack as _pack

    h, w = grid
    f = 1 if src is None else 2
    pc = _pack.pack([(h, w, f, len(tau_c))])
    pu = _pack.pack([(h, w, f, len(tau_u))])
    z = np.asarray(eps, np.float64).copy()
    vs = []
    for i in range(len(schedule) - 1):
        t = np.full(1, schedule[i])
        rows = _image_rows(z, src)
        vc = velocity_model(rows, tau_c, t, W, pc, heads)
        vu = velocity_model(rows, tau_u, t, W, pu, heads)
        vhat = cfg_combine(vc, vu, g)
        vs.append(vhat)
        z = euler_step(z, vhat, schedule[i], schedule[i + 1])
    return z, vs
