"""GPU parity of whole passes: the training forward with the RF loss and the
packed-CFG Euler sampler."""

import numpy as np
import pytest
import torch

from helpers import TOL, assert_close, f64_block, oracle_pack, to_np
from oracle import block as OB
from oracle import flow as OF
from resolution_image_gen_amd import configs as CF
from resolution_image_gen_amd import synthetic as S

pytestmark = pytest.mark.gpu


def _oracle_train(wl, W, inp, samples):
    ref = oracle_pack(samples)
    zt = OF.make_xt(inp["z"], inp["eps"], inp["t"], ref)
    Wd = {k: np.asarray(v, np.float64) for k, v in W.np_wrap.items()}
    Wd["blocks"] = [f64_block(nb) for nb in W.np_blocks]
    v = OF.velocity_model(zt, inp["tau"], inp["t"], Wd, ref, wl.dims.heads)
    sse, loss = OF.loss(v, inp["z"], inp["eps"], ref)
    return v, sse, loss


@pytest.mark.parametrize("name,recipe", [("tiny_f32", "default"), ("tiny_f32", "stress"),
                                         ("pack256_bf16", "default")])
def test_training_forward(name, recipe):
    from resolution_image_gen_amd import runner as R

    wl = CF.WORKLOADS[name]
    print(f"train forward {name} {recipe}", flush=True)
    W = R.Weights(wl, recipe=recipe)
    inp = R.training_inputs(wl)
    tf = R.TrainForward(wl, W, inp)
    tf.run()
    torch.cuda.synchronize()
    v, sse, loss = _oracle_train(wl, W, inp, wl.samples)
    tol = TOL[wl.dtype]
    assert_close("v", to_np(tf.v), v, tol)
    assert_close("sse", to_np(tf.sse), sse, tol)
    assert abs(tf.loss.item() - loss) <= tol * abs(loss)
    # a second run is bitwise identical
    v1 = tf.v.clone()
    tf.run()
    assert torch.equal(v1, tf.v)


def test_training_forward_edit_pack_small():
    """Editing pack (3D RoPE, source rows clean, loss on target rows only) at
    reduced width, fp32."""
    from resolution_image_gen_amd import runner as R

    wl = CF.Workload("edit_small_f32", CF.TINY, "f32", ((12, 10, 2, 24), (5, 7, 2, 3)), img_budget=10 ** 6)
    W = R.Weights(wl, recipe="stress")
    inp = R.training_inputs(wl)
    tf = R.TrainForward(wl, W, inp)
    tf.run()
    torch.cuda.synchronize()
    v, sse, loss = _oracle_train(wl, W, inp, wl.samples)
    assert_close("v", to_np(tf.v), v, TOL["f32"])
    assert_close("sse", to_np(tf.sse), sse, TOL["f32"])


def _small_sampler_wl(dtype, depth=2):
    d = CF.Dims(hidden=512, heads=4, head_dim=128, mlp=2048, c_lat=64, d_txt=512) if dtype == "bf16" else CF.TINY
    return CF.Workload(f"sampler_small_{dtype}", d, dtype, ((12, 16, 1, 24), (12, 16, 1, 24)), img_budget=384,
                       depth=depth, steps=4, guidance=4.0)


BASE20 = tuple(1.0 - i / 20 for i in range(21))   # 20 uniform Euler steps, 1 -> 0


@pytest.mark.parametrize("dtype,schedule,edit", [("f32", None, False), ("bf16", None, False),
                                                  ("f32", BASE20, False), ("f32", None, True),
                                                  ("bf16", None, True)])
def test_sampler_vs_oracle(dtype, schedule, edit):
    """Generation and (edit=True) editing samplers: each sample holds a noised
    target and, for an edit, the clean source latent of the same grid."""
    from resolution_image_gen_amd import runner as R

    wl = _small_sampler_wl(dtype)
    if schedule is not None:
        wl = CF.Workload(wl.name, wl.dims, dtype, wl.samples, wl.img_budget, depth=wl.depth,
                         steps=len(schedule) - 1, guidance=wl.guidance, schedule=schedule)
    print(f"sampler {dtype} {len(wl.schedule) - 1} steps edit={edit}", flush=True)
    W = R.Weights(wl, recipe="stress")
    h, w = wl.samples[0][:2]
    eps = S.normal((h * w, wl.dims.c_lat), 1.0, dtype, wl.name, "eps")
    tau_c = S.text(24, wl.dims.d_txt, dtype, wl.name, "tau_c")
    tau_u = S.text(24, wl.dims.d_txt, dtype, wl.name, "tau_u")
    src = S.normal((h * w, wl.dims.c_lat), 1.0, dtype, wl.name, "src") if edit else None
    vs = []
    sm = R.Sampler(wl, W, eps, tau_c, tau_u, src=src)
    sm.run(on_step=lambda i, s: vs.append(to_np(s.v)))
    torch.cuda.synchronize()
    Wd = {k: np.asarray(v, np.float64) for k, v in W.np_wrap.items()}
    Wd["blocks"] = [f64_block(nb) for nb in W.np_blocks]
    g = wl.guidance
    z_ref, vhat_ref = OF.sample_packed_cfg(eps, tau_c, tau_u, Wd, (h, w), wl.dims.heads, g, wl.schedule, src=src)
    assert len(vs) == len(vhat_ref) == len(wl.schedule) - 1
    tol = TOL[dtype]
    n = h * w
    # step 0 runs on identical inputs: each branch's raw velocity is held to the bar
    f = 2 if edit else 1
    pk = oracle_pack([(h, w, f, 24), (h, w, f, 24)])
    rows = np.concatenate([eps, src]) if edit else eps
    v0 = OF.velocity_model(np.concatenate([rows, rows]), np.concatenate([tau_c, tau_u]), np.ones(2), Wd, pk,
                           wl.dims.heads)
    assert_close("v_cond step 0", vs[0][:n], v0[:n], tol)
    assert_close("v_uncond step 0", vs[0][n:], v0[n:], tol)
    # guidance amplifies branch errors: |err(vhat)| <= (|1-g| + g) * tol * max|v|
    vmax = np.max(np.abs(v0))
    for i, v in enumerate(vs):
        bound = (abs(1 - g) + g) * tol * vmax / np.max(np.abs(vhat_ref[i]))
        assert_close(f"vhat step {i}", OF.cfg_combine(v[:n], v[n:], g), vhat_ref[i], bound)
    # z_final = eps + sum_i dt_i vhat_i: the same bound carried through the four steps
    zb = (abs(1 - g) + g) * tol * vmax / np.max(np.abs(z_ref))
    assert_close("z_final", to_np(sm.z), z_ref, zb)
    if edit:   # the source rows of both samples still hold the clean source, bit for bit
        zt = to_np(sm.zt)
        np.testing.assert_array_equal(zt[n:2 * n], src)
        np.testing.assert_array_equal(zt[3 * n:], src)


def test_sampler_vs_oracle_headline_width():
    """The 4-step packed-CFG sampler at its own width and pack (hidden 3,072,
    24 x 128 heads, MLP 12,288, latent 128; cond + uncond each a 64 x 64 grid
    + 256 text tokens, 8,704 tokens; guidance 4; bf16), cut to one block and
    the schedule's first two steps (1 -> 0.75 -> 0.5) so the float64 oracle
    finishes in seconds: both branches' step-0 velocities at the bar, the
    guided velocities and the latent after two steps at the guidance bound."""
    import time

    from resolution_image_gen_amd import runner as R

    sched = (1.0, 0.75, 0.5)
    wl = CF.Workload("sampler1024_cfg_bf16_2step", CF.B4, "bf16", ((64, 64, 1, 256), (64, 64, 1, 256)),
                     img_budget=8192, depth=1, steps=2, guidance=4.0, schedule=sched)
    t0 = time.time()
    W = R.Weights(wl, recipe="stress")
    h, w = 64, 64
    n = h * w
    eps = S.normal((n, wl.dims.c_lat), 1.0, "bf16", wl.name, "eps")
    tau_c = S.text(256, wl.dims.d_txt, "bf16", wl.name, "tau_c")
    tau_u = S.text(256, wl.dims.d_txt, "bf16", wl.name, "tau_u")
    vs = []
    sm = R.Sampler(wl, W, eps, tau_c, tau_u)
    sm.run(on_step=lambda i, st: vs.append(to_np(st.v)))
    torch.cuda.synchronize()
    print(f"headline-width sampler on the GPU after {time.time() - t0:.1f} s", flush=True)
    Wd = {k: np.asarray(v, np.float64) for k, v in W.np_wrap.items()}
    Wd["blocks"] = [f64_block(nb) for nb in W.np_blocks]
    g = wl.guidance
    pk = oracle_pack([(h, w, 1, 256), (h, w, 1, 256)])
    v0 = OF.velocity_model(np.concatenate([eps, eps]), np.concatenate([tau_c, tau_u]), np.ones(2), Wd, pk,
                           wl.dims.heads)
    tol = TOL["bf16"]
    assert_close("v_cond step 0", vs[0][:n], v0[:n], tol)
    assert_close("v_uncond step 0", vs[0][n:], v0[n:], tol)
    z_ref, vhat_ref = OF.sample_packed_cfg(eps, tau_c, tau_u, Wd, (h, w), wl.dims.heads, g, sched)
    print(f"oracle done after {time.time() - t0:.1f} s", flush=True)
    assert len(vs) == len(vhat_ref) == 2
    vmax = np.max(np.abs(v0))
    for i, v in enumerate(vs):
        bound = (abs(1 - g) + g) * tol * vmax / np.max(np.abs(vhat_ref[i]))
        assert_close(f"vhat step {i}", OF.cfg_combine(v[:n], v[n:], g), vhat_ref[i], bound)
    zb = (abs(1 - g) + g) * tol * vmax / np.max(np.abs(z_ref))
    assert_close("z after two steps", to_np(sm.z), z_ref, zb)


def test_packed_cfg_equals_two_pass_on_gpu():
    """Packing cond + uncond in one forward reproduces two separate forwards."""
    from resolution_image_gen_amd import binding as B
    from resolution_image_gen_amd import runner as R

    wl = _small_sampler_wl("bf16", depth=1)
    W = R.Weights(wl, recipe="stress")
    h, w = wl.samples[0][:2]
    dims = W.dims
    C = wl.dims.c_lat
    z = torch.from_numpy(S.normal((h * w, C), 1.0, "bf16", "pcfg", "z")).cuda().to(torch.bfloat16)
    tc = torch.from_numpy(S.text(24, wl.dims.d_txt, "bf16", "pcfg", "c")).cuda().to(torch.bfloat16)
    tu = torch.from_numpy(S.text(24, wl.dims.d_txt, "bf16", "pcfg", "u")).cuda().to(torch.bfloat16)
    t = torch.full((2,), 0.6, device="cuda")

    def forward(samples, zt, tau, tt):
        pk = B.pack(samples)
        c = torch.empty(pk.B, wl.dims.hidden, dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(B.workspace_size(dims, pk), dtype=torch.uint8, device="cuda")
        xi = torch.empty(pk.n_img, wl.dims.hidden, dtype=torch.bfloat16, device="cuda")
        xt = torch.empty(pk.n_txt, wl.dims.hidden, dtype=torch.bfloat16, device="cuda")
        v = torch.empty(pk.n_tgt, C, dtype=torch.bfloat16, device="cuda")
        B.cond(dims, W.wrap["w_t1"], W.wrap["w_t2"], tt, c, ws)
        B.embed(dims, W.wrap["w_in"], W.wrap["w_txt"], pk, zt, tau, xi, xt)
        B.block_fwd(dims, W.bw[0], pk, c, xi, xt, ws)
        B.final(dims, W.wrap["w_fmod"], W.wrap["w_out"], pk, c, xi, v, ws)
        return v

    vp = forward([(h, w, 1, 24), (h, w, 1, 24)], torch.cat([z, z]), torch.cat([tc, tu]), t)
    vc = forward([(h, w, 1, 24)], z, tc, t[:1])
    vu = forward([(h, w, 1, 24)], z, tu, t[:1])
    torch.cuda.synchronize()
    n = h * w
    # the per-row work is independent of the pack, so the results agree to the last bit
    assert torch.equal(vp[:n], vc), (vp[:n].float() - vc.float()).abs().max()
    assert torch.equal(vp[n:], vu)


@pytest.mark.parametrize("case,tu_len", [("small", 24), ("small", 9), ("wide64x64", 256), ("edit_small", 9),
                                         ("edit_wide64x64", 256)])
def test_two_pass_sampler_equals_packed(case, tu_len):
    """The 4-step sampler with its CFG branches as two separate forwards per
    step ends on the same bits as the packed one (eager and graph-replayed);
    the unconditional text may be shorter than the conditional one.  The
    64x64-grid case runs every launch at twice the rows in the packed form
    (8,704 vs 4,352), where tile and split choices would differ if they
    depended on the row count."""
    from resolution_image_gen_amd import runner as R

    if case.endswith("small"):
        wl = _small_sampler_wl("bf16", depth=2)
        W = R.Weights(wl, recipe="stress")
    else:
        d = CF.Dims(hidden=1024, heads=8, head_dim=128, mlp=4096, c_lat=128, d_txt=1024)
        wl = CF.Workload("sampler_wide_bf16", d, "bf16", ((64, 64, 1, 256), (64, 64, 1, 256)), img_budget=8192,
                         depth=2, steps=4, guidance=4.0)
        W = R.Weights(wl, source="torch")
    h, w = wl.samples[0][:2]
    eps = S.normal((h * w, wl.dims.c_lat), 1.0, "bf16", wl.name, "eps2")
    tau_c = S.text(24, wl.dims.d_txt, "bf16", wl.name, "tau_c2")
    tau_u = S.text(tu_len, wl.dims.d_txt, "bf16", wl.name, "tau_u2")
    src = S.normal((h * w, wl.dims.c_lat), 1.0, "bf16", wl.name, "src2") if case.startswith("edit") else None
    print(f"two-pass sampler {case} tu={tu_len}", flush=True)
    packed = R.Sampler(wl, W, eps, tau_c, tau_u, src=src)
    two = R.Sampler(wl, W, eps, tau_c, tau_u, two_pass=True, src=src)
    packed.run()
    two.run()
    torch.cuda.synchronize()
    assert torch.isfinite(packed.z).all()
    assert torch.equal(packed.z, two.z), (packed.z - two.z).abs().max()
    eager = two.z.clone()
    two.capture()
    two.z.zero_()
    two.replay()
    torch.cuda.synchronize()
    assert torch.equal(two.z, eager)


def test_sampler_graph_replays_match_eager():
    """A whole 4-step pack recorded as a HIP graph replays to the eager result,
    every time, with eager work and synchronisations in between."""
    from resolution_image_gen_amd import runner as R

    wl = _small_sampler_wl("bf16", depth=2)
    W = R.Weights(wl, recipe="stress")
    h, w = wl.samples[0][:2]
    eps = S.normal((h * w, wl.dims.c_lat), 1.0, "bf16", wl.name, "eps")
    tau_c = S.text(24, wl.dims.d_txt, "bf16", wl.name, "tau_c")
    tau_u = S.text(24, wl.dims.d_txt, "bf16", wl.name, "tau_u")
    sm = R.Sampler(wl, W, eps, tau_c, tau_u)
    sm.run()
    torch.cuda.synchronize()
    eager = sm.z.clone()
    sm.capture()
    for i in range(4):
        sm.z.zero_()
        junk = torch.randn(1000, 1000, device="cuda") @ torch.randn(1000, 1000, device="cuda")
        torch.cuda.synchronize()
        sm.replay()
        torch.cuda.synchronize()
        assert torch.equal(sm.z, eager), f"replay {i} differs"
        del junk


_SMALL_BF16 = CF.Dims(hidden=512, heads=4, head_dim=128, mlp=2048, c_lat=64, d_txt=512)


@pytest.mark.parametrize("name", ["tiny_f32", "pack256_bf16", "edit_small_bf16"])
def test_fused_rf_entries_same_bits(name):
    """rf_embed equals rf_make_xt then mmdit_embed, and rf_final_loss equals
    mmdit_final_mod then rf_loss, bit for bit.  The bf16 packs take the fused
    kernels (the noising in the image embedding's A staging; the loss's row
    sums in the final GEMM's split-K reduction), f32 runs the two in sequence;
    the edit pack has clean source rows (frame 1) next to the noised targets."""
    from resolution_image_gen_amd import binding as B
    from resolution_image_gen_amd import runner as R

    if name == "edit_small_bf16":
        wl = CF.Workload(name, _SMALL_BF16, "bf16", ((12, 10, 2, 24), (5, 7, 2, 3), (8, 8, 1, 16)),
                         img_budget=10 ** 6)
    else:
        wl = CF.WORKLOADS[name]
    print(f"fused rf entries {name}", flush=True)
    W = R.Weights(wl)
    inp = R.training_inputs(wl)
    tf = R.TrainForward(wl, W, inp)
    tf.run()
    torch.cuda.synchronize()
    pk, dm = tf.pk, tf.dims
    fused = wl.dtype == "bf16"
    # embedding
    zt1, x1, xt1 = torch.empty_like(tf.zt), torch.empty_like(tf.x_img), torch.empty_like(tf.x_txt)
    zt2, x2, xt2 = torch.empty_like(tf.zt), torch.empty_like(tf.x_img), torch.empty_like(tf.x_txt)
    B.timing_enable(True)
    B.rf_embed(dm, W.wrap["w_in"], W.wrap["w_txt"], pk, tf.z, tf.eps, tf.t, tf.tau, x1, xt1, zt1)
    rep = B.timing_report()
    B.timing_enable(False)
    B.rf_make_xt(pk, tf.z, tf.eps, tf.t, zt2)
    B.embed(dm, W.wrap["w_in"], W.wrap["w_txt"], pk, zt2, tf.tau, x2, xt2)
    torch.cuda.synchronize()
    n_img, n_txt = pk.n_img, pk.n_txt
    assert torch.equal(zt1[:n_img], zt2[:n_img])
    assert torch.equal(x1[:n_img], x2[:n_img])
    assert torch.equal(xt1[:n_txt], xt2[:n_txt])
    assert ("embed_img_xt" in rep and "make_xt_kernel" not in rep) == fused, sorted(rep)
    # final layer + loss on the blocks' output
    v1, v2 = torch.empty_like(tf.v), torch.empty_like(tf.v)
    s1, s2 = torch.empty_like(tf.sse), torch.empty_like(tf.sse)
    l1, l2 = torch.empty_like(tf.loss), torch.empty_like(tf.loss)
    B.timing_enable(True)
    B.rf_final_loss(dm, W.wrap["w_out"], pk, tf.side.modf, tf.x_img, tf.z, tf.eps, v1, s1, l1, tf.ws)
    rep = B.timing_report()
    B.timing_enable(False)
    B.final_mod(dm, W.wrap["w_out"], pk, tf.side.modf, tf.x_img, v2, tf.ws)
    B.rf_loss(pk, v2, tf.z, tf.eps, s2, l2, tf.ws)
    torch.cuda.synchronize()
    n_tgt = pk.n_tgt
    assert torch.equal(v1[:n_tgt], v2[:n_tgt])
    assert torch.equal(s1[:pk.B], s2[:pk.B])
    assert torch.equal(l1, l2)
    if name == "pack256_bf16":
        assert "splitk_reduce_sse_kernel" in rep and "row_sse_kernel" not in rep, sorted(rep)
    # the training forward (which calls both) matched its own unfused parts
    assert torch.equal(tf.v[:n_tgt], v2[:n_tgt]) and torch.equal(tf.loss, l2)


def test_sampler_all_steps_vectors_same_bits():
    """The packed sampler computes every step's adaLN vectors in one pass over
    the weights (4 steps x 2 samples = 8 rows of the weight-streaming GEMV);
    the result equals the per-step vectors' bit for bit."""
    from resolution_image_gen_amd import runner as R

    wl = _small_sampler_wl("bf16", depth=2)
    W = R.Weights(wl, recipe="stress")
    h, w = wl.samples[0][:2]
    eps = S.normal((h * w, wl.dims.c_lat), 1.0, "bf16", wl.name, "eps3")
    tau_c = S.text(24, wl.dims.d_txt, "bf16", wl.name, "tau_c3")
    tau_u = S.text(20, wl.dims.d_txt, "bf16", wl.name, "tau_u3")
    sm = R.Sampler(wl, W, eps, tau_c, tau_u)
    assert sm.all_steps
    sm.run()
    torch.cuda.synchronize()
    z_all = sm.z.clone()
    sm.all_steps = False
    sm.run()
    torch.cuda.synchronize()
    assert torch.equal(sm.z, z_all), (sm.z - z_all).abs().max()
