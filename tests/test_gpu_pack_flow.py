"""GPU parity: packing (bit-exact) and the rectified-flow kernels."""

import numpy as np
import pytest
import torch

from helpers import TOL, assert_close, oracle_pack, to_np
from oracle import flow as OF

pytestmark = pytest.mark.gpu

SAMPLE_SETS = {
    "tiny": [(16, 16, 1, 32), (8, 8, 1, 32)],
    "pack256": [(16, 16, 1, 128)] * 16,
    "native1024": [(64, 64, 1, 256), (48, 84, 1, 256), (84, 48, 1, 256), (32, 128, 1, 256)],
    "edit2048": [(128, 128, 2, 512)],
    "ragged": [(3, 5, 2, 7), (1, 1, 1, 0), (4, 2, 2, 3)],
    "no_text": [(7, 9, 1, 0)],
    "many": [(1 + i % 3, 2 + i % 5, 1 + i % 2, i % 4) for i in range(70)],
    "max_samples": [(1 + i % 4, 1 + i % 3, 1 + i % 2, i % 6) for i in range(256)],
    # long samples whose target rows start and end off 4-row boundaries
    "long_ragged": [(3, 5, 1, 0), (127, 129, 1, 0), (1, 7, 2, 3), (64, 65, 1, 0)],
    # past 131,072 target rows (the loss's per-sample sums take one block per
    # sample), sample boundaries off 4-row boundaries
    "large_ragged": [(257, 259, 1, 0), (3, 5, 1, 0), (255, 255, 1, 0)],
}


@pytest.fixture(scope="module")
def B():
    from resolution_image_gen_amd import binding

    return binding


@pytest.mark.parametrize("name", list(SAMPLE_SETS))
def test_pack_bit_exact(B, name):
    samples = SAMPLE_SETS[name]
    print(f"pack {name}: {len(samples)} samples", flush=True)
    pk = B.pack(samples)
    torch.cuda.synchronize()
    ref = oracle_pack(samples)
    assert pk.B == ref["B"] and pk.max_joint == ref["max_joint"]
    assert pk.n_img == ref["cu_img"][-1] and pk.n_txt == ref["cu_txt"][-1] and pk.n_tgt == ref["cu_tgt"][-1]
    for key in ("cu_txt", "cu_img", "cu_joint", "cu_tgt"):
        np.testing.assert_array_equal(pk.t[key].cpu().numpy(), ref[key], err_msg=key)
    np.testing.assert_array_equal(pk.t["tgt_len"].cpu().numpy()[:pk.B], ref["tgt_len"])
    n_img, n_txt, n_tgt = pk.n_img, pk.n_txt, pk.n_tgt
    np.testing.assert_array_equal(pk.t["seg_img"].cpu().numpy()[:n_img], ref["seg_img"])
    np.testing.assert_array_equal(pk.t["seg_txt"].cpu().numpy()[:n_txt], ref["seg_txt"])
    np.testing.assert_array_equal(pk.t["pos_img"].cpu().numpy()[:3 * n_img].reshape(-1, 3), ref["pos_img"])
    np.testing.assert_array_equal(pk.t["tgt_row"].cpu().numpy()[:n_tgt], ref["tgt_rows"])
    # plan on the host agrees with the oracle plan
    from oracle import pack as OP

    budget = max(ref["cu_img"][-1], 1)
    joint = budget + ref["cu_txt"][-1]
    assert B.pack_plan(samples, budget) == OP.plan(samples, budget)
    assert B.pack_plan(samples, budget, joint) == OP.plan(samples, budget, joint)
    half = max(ref["max_joint"], joint // 2)
    assert B.pack_plan(samples, budget, half) == OP.plan(samples, budget, half)


def test_pack_plan_errors(B):
    with pytest.raises(B.MmditError) as e:
        B.pack_plan([(128, 128, 2, 0)], 16384)
    assert e.value.status == -2
    with pytest.raises(B.MmditError):
        B.pack_plan([(0, 4, 1, 0)], 100)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gather_bit_exact(B, dtype):
    samples = SAMPLE_SETS["ragged"]
    pk = B.pack(samples)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    g = torch.Generator(device="cuda").manual_seed(1)
    for which, key in ((0, "h_cu_img"), (1, "h_cu_txt"), (2, "h_cu_tgt")):
        cu = pk.host(key)
        srcs = [torch.randn(cu[b + 1] - cu[b], 64, device="cuda", generator=g).to(dt) for b in range(pk.B)]
        out = torch.full((max(cu[-1], 1), 64), float("nan"), device="cuda", dtype=dt)
        B.pack_gather(pk, which, srcs, out)
        torch.cuda.synchronize()
        want = torch.cat(srcs)
        assert torch.equal(out[:cu[-1]], want), which


def _rf_inputs(samples, C, dtype, seed=0):
    from resolution_image_gen_amd import synthetic as S

    ref = oracle_pack(samples)
    n = ref["cu_img"][-1]
    z = S.normal((n, C), 1.0, dtype, "rf", seed, "z")
    eps = S.normal((n, C), 1.0, dtype, "rf", seed, "eps")
    t = S.uniform((len(samples),), "f32", "rf", seed, "t")
    return ref, z, eps, t


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", ["ragged", "native1024", "edit2048"])
def test_make_xt(B, dtype, name):
    samples = SAMPLE_SETS[name]
    C = 128
    ref, z, eps, t = _rf_inputs(samples, C, dtype)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    pk = B.pack(samples)
    zd, ed = torch.from_numpy(z).cuda().to(dt), torch.from_numpy(eps).cuda().to(dt)
    td = torch.from_numpy(t).cuda()
    zt = torch.empty_like(zd)
    B.rf_make_xt(pk, zd, ed, td, zt)
    want = OF.make_xt(z, eps, t, ref)
    assert_close(f"zt[{name},{dtype}]", to_np(zt), want, TOL[dtype] if dtype == "bf16" else 1e-6)
    # source rows are copied bit-exactly; t = 0 and t = 1 give z and eps on target rows
    src = np.setdiff1d(np.arange(len(z)), ref["tgt_rows"])
    assert np.array_equal(to_np(zt)[src], z[src].astype(np.float64))
    B.rf_make_xt(pk, zd, ed, torch.zeros_like(td), zt)
    assert torch.equal(zt, zd)
    B.rf_make_xt(pk, zd, ed, torch.ones_like(td), zt)
    rows = torch.from_numpy(ref["tgt_rows"]).cuda()
    assert torch.equal(zt[rows], ed[rows])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", ["ragged", "pack256", "edit2048", "many", "long_ragged", "large_ragged"])
def test_rf_loss(B, dtype, name):
    samples = SAMPLE_SETS[name]
    C = 64
    ref, z, eps, _ = _rf_inputs(samples, C, dtype, seed=1)
    from resolution_image_gen_amd import synthetic as S

    v = S.normal((ref["cu_tgt"][-1], C), 1.0, dtype, "rf", name, "v")
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    pk = B.pack(samples)
    vd, zd, ed = (torch.from_numpy(a).cuda().to(dt) for a in (v, z, eps))
    sse = torch.empty(pk.B, device="cuda")
    loss = torch.empty(1, device="cuda")
    ws = torch.empty(pk.n_tgt * 4 + 256, dtype=torch.uint8, device="cuda")
    B.rf_loss(pk, vd, zd, ed, sse, loss, ws)
    want_sse, want_loss = OF.loss(v, z, eps, ref)
    assert_close(f"sse[{name},{dtype}]", to_np(sse), want_sse, 1e-5)
    assert abs(loss.item() - want_loss) <= 1e-5 * abs(want_loss)
    # exact target velocity gives zero loss; source-row eps is never read into the loss
    B.rf_loss(pk, vd, zd, ed, sse, loss, ws)
    first = sse.clone()
    ed2 = ed.clone()
    src = np.setdiff1d(np.arange(len(z)), ref["tgt_rows"])
    if len(src):
        ed2[torch.from_numpy(src).cuda()] += 100.0
    B.rf_loss(pk, vd, zd, ed2, sse, loss, ws)
    assert torch.equal(sse, first)            # also: deterministic, bitwise
    if dtype == "f32":
        rows = torch.from_numpy(ref["tgt_rows"]).cuda()
        vt = (zd[rows] - ed[rows]).contiguous()
        B.rf_loss(pk, vt, zd, ed, sse, loss, ws)
        assert torch.all(sse == 0) and loss.item() == 0.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name", ["ragged", "pack256", "edit2048", "many", "long_ragged", "large_ragged"])
def test_rf_nft_loss(B, dtype, name):
    """Negative-aware loss against the oracle's definition; rewards of 1 give
    rf_loss(v_pos) bit for bit, rewards of 0 rf_loss(v_neg)."""
    samples = SAMPLE_SETS[name]
    C = 64
    ref, z, eps, _ = _rf_inputs(samples, C, dtype, seed=2)
    from resolution_image_gen_amd import synthetic as S

    n_tgt = ref["cu_tgt"][-1]
    vp = S.normal((n_tgt, C), 1.0, dtype, "nft", name, "v_pos")
    vn = S.normal((n_tgt, C), 1.0, dtype, "nft", name, "v_neg")
    r = S.uniform((len(samples),), "f32", "nft", name, "r")
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    pk = B.pack(samples)
    vpd, vnd, zd, ed = (torch.from_numpy(a).cuda().to(dt) for a in (vp, vn, z, eps))
    rd = torch.from_numpy(r).cuda()
    sse = torch.empty(pk.B, device="cuda")
    loss = torch.empty(1, device="cuda")
    ws = torch.empty(pk.n_tgt * 4 + 256, dtype=torch.uint8, device="cuda")
    print(f"rf_nft_loss {name} {dtype}: {pk.B} samples, {pk.n_tgt} target rows", flush=True)
    B.rf_nft_loss(pk, vpd, vnd, zd, ed, rd, sse, loss, ws)
    want_sse, want_loss = OF.nft_loss(vp, vn, z, eps, r, ref)
    assert_close(f"nft sse[{name},{dtype}]", to_np(sse), want_sse, 1e-5)
    assert abs(loss.item() - want_loss) <= 1e-5 * abs(want_loss)
    first = sse.clone()
    B.rf_nft_loss(pk, vpd, vnd, zd, ed, rd, sse, loss, ws)
    assert torch.equal(sse, first)                      # deterministic, bitwise
    sse2, loss2 = torch.empty_like(sse), torch.empty_like(loss)
    for rv, vd in ((1.0, vpd), (0.0, vnd)):
        B.rf_nft_loss(pk, vpd, vnd, zd, ed, torch.full_like(rd, rv), sse, loss, ws)
        B.rf_loss(pk, vd, zd, ed, sse2, loss2, ws)
        assert torch.equal(sse, sse2) and torch.equal(loss, loss2), rv


def test_rf_loss_past_the_launch_grid_cap(B):
    """More target rows (2 x 8,388,608 + 4,096 > 2^24) than one 16-lane group
    per row of the largest grid the host launches: the groups stride over the
    rest (the whole last sample lies past 2^24 rows).  Closed form: z = eps,
    v = 0 except planted rows of ones, so each SSE is C times its planted
    rows, exactly."""
    C = 8
    samples = [(2048, 4096, 1, 0), (2048, 4096, 1, 0), (64, 64, 1, 0)]
    lens = [h * w for h, w, _, _ in samples]
    starts = np.concatenate([[0], np.cumsum(lens)])
    print("rf_loss, 16,781,312 target rows", flush=True)
    pk = B.pack(samples)
    n = pk.n_tgt
    assert n == sum(lens) and n > 1 << 24 and starts[2] >= 1 << 24
    g = torch.Generator(device="cuda").manual_seed(7)
    z = torch.randint(-4, 5, (n, C), device="cuda", generator=g).float()
    eps = z.clone()
    v = torch.zeros(n, C, device="cuda")
    planted = {0: [0], 1: [100, lens[1] - 1], 2: [0, 17, lens[2] - 1]}
    for b, rows in planted.items():
        for r in rows:
            v[int(starts[b]) + r] = 1.0
    sse = torch.empty(len(samples), device="cuda")
    loss = torch.empty(1, device="cuda")
    ws = torch.full((n * 4 + 256,), 255, dtype=torch.uint8, device="cuda")   # NaN until written
    B.rf_loss(pk, v, z, eps, sse, loss, ws)
    want = torch.tensor([float(C * len(planted[b])) for b in range(len(samples))], device="cuda")
    assert torch.equal(sse, want), (sse, want)
    want_loss = sum(C * len(planted[b]) / (lens[b] * C) for b in range(len(samples))) / len(samples)
    assert abs(loss.item() - want_loss) <= 1e-6 * want_loss
    del z, eps, v, ws
    torch.cuda.empty_cache()


def test_euler_exact_on_linear_flow(B):
    # z_1 = eps and v == z* - eps: four Euler steps land on z*
    from resolution_image_gen_amd import synthetic as S

    C = 128
    pk = B.pack([(8, 16, 1, 4), (8, 16, 1, 4)])
    zs = S.normal((128, C), 1.0, "bf16", "euler", "zstar")
    eps = S.normal((128, C), 1.0, "bf16", "euler", "eps")
    vrow = torch.from_numpy(zs - eps).cuda().to(torch.float32)     # exact in f32
    v = torch.cat([vrow, vrow]).contiguous()
    z = torch.from_numpy(eps).cuda().clone()
    zt = torch.zeros(pk.n_img, C, device="cuda")
    sched = OF.SCHEDULE
    for i in range(4):
        B.rf_euler_step(pk, v, 0, 1, 4.0, sched[i], sched[i + 1], z, zt)
    torch.cuda.synchronize()
    err = np.max(np.abs(z.cpu().numpy().astype(np.float64) - zs))
    print(f"  euler linear-flow max abs err {err:.3e}", flush=True)
    assert err <= 4 * 2.0 ** -23 * 8
    assert torch.equal(zt[:128], z) and torch.equal(zt[128:], z)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cfg_euler_against_oracle(B, dtype):
    from resolution_image_gen_amd import synthetic as S

    C = 128
    samples = [(12, 20, 1, 9), (12, 20, 1, 5)]
    pk = B.pack(samples)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    v = S.normal((480, C), 1.0, dtype, "cfg", "v")
    z0 = S.normal((240, C), 1.0, "f32", "cfg", "z")
    vd = torch.from_numpy(v).cuda().to(dt)
    for g in (0.0, 1.0, 4.0):
        z = torch.from_numpy(z0).cuda().clone()
        zt = torch.zeros(480, C, device="cuda", dtype=dt)
        B.rf_euler_step(pk, vd, 0, 1, g, 0.75, 0.5, z, zt)
        want = OF.euler_step(z0, OF.cfg_combine(v[:240], v[240:], g), 0.75, 0.5)
        assert_close(f"euler g={g}", (z.cpu().numpy() - z0) / 0.25, (want - z0) / 0.25, 1e-6)
        assert torch.equal(zt[:240], z.to(dt)) and torch.equal(zt[240:], z.to(dt))
    # v_c == v_u gives v_u for any guidance: bitwise equal to the unguided step
    vsame = torch.cat([vd[:240], vd[:240]]).contiguous()
    z1 = torch.from_numpy(z0).cuda().clone()
    z2 = torch.from_numpy(z0).cuda().clone()
    B.rf_euler_step(pk, vsame, 0, 1, 4.0, 0.75, 0.5, z1)
    B.rf_euler_step(pk, vsame, 0, -1, 0.0, 0.75, 0.5, z2)
    assert torch.equal(z1, z2)


def test_pack_latent(B):
    pk = B.pack([(4, 4, 1, 2), (4, 4, 1, 3)])
    z = torch.randn(16, 64, device="cuda")
    zt = torch.zeros(32, 64, device="cuda", dtype=torch.bfloat16)
    B.rf_pack_latent(pk, z, 0, 1, zt)
    assert torch.equal(zt[:16], z.to(torch.bfloat16)) and torch.equal(zt[16:], z.to(torch.bfloat16))


def test_empty_pack_calls_are_no_ops(B):
    """A pack of no samples: every call returns without launching work on the
    caller's buffers; the loss of nothing is 0."""
    from resolution_image_gen_amd import configs as CF
    from resolution_image_gen_amd import synthetic as S

    pk = B.pack([])
    assert (pk.B, pk.n_img, pk.n_txt, pk.n_tgt) == (0, 0, 0, 0)
    d = CF.TINY
    dims = B.Dims(d, "f32")
    f = dict(dtype=torch.float32, device="cuda")
    C, H = d.c_lat, d.hidden
    z, eps, zt = (torch.full((1, C), 7.0, **f) for _ in range(3))
    t = torch.full((1,), 0.5, **f)
    B.rf_make_xt(pk, z, eps, t, zt)
    sse = torch.full((1,), 7.0, **f)
    loss = torch.full((1,), 7.0, **f)
    B.rf_loss(pk, z, z, eps, sse, loss, torch.empty(256, dtype=torch.uint8, device="cuda"))
    wb = {s: {k: torch.from_numpy(v).cuda() for k, v in w.items()}
          for s, w in S.block_weights(d, "f32", "empty", 0).items()}
    x_img, x_txt, c = (torch.full((1, H), 7.0, **f) for _ in range(3))
    ws = torch.empty(max(B.workspace_size(dims, pk), 256), dtype=torch.uint8, device="cuda")
    B.block_fwd(dims, wb, pk, c, x_img, x_txt, ws)
    mod = torch.full((2, 1, 6 * H), 7.0, **f)
    B.block_fwd_mod(dims, wb, pk, mod, x_img, x_txt, ws)
    v = torch.full((1, C), 7.0, **f)
    w_f, w_o = torch.zeros(2 * H, H, **f), torch.zeros(C, H, **f)
    B.final(dims, w_f, w_o, pk, c, x_img, v, ws)
    w_in, w_txt = torch.zeros(H, C, **f), torch.zeros(H, d.d_txt, **f)
    tau = torch.full((1, d.d_txt), 7.0, **f)
    B.rf_embed(dims, w_in, w_txt, pk, z, eps, t, tau, x_img, x_txt, zt)
    modf = torch.full((1, 2 * H), 7.0, **f)
    loss2 = torch.full((1,), 7.0, **f)
    B.rf_final_loss(dims, w_o, pk, modf, x_img, z, eps, v, sse, loss2, ws)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and loss2.item() == 0.0
    for a in (zt, sse, x_img, x_txt, v):
        assert torch.all(a == 7.0)
