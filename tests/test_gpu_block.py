"""GPU parity of the whole block (mmdit_block_fwd) against the oracle.

Residual streams dominate the block output at N(0, 0.02) weights, so parity
is asserted on every intermediate the library exposes (workspace), on the
branch deltas x_out - x_in, and on a "stress" recipe whose weights
N(0, 1/sqrt(fan_in)) make every branch O(1).  Full-size packs (native 1024^2
and the 2048^2 edit pack) are checked on sampled rows the oracle computes one
by one.
"""

import numpy as np
import pytest
import torch

from helpers import TOL, assert_close, f64_block, oracle_pack, to_np
from oracle import block as OB
from resolution_image_gen_amd import configs as CF
from resolution_image_gen_amd import synthetic as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from resolution_image_gen_amd import binding

    return binding


def _tdt(dtype):
    return torch.float32 if dtype == "f32" else torch.bfloat16


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(_tdt(dtype))


def _dev_block(nb, dtype):
    return {s: {k: (torch.from_numpy(v).cuda() if k in ("g_q", "g_k") else _dev(v, dtype))
                for k, v in nb[s].items()} for s in nb}


def _inputs(d, dtype, samples, key, recipe="default"):
    ref = oracle_pack(samples)
    nb = S.block_weights(d, dtype, key, 0, recipe)
    if recipe == "stress":   # non-trivial QK-norm gains too
        for s in nb:
            nb[s]["g_q"] = (1 + 0.2 * S.normal((d.head_dim,), 1.0, "f32", key, s, "gq")).astype(np.float32)
            nb[s]["g_k"] = (1 + 0.2 * S.normal((d.head_dim,), 1.0, "f32", key, s, "gk")).astype(np.float32)
    x_img = S.residual(ref["cu_img"][-1], d.hidden, dtype, key, "x_img")
    x_txt = S.residual(max(ref["cu_txt"][-1], 1), d.hidden, dtype, key, "x_txt")[:ref["cu_txt"][-1]]
    c = S.normal((len(samples), d.hidden), 1.0, dtype, key, "c")
    return ref, nb, x_img, x_txt, c


def _run_block(B, d, dtype, samples, nb, x_img, x_txt, c):
    dims = B.Dims(d, dtype)
    pk = B.pack(samples)
    xi = _dev(x_img, dtype)
    xt = _dev(x_txt if len(x_txt) else np.zeros((1, d.hidden), np.float32), dtype)
    ws = torch.empty(B.workspace_size(dims, pk), dtype=torch.uint8, device="cuda")
    B.block_fwd(dims, _dev_block(nb, dtype), pk, _dev(c, dtype), xi, xt, ws)
    torch.cuda.synchronize()
    return dims, pk, xi, xt, ws


def _delta_tol(tol, dtype, x_out, delta):
    """Bound for the branch delta x_out - x_in of a block: the bar, plus the
    storage rounding of the residual stream.  The block stores x twice in the
    model dtype (after the attention branch and after the MLP branch), each a
    correctly rounded fused x + gate * branch, so the delta carries up to two
    half-ulps of |x| (unit roundoff 2^-9 in bf16, 2^-24 in float32) that no
    arithmetic can remove; relative to max|delta| that is
    2 u max|x_out| / max|delta|, large when the branches are small against x
    (N(0, 0.02) weights), negligible for the stress recipe."""
    u = 2.0 ** -9 if dtype == "bf16" else 2.0 ** -24
    return tol + 2 * u * float(np.max(np.abs(x_out))) / float(np.max(np.abs(delta)))


def _ws_view(ws, off, rows, cols, dtype):
    es = 4 if dtype == "f32" else 2
    t = ws[off:off + rows * cols * es].view(_tdt(dtype))
    return t.view(rows, cols)


BLOCK_CASES = {
    "tiny_f32": (CF.TINY, "f32", CF.WORKLOADS["tiny_f32"].samples, "default"),
    "tiny_f32_stress": (CF.TINY, "f32", CF.WORKLOADS["tiny_f32"].samples, "stress"),
    "tiny_f32_edit": (CF.TINY, "f32", [(6, 5, 2, 7), (3, 9, 1, 0), (2, 2, 2, 40)], "stress"),
    "pack256_bf16": (CF.B4, "bf16", CF.WORKLOADS["pack256_bf16"].samples, "default"),
    "pack256_bf16_stress": (CF.B4, "bf16", CF.WORKLOADS["pack256_bf16"].samples, "stress"),
    "ragged_bf16_stress": (CF.B4, "bf16", [(13, 11, 2, 33), (7, 20, 1, 0), (1, 1, 1, 5)], "stress"),
    # no text rows at all: single-problem launches, attention over image tokens only
    "no_text_bf16_stress": (CF.B4, "bf16", [(9, 14, 1, 0), (5, 6, 2, 0), (1, 3, 1, 0)], "stress"),
    # the largest pack the library takes (256 samples): per-sample offsets
    # crossing the 64-sample chunks of the pack kernels, many tiny attention
    # problems, per-sample adaLN vectors
    "max_samples_bf16_stress": (CF.B4, "bf16", [(1 + i % 3, 1 + i % 4, 1 + (i % 7 == 0), i % 5) for i in range(256)],
                                "stress"),
}


@pytest.mark.parametrize("case", list(BLOCK_CASES))
def test_block_fwd_vs_oracle(B, case):
    d, dtype, samples, recipe = BLOCK_CASES[case]
    print(f"block {case}", flush=True)
    ref, nb, x_img, x_txt, c = _inputs(d, dtype, samples, case, recipe)
    dims, pk, xi, xt, ws = _run_block(B, d, dtype, samples, nb, x_img, x_txt, c)
    want = OB.block_forward(x_img, x_txt, c, f64_block(nb), ref, d.heads)
    tol = TOL[dtype]
    H = d.hidden
    ni, nt = ref["cu_img"][-1], ref["cu_txt"][-1]
    got_i = to_np(xi)
    assert_close("x_out_img", got_i, want["x_out_img"], tol)
    dref = want["x_out_img"] - x_img
    assert_close("delta_img (x_out - x_in)", got_i - x_img, dref, _delta_tol(tol, dtype, want["x_out_img"], dref))
    if nt:
        got_t = to_np(xt)[:nt]
        assert_close("x_out_txt", got_t, want["x_out_txt"], tol)
        dref = want["x_out_txt"] - x_txt
        assert_close("delta_txt", got_t - x_txt, dref, _delta_tol(tol, dtype, want["x_out_txt"], dref))
    # intermediates kept in the workspace
    L = B.workspace_layout(dims, pk)
    N = ni + nt
    qkv = to_np(_ws_view(ws, L["qkv"], N, 3 * H, dtype))
    o = to_np(_ws_view(ws, L["o"], N, H, dtype))
    h2 = to_np(_ws_view(ws, L["h"], N, H, dtype))
    u = to_np(_ws_view(ws, L["u"], N, d.mlp, dtype))
    for s, r0, r1 in (("img", 0, ni), ("txt", ni, N)):
        if r1 == r0:
            continue
        n = r1 - r0
        assert_close(f"q_{s}", qkv[r0:r1, :H], want[f"q_{s}"].reshape(n, H), tol)
        assert_close(f"k_{s}", qkv[r0:r1, H:2 * H], want[f"k_{s}"].reshape(n, H), tol)
        assert_close(f"v_{s}", qkv[r0:r1, 2 * H:], want[f"v_{s}"].reshape(n, H), tol)
        # attention output: normwise, and row-wise per (token, head)
        assert_close(f"o_{s}", o[r0:r1].reshape(n * d.heads, d.head_dim),
                     want[f"o_{s}"].reshape(n * d.heads, d.head_dim), tol, rows=True)
        assert_close(f"h2_{s}", h2[r0:r1], want[f"h2_{s}"], tol)
        assert_close(f"u_{s}", u[r0:r1], want[f"u_{s}"], tol)
    mod_i = ws[L["mod_img"]:L["mod_img"] + len(samples) * 6 * H * 4].view(torch.float32).cpu().numpy()
    want_mod = np.concatenate(OB.modulation(c, nb["img"]["w_mod"]), axis=1).reshape(-1)
    assert_close("mod_img", mod_i, want_mod, tol)


def test_block_adaln_zero_is_identity(B):
    d, dtype = CF.B4, "bf16"
    samples = [(16, 16, 1, 64), (8, 12, 2, 10)]
    ref, nb, x_img, x_txt, c = _inputs(d, dtype, samples, "zero")
    for s in nb:
        nb[s]["w_mod"][:] = 0.0
    _, _, xi, xt, _ = _run_block(B, d, dtype, samples, nb, x_img, x_txt, c)
    assert np.array_equal(to_np(xi), x_img.astype(np.float64))
    assert np.array_equal(to_np(xt)[:len(x_txt)], x_txt.astype(np.float64))


@pytest.mark.parametrize("case", ["tiny_f32_edit", "ragged_bf16_stress"])
def test_split_modulation_calls_match_fused(B, case):
    """block_modulation + block_fwd_mod and modulation + final_mod, the calls
    the runner splits over two streams, end on the same bits as block_fwd and
    final."""
    d, dtype, samples, recipe = BLOCK_CASES[case]
    ref, nb, x_img, x_txt, c = _inputs(d, dtype, samples, case, recipe)
    dims, pk, xi1, xt1, ws = _run_block(B, d, dtype, samples, nb, x_img, x_txt, c)
    wb = _dev_block(nb, dtype)
    cd = _dev(c, dtype)
    mod = torch.full((2, len(samples), 6 * d.hidden), float("nan"), dtype=torch.float32, device="cuda")
    B.block_modulation(dims, wb, cd, mod)
    xi2 = _dev(x_img, dtype)
    xt2 = _dev(x_txt if len(x_txt) else np.zeros((1, d.hidden), np.float32), dtype)
    B.block_fwd_mod(dims, wb, pk, mod, xi2, xt2, ws)
    torch.cuda.synchronize()
    assert torch.equal(xi1, xi2) and torch.equal(xt1, xt2)
    # the vectors are W_mod SiLU(c) of each stream
    for si, st in enumerate(("img", "txt")):
        want = OB.silu(c.astype(np.float64)) @ nb[st]["w_mod"].astype(np.float64).T
        assert_close(f"mod[{st}]", to_np(mod[si]), want, TOL[dtype])
    # final layer
    wf = S.normal((2 * d.hidden, d.hidden), 0.02, dtype, case, "wf")
    wo = S.normal((d.c_lat, d.hidden), 0.02, dtype, case, "wo")
    v1 = torch.empty(pk.n_tgt, d.c_lat, dtype=_tdt(dtype), device="cuda")
    v2 = torch.full_like(v1, float("nan"))
    B.final(dims, _dev(wf, dtype), _dev(wo, dtype), pk, cd, xi1, v1, ws)
    modf = torch.empty(len(samples), 2 * d.hidden, dtype=torch.float32, device="cuda")
    B.modulation(dims, _dev(wf, dtype), 2, cd, modf)
    B.final_mod(dims, _dev(wo, dtype), pk, modf, xi1, v2, ws)
    torch.cuda.synchronize()
    assert torch.equal(v1, v2)


def test_block_deterministic_and_sample_order_invariant(B):
    d, dtype = CF.B4, "bf16"
    samples = [(16, 16, 1, 128), (9, 13, 1, 77), (5, 3, 2, 0), (1, 1, 1, 1)]
    ref, nb, x_img, x_txt, c = _inputs(d, dtype, samples, "perm", "stress")
    _, _, xi1, xt1, _ = _run_block(B, d, dtype, samples, nb, x_img, x_txt, c)
    _, _, xi2, xt2, _ = _run_block(B, d, dtype, samples, nb, x_img, x_txt, c)
    assert torch.equal(xi1, xi2) and torch.equal(xt1, xt2), "block_fwd is not bitwise reproducible"
    perm = [2, 0, 3, 1]
    cu_i, cu_t = ref["cu_img"], ref["cu_txt"]

    def cat(a, cu):
        return np.concatenate([a[cu[p]:cu[p + 1]] for p in perm])

    _, _, xi3, xt3, _ = _run_block(B, d, dtype, [samples[p] for p in perm], nb, cat(x_img, cu_i),
                                   cat(x_txt, cu_t), c[perm])
    a, b = xi1.cpu(), xi3.cpu()
    assert torch.equal(torch.cat([a[cu_i[p]:cu_i[p + 1]] for p in perm]), b), "image rows differ after permuting"
    a, b = xt1.cpu(), xt3.cpu()
    assert torch.equal(torch.cat([a[cu_t[p]:cu_t[p + 1]] for p in perm]), b[:cu_t[-1]]), "text rows differ"


@pytest.mark.parametrize("name", ["native1024_bf16", "edit2048_bf16", "sampler1024_cfg_bf16"])
def test_block_full_size_sampled_rows(B, name):
    """Full-size packs in the launch configuration of the benchmark; the oracle
    recomputes sampled rows of two samples from the block inputs.  At the
    1024^2 packed-CFG pack (408 MLP-down tiles: one full round of 256 CUs and
    a last round 59% full) the MLP down projection takes the stream-K last
    round: the second sample's image rows and all text rows lie in split
    tiles."""
    wl = CF.WORKLOADS[name]
    d, dtype, samples = wl.dims, wl.dtype, list(wl.samples)
    print(f"full-size {name}", flush=True)
    ref, nb, x_img, x_txt, c = _inputs(d, dtype, samples, name, "stress")
    _, _, xi, xt, _ = _run_block(B, d, dtype, samples, nb, x_img, x_txt, c)
    got_i, got_t = to_np(xi), to_np(xt)
    rng = np.random.default_rng(0)
    nbf = f64_block(nb)
    for b in sorted({0, len(samples) - 1}):
        Ii = ref["cu_img"][b + 1] - ref["cu_img"][b]
        Tt = ref["cu_txt"][b + 1] - ref["cu_txt"][b]
        # first, last, a band across the tile boundary, random rows
        irows = np.unique(np.concatenate([[0, Ii - 1], np.arange(120, 136), rng.integers(0, Ii, 24)]))
        trows = np.unique(np.concatenate([[0, Tt - 1], rng.integers(0, Tt, 8)]))
        want = OB.block_forward_rows(x_img, x_txt, c, nbf, ref, d.heads, b, irows, trows)
        i0, t0 = ref["cu_img"][b], ref["cu_txt"][b]
        assert_close(f"x_out_img[b={b}]", got_i[i0 + irows], want["x_out_img"], TOL[dtype])
        assert_close(f"delta_img[b={b}]", got_i[i0 + irows] - x_img[i0 + irows],
                     want["x_out_img"] - x_img[i0 + irows], TOL[dtype], rows=True)
        assert_close(f"delta_txt[b={b}]", got_t[t0 + trows] - x_txt[t0 + trows],
                     want["x_out_txt"] - x_txt[t0 + trows], TOL[dtype], rows=True)


def test_block_last_round_split_ragged_tail():
    """A pack whose four GEMMs span a few full rounds of 256x256 tiles on a
    256-CU device and end in a short last round: those tiles are computed as
    K chunks and summed by a second kernel.  The text rows (1218 of them) end
    in a ragged tile that falls in that last round; every text row of the last
    two samples and sampled image rows are checked."""
    from resolution_image_gen_amd import binding as B

    d = CF.Dims(hidden=1024, heads=8, head_dim=128, mlp=4096, c_lat=64, d_txt=1024)
    dtype = "bf16"
    samples = [(16, 24, 1, 29)] * 42
    print("last-round split, 42 x (384 + 29) rows, hidden 1024", flush=True)
    ref, nb, x_img, x_txt, c = _inputs(d, dtype, samples, "tailsplit", "stress")
    _, _, xi, xt, _ = _run_block(B, d, dtype, samples, nb, x_img, x_txt, c)
    got_i, got_t = to_np(xi), to_np(xt)
    nbf = f64_block(nb)
    rng = np.random.default_rng(1)
    for b in (40, 41):
        Ii = ref["cu_img"][b + 1] - ref["cu_img"][b]
        Tt = ref["cu_txt"][b + 1] - ref["cu_txt"][b]
        irows = np.unique(rng.integers(0, Ii, 16))
        trows = np.arange(Tt)
        want = OB.block_forward_rows(x_img, x_txt, c, nbf, ref, d.heads, b, irows, trows)
        i0, t0 = ref["cu_img"][b], ref["cu_txt"][b]
        assert_close(f"delta_img[b={b}]", got_i[i0 + irows] - x_img[i0 + irows],
                     want["x_out_img"] - x_img[i0 + irows], TOL[dtype], rows=True)
        assert_close(f"delta_txt[b={b}]", got_t[t0 + trows] - x_txt[t0 + trows],
                     want["x_out_txt"] - x_txt[t0 + trows], TOL[dtype], rows=True)


def test_block_sample_order_invariant_with_last_round_split():
    """Shapes like the test above's (last-round sub-tiles on a 256-CU device):
    reversing the samples moves rows between full tiles and shared last-round
    tiles, and every row must still come out bitwise the same."""
    from resolution_image_gen_amd import binding as B

    d = CF.Dims(hidden=1024, heads=8, head_dim=128, mlp=4096, c_lat=64, d_txt=1024)
    dtype = "bf16"
    samples = [(16, 24, 1, 29)] * 40 + [(8, 8, 1, 7), (20, 20, 1, 300)]
    print("sample order, 42 samples, hidden 1024", flush=True)
    ref, nb, x_img, x_txt, c = _inputs(d, dtype, samples, "tailperm", "stress")
    _, _, xi1, xt1, _ = _run_block(B, d, dtype, samples, nb, x_img, x_txt, c)
    perm = list(range(len(samples)))[::-1]
    cu_i, cu_t = ref["cu_img"], ref["cu_txt"]

    def cat(a, cu):
        return np.concatenate([a[cu[p]:cu[p + 1]] for p in perm])

    _, _, xi2, xt2, _ = _run_block(B, d, dtype, [samples[p] for p in perm], nb, cat(x_img, cu_i),
                                   cat(x_txt, cu_t), c[perm])
    a, b = xi1.cpu(), xi2.cpu()
    assert torch.equal(torch.cat([a[cu_i[p]:cu_i[p + 1]] for p in perm]), b), "image rows differ after permuting"
    a, b = xt1.cpu(), xt2.cpu()
    assert torch.equal(torch.cat([a[cu_t[p]:cu_t[p + 1]] for p in perm]), b[:cu_t[-1]]), "text rows differ"


def test_fused_qkv_epilogue_same_bits_as_separate_kernel(B):
    """At the 1024^2 packed-CFG shape (cond + uncond, 64x64 grid + 256 text
    each: 1,224 QKV tiles of 256x256, no last-round split on 256 CUs) the QKV
    projection applies QK-RMSNorm + RoPE in its LDS epilogue.  It must give
    the same bits as the plain projection followed by the separate QK kernel,
    recomputed here from the block's own pre-attention norm; the training
    forward's copy of q and k before their norm must equal the plain
    projection's."""
    import ctypes  # noqa: F401

    d, dtype = CF.B4, "bf16"
    samples = [(64, 64, 1, 256), (64, 64, 1, 256)]
    print("fused QKV epilogue at 2 x (64x64 + 256)", flush=True)
    ref, nb, x_img, x_txt, c = _inputs(d, dtype, samples, "qkfuse", "stress")
    dims, pk, xi, xt, ws = _run_block(B, d, dtype, samples, nb, x_img, x_txt, c)
    H = d.hidden
    ni, nt = int(ref["cu_img"][-1]), int(ref["cu_txt"][-1])
    L = B.workspace_layout(dims, pk)
    nbs = len(samples)
    wb = _dev_block(nb, dtype)
    fused = _ws_view(ws, L["qkv"], ni + nt, 3 * H, dtype).clone()
    raws = {}
    for s, r0, n, x, seg, pos in (("img", 0, ni, x_img, pk.t["seg_img"], pk.t["pos_img"]),
                                  ("txt", ni, nt, x_txt, pk.t["seg_txt"], None)):
        mod = ws[L["mod_" + s]:L["mod_" + s] + nbs * 6 * H * 4].view(torch.float32).view(nbs, 6 * H)
        h1 = torch.empty(n, H, dtype=torch.bfloat16, device="cuda")
        B.rms_modulate(dims, _dev(x, dtype), seg, mod, 0, H, h1)
        plain = torch.empty(n, 3 * H, dtype=torch.bfloat16, device="cuda")
        B.linear(h1, wb[s]["w_qkv"], plain, B.EPI_STORE)
        raws[s] = plain[:, :2 * H].clone()
        B.qk_norm_rope(dims, plain, pos, wb[s]["g_q"], wb[s]["g_k"])
        torch.cuda.synchronize()
        got = fused[r0:r0 + n]
        diff = (got.float() - plain.float()).abs().max().item()
        print(f"  {s}: max |fused - separate| = {diff:.3e}", flush=True)
        assert torch.equal(got, plain), s
    # training forward: same normalised q, k, v and the raw q, k kept
    saved = torch.empty(B.block_saved_size(dims, pk), dtype=torch.uint8, device="cuda")
    xi2, xt2 = _dev(x_img, dtype), _dev(x_txt, dtype)
    B.block_fwd_train(dims, wb, pk, _dev(c, dtype), xi2, xt2, saved, ws)
    torch.cuda.synchronize()
    assert torch.equal(xi2, xi) and torch.equal(xt2, xt)

    def a256(x):
        return (x + 255) // 256 * 256

    # saved layout: mod_img, mod_txt [B, 6H] f32; x_in, h1 [N, H]; qkv [N, 3H]; qk_raw [N, 2H] (bf16)
    N = ni + nt
    off = a256(a256(nbs * 6 * H * 4) + nbs * 6 * H * 4)
    off = a256(off + N * H * 2)                    # x_in
    off = a256(off + N * H * 2)                    # h1
    qkv_s = saved[off:off + N * 3 * H * 2].view(torch.bfloat16).view(N, 3 * H)
    off = a256(off + N * 3 * H * 2)
    raw_s = saved[off:off + N * 2 * H * 2].view(torch.bfloat16).view(N, 2 * H)
    assert torch.equal(qkv_s, fused)
    assert torch.equal(raw_s[:ni], raws["img"]) and torch.equal(raw_s[ni:], raws["txt"])
