"""GPU parity of each kernel of the block against the oracle, on seeded inputs."""

import numpy as np
import pytest
import torch

from helpers import TOL, assert_close, oracle_pack, to_np
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


CASES = {
    # name: (dims, dtype, samples)
    "tiny_f32": (CF.TINY, "f32", [(16, 16, 1, 32), (8, 8, 1, 32)]),
    "ragged_bf16_d128": (CF.B4, "bf16", [(16, 16, 1, 128), (9, 13, 1, 77), (5, 3, 2, 0), (1, 1, 1, 1)]),
    "ragged_bf16_d64": (CF.Dims(hidden=512, heads=8, head_dim=64, mlp=2048, c_lat=64, d_txt=512), "bf16",
                        [(11, 7, 2, 19), (4, 4, 1, 64), (1, 2, 1, 0)]),
    # long samples: many 64-key tiles per query block, ragged last tiles
    "long_bf16_d128": (CF.B4, "bf16", [(48, 50, 1, 37), (40, 52, 1, 100), (3, 5, 1, 7)]),
    "long_bf16_d64": (CF.Dims(hidden=512, heads=8, head_dim=64, mlp=2048, c_lat=64, d_txt=512), "bf16",
                      [(50, 44, 1, 19), (21, 30, 2, 33)]),
    # a sample past 16384 joint tokens (also run with 256-query blocks of 8 waves)
    "long16k_bf16_d128": (CF.Dims(hidden=256, heads=2, head_dim=128, mlp=1024, c_lat=64, d_txt=256), "bf16",
                          [(128, 130, 1, 210), (7, 9, 1, 30)]),
    "long16k_bf16_d64": (CF.Dims(hidden=256, heads=4, head_dim=64, mlp=1024, c_lat=64, d_txt=256), "bf16",
                         [(128, 130, 1, 210), (3, 5, 1, 7)]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_rms_modulate(B, case):
    d, dtype, samples = CASES[case]
    ref = oracle_pack(samples)
    dims = B.Dims(d, dtype)
    pk = B.pack(samples)
    H = d.hidden
    x = S.normal((ref["cu_img"][-1], H), 1.5, dtype, "k2", case, "x")
    mod = S.normal((len(samples), 6 * H), 0.5, "f32", "k2", case, "mod")
    y = torch.empty(x.shape, dtype=_tdt(dtype), device="cuda")
    modd = torch.from_numpy(mod).cuda()
    B.rms_modulate(dims, _dev(x, dtype), pk.t["seg_img"], modd, 3 * H, 4 * H, y)
    seg = ref["seg_img"]
    want = OB.modulate(OB.rms_norm(x.astype(np.float64)), mod[seg, 3 * H:4 * H], mod[seg, 4 * H:5 * H])
    assert_close(f"rms_modulate[{case}]", to_np(y), want, TOL[dtype] if dtype == "bf16" else 1e-5)
    # target-row gather used by the final layer
    yt = torch.empty((ref["cu_tgt"][-1], H), dtype=_tdt(dtype), device="cuda")
    B.rms_modulate(dims, _dev(x, dtype), pk.t["seg_img"], modd, 0, H, yt, row_map=pk.t["tgt_row"])
    rows = ref["tgt_rows"]
    want = OB.modulate(OB.rms_norm(x[rows].astype(np.float64)), mod[seg[rows], :H], mod[seg[rows], H:2 * H])
    assert_close(f"rms_modulate_tgt[{case}]", to_np(yt), want, TOL[dtype] if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("case", list(CASES))
def test_qk_norm_rope(B, case):
    d, dtype, samples = CASES[case]
    ref = oracle_pack(samples)
    dims = B.Dims(d, dtype)
    pk = B.pack(samples)
    H, D, heads = d.hidden, d.head_dim, d.heads
    n = ref["cu_img"][-1]
    qkv = S.normal((n, 3 * H), 1.0, dtype, "k3", case, "qkv")
    gq = 1 + 0.1 * S.normal((D,), 1.0, "f32", "k3", case, "gq")
    gk = 1 + 0.1 * S.normal((D,), 1.0, "f32", "k3", case, "gk")
    for pos_mode in ("image", "text"):
        t = _dev(qkv, dtype)
        pos = pk.t["pos_img"] if pos_mode == "image" else None
        B.qk_norm_rope(dims, t, pos, torch.from_numpy(gq).cuda(), torch.from_numpy(gk).cuda())
        p = ref["pos_img"] if pos_mode == "image" else np.zeros((n, 3))
        q = OB.apply_rope(OB.rms_norm(qkv[:, :H].reshape(n, heads, D).astype(np.float64)) * gq, p)
        k = OB.apply_rope(OB.rms_norm(qkv[:, H:2 * H].reshape(n, heads, D).astype(np.float64)) * gk, p)
        got = to_np(t)
        tol = TOL[dtype] if dtype == "bf16" else 1e-5
        assert_close(f"q[{case},{pos_mode}]", got[:, :H], q.reshape(n, H), tol)
        assert_close(f"k[{case},{pos_mode}]", got[:, H:2 * H], k.reshape(n, H), tol)
        assert np.array_equal(got[:, 2 * H:], qkv[:, 2 * H:].astype(np.float64)), "v must pass through"


@pytest.mark.parametrize("bands", [(0, 64, 64), (64, 32, 32), (128, 0, 0)])
def test_qk_norm_rope_other_bands(B, bands):
    """Band widths other than the default split (frame, row, col) =
    (32, 48, 48): the rotation table follows mmdit_dims.rope_dims."""
    import dataclasses

    from resolution_image_gen_amd import configs as CF

    d = dataclasses.replace(CF.B4, rope_dims=bands)
    samples = [(5, 7, 2, 3), (16, 9, 1, 4)]
    ref = oracle_pack(samples)
    dims = B.Dims(d, "f32")
    pk = B.pack(samples)
    H, D, heads = d.hidden, d.head_dim, d.heads
    n = ref["cu_img"][-1]
    qkv = S.normal((n, 3 * H), 1.0, "f32", "k3b", str(bands), "qkv")
    gq = 1 + 0.1 * S.normal((D,), 1.0, "f32", "k3b", str(bands), "gq")
    gk = np.ones(D, np.float32)
    t = _dev(qkv, "f32")
    B.qk_norm_rope(dims, t, pk.t["pos_img"], torch.from_numpy(gq).cuda(), torch.from_numpy(gk).cuda())
    q = OB.apply_rope(OB.rms_norm(qkv[:, :H].reshape(n, heads, D).astype(np.float64)) * gq, ref["pos_img"],
                      bands=bands)
    k = OB.apply_rope(OB.rms_norm(qkv[:, H:2 * H].reshape(n, heads, D).astype(np.float64)) * gk, ref["pos_img"],
                      bands=bands)
    got = to_np(t)
    assert_close(f"q[{bands}]", got[:, :H], q.reshape(n, H), 1e-5)
    assert_close(f"k[{bands}]", got[:, H:2 * H], k.reshape(n, H), 1e-5)


@pytest.mark.parametrize("case", list(CASES))
def test_attention(B, case, monkeypatch):
    d, dtype, samples = CASES[case]
    ref = oracle_pack(samples)
    dims = B.Dims(d, dtype)
    pk = B.pack(samples)
    H, D, heads = d.hidden, d.head_dim, d.heads
    ni, nt = ref["cu_img"][-1], ref["cu_txt"][-1]
    # q, k like QK-normed vectors (entries ~N(0,1), norm sqrt(D)), scaled so softmax is peaked
    qi = S.normal((ni, 3 * H), 1.0, dtype, "k5", case, "img")
    qt = S.normal((max(nt, 1), 3 * H), 1.0, dtype, "k5", case, "txt")
    qi[:, :H] *= 2.0
    qt[:, :H] *= 2.0
    qi, qt = S.round_bf16(qi) if dtype == "bf16" else qi, S.round_bf16(qt) if dtype == "bf16" else qt
    oi = torch.full((ni, H), float("nan"), dtype=_tdt(dtype), device="cuda")
    ot = torch.full((max(nt, 1), H), float("nan"), dtype=_tdt(dtype), device="cuda")
    B.attention(dims, pk, _dev(qi, dtype), _dev(qt, dtype), oi, ot)

    def split(a, n):
        a = a[:n].astype(np.float64)
        return [a[:, i * H:(i + 1) * H].reshape(n, heads, D) for i in range(3)]

    want_t, want_i = OB.packed_attention(*split(qt, nt), *split(qi, ni), ref)
    tol = TOL[dtype] if dtype == "bf16" else 1e-5
    assert_close(f"o_img[{case}]", to_np(oi), want_i.reshape(ni, H), tol)
    if nt:
        assert_close(f"o_txt[{case}]", to_np(ot)[:nt], want_t.reshape(nt, H), tol)
    if dtype == "bf16" and case.startswith("long"):
        # every query takes the same keys in the same order whatever the block
        # shape: 8-wave blocks give the same bits
        oi8, ot8 = torch.empty_like(oi), torch.empty_like(ot)
        monkeypatch.setenv("MMDIT_ATTN_WAVES", "8")
        B.attention(dims, pk, _dev(qi, dtype), _dev(qt, dtype), oi8, ot8)
        torch.cuda.synchronize()
        monkeypatch.delenv("MMDIT_ATTN_WAVES")
        assert torch.equal(oi8, oi) and torch.equal(ot8[:nt], ot[:nt])


LINEAR_CASES = [
    # (dtype, M, N, K, epilogue, a_silu)   -- covers each kernel path and epilogue
    ("f32", 300, 192, 96, 0, False),
    ("f32", 77, 320, 256, 2, False),
    ("f32", 5, 1536, 256, 1, True),
    ("bf16", 1000, 384, 256, 0, False),       # MFMA 128x128, ragged M
    ("bf16", 4096, 4096, 128, 0, False),      # MFMA 256x128
    ("bf16", 4000, 8192, 128, 2, False),      # MFMA 256x256, ragged M, GELU (two rounds: persistent blocks)
    ("bf16", 4500, 8192, 128, 2, False),      # persistent blocks + last-round sub-tiles in one launch, GELU
    ("bf16", 4500, 8192, 192, 3, False),      # persistent blocks, gated residual, ragged M
    ("bf16", 4096, 8192, 256, 0, False),      # persistent blocks, plain store
    ("bf16", 300, 512, 128, 1, True),         # MFMA with SiLU on A (M > 16), float32 out
    ("bf16", 515, 320, 192, 2, False),        # MFMA 128x64 (N % 128 != 0), GELU
    ("bf16", 700, 256, 512, 3, False),        # gated residual
    ("bf16", 5, 1024, 512, 1, True),          # skinny, float32 out, SiLU on A
    ("bf16", 16, 768, 256, 0, True),          # skinny, M = 16
    ("bf16", 40, 100, 72, 0, False),          # shapes outside the MFMA kernels: SIMT bf16
]


@pytest.mark.parametrize("dtype,M,N,K,epi,silu", LINEAR_CASES)
def test_linear(B, dtype, M, N, K, epi, silu):
    key = ("lin", dtype, M, N, K, epi)
    A = S.normal((M, K), 1.0, dtype, *key, "A")
    W = S.normal((N, K), 1.0 / np.sqrt(K), dtype, *key, "W")
    seg = (np.arange(M) * 3 // max(M, 1)).astype(np.int32)
    gate = S.normal((3, N + 32), 1.0, "f32", *key, "gate")
    Y0 = S.normal((M, N), 1.0, dtype, *key, "Y0")
    out_dt = torch.float32 if epi == 1 else _tdt(dtype)
    Y = torch.from_numpy(Y0).cuda().to(out_dt)
    B.linear(_dev(A, dtype), _dev(W, dtype), Y, epilogue=epi,
             gate=torch.from_numpy(gate).cuda() if epi == 3 else None, gate_stride=N + 32,
             seg=torch.from_numpy(seg).cuda() if epi == 3 else None, a_silu=silu)
    a = A.astype(np.float64)
    if silu:
        a = OB.silu(a)
    y = OB.linear(a, W)
    if epi == 2:
        y = OB.gelu(y)
    if epi == 3:
        want = Y0.astype(np.float64) + gate[seg, :N] * y
        assert_close("gated residual delta", to_np(Y) - Y0, want - Y0, TOL[dtype] if dtype == "bf16" else 1e-5)
        return
    tol = TOL[dtype] if (dtype == "bf16") else 1e-5
    assert_close(f"linear {key}", to_np(Y), y, tol)


@pytest.mark.parametrize("epi", [0, 2])
def test_linear_rows_independent_of_launch(B, epi):
    """The 1024^2 packed-CFG pack's MLP up shape (8,704 x 12,288 x 3,072: a
    persistent launch with last-round sub-tiles) gives every row the bits the
    same row gets in a launch of 256 rows (one round, other tiles): each
    element takes the same k order in every tile shape."""
    M, N, K = 8704, 12288, 3072
    g = torch.Generator(device="cuda").manual_seed(7)
    A = torch.randn(M, K, generator=g, device="cuda").to(torch.bfloat16)
    W = (torch.randn(N, K, generator=g, device="cuda") * K ** -0.5).to(torch.bfloat16)
    Y = torch.empty(M, N, device="cuda", dtype=torch.bfloat16)
    B.linear(A, W, Y, epilogue=epi)
    for r0 in (0, 4224, M - 256):
        Ys = torch.empty(256, N, device="cuda", dtype=torch.bfloat16)
        B.linear(A[r0:r0 + 256].contiguous(), W, Ys, epilogue=epi)
        assert torch.equal(Ys, Y[r0:r0 + 256]), f"rows {r0}..{r0 + 255} differ"


@pytest.mark.parametrize("case", ["tiny_f32", "pack256_bf16"])
def test_cond_and_modulation(B, case):
    wl = CF.WORKLOADS[case]
    d = wl.dims
    dims = B.Dims(d, wl.dtype)
    ww = S.wrapper_weights(d, wl.dtype, wl.name)
    bw = S.stream_weights(d, wl.dtype, wl.name, 0, "img")
    t = S.timesteps(len(wl.samples), wl.name)
    c = torch.empty(len(t), d.hidden, dtype=_tdt(wl.dtype), device="cuda")
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    B.cond(dims, _dev(ww["w_t1"], wl.dtype), _dev(ww["w_t2"], wl.dtype), torch.from_numpy(t).cuda(), c, ws)
    want = OB.cond(t, ww["w_t1"], ww["w_t2"])
    tol = TOL[wl.dtype] if wl.dtype == "bf16" else 1e-4
    assert_close(f"c[{case}]", to_np(c), want, tol)
    # modulation from a seeded c (never from a GPU output)
    cs = S.normal((len(t), d.hidden), 1.0, wl.dtype, wl.name, "c_syn")
    mod = torch.empty(len(t), 6 * d.hidden, dtype=torch.float32, device="cuda")
    B.modulation(dims, _dev(bw["w_mod"], wl.dtype), 6, _dev(cs, wl.dtype), mod)
    want_m = np.concatenate(OB.modulation(cs, bw["w_mod"]), axis=1)
    assert_close(f"mod[{case}]", to_np(mod), want_m, tol)
