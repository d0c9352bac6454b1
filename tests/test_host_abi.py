"""Host-only checks of the C ABI (no GPU): exports, struct layout, the host
planner against the oracle, and argument validation that fails before any
launch."""

import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

from oracle import pack as OP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmdit.h")


@pytest.fixture(scope="module")
def B():
    from resolution_image_gen_amd import binding

    return binding


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:mmdit|rf)_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(B):
    names = declared_functions()
    assert len(names) >= 20, names
    for n in names:
        assert hasattr(B._lib, n), f"{n} declared in mmdit.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", B.lib_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T ((?:mmdit|rf)_\w+)", out))
    assert set(names) <= exported
    assert B._lib.mmdit_version().decode().startswith("mmdit")


LAYOUT_PROBE = r"""
#include <stdio.h>
#include <stddef.h>
#include "mmdit.h"
#define F(T, f) printf(#T "." #f " %zu\n", offsetof(T, f));
int main(void) {
  printf("mmdit_pack_t %zu\nmmdit_dims %zu\nmmdit_sample %zu\nmmdit_block_w %zu\n", sizeof(mmdit_pack_t),
         sizeof(mmdit_dims), sizeof(mmdit_sample), sizeof(mmdit_block_w));
  F(mmdit_pack_t, n_img) F(mmdit_pack_t, cu_txt) F(mmdit_pack_t, tgt_row) F(mmdit_pack_t, h_cu_txt)
  F(mmdit_pack_t, h_cu_img) F(mmdit_pack_t, h_cu_tgt) F(mmdit_pack_t, h_frames)
  F(mmdit_dims, rope_dims) F(mmdit_dims, rope_theta) F(mmdit_dims, dtype) F(mmdit_block_w, txt)
  return 0;
}
"""


def test_struct_layout_matches_binding(B):
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "probe.c"), os.path.join(d, "probe")
        open(src, "w").write(LAYOUT_PROBE)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    c = dict(line.rsplit(" ", 1) for line in out.strip().splitlines())
    c = {k: int(v) for k, v in c.items()}
    assert c["mmdit_pack_t"] == ctypes.sizeof(B._PackT)
    assert c["mmdit_dims"] == ctypes.sizeof(B._DimsT)
    assert c["mmdit_sample"] == ctypes.sizeof(B._Sample)
    assert c["mmdit_block_w"] == ctypes.sizeof(B._BlockW)
    for f in ("n_img", "cu_txt", "tgt_row", "h_cu_txt", "h_cu_img", "h_cu_tgt", "h_frames"):
        assert c[f"mmdit_pack_t.{f}"] == getattr(B._PackT, f).offset, f
    assert c["mmdit_dims.rope_dims"] == B._DimsT.rope_dims.offset
    assert c["mmdit_dims.rope_theta"] == B._DimsT.rope_theta.offset
    assert c["mmdit_dims.dtype"] == B._DimsT.dtype.offset
    assert c["mmdit_block_w.txt"] == B._BlockW.txt.offset


def test_host_plan_matches_oracle_random(B):
    rng = np.random.default_rng(0)
    for _ in range(300):
        n = int(rng.integers(0, 12))
        s = [(int(rng.integers(1, 40)), int(rng.integers(1, 40)), int(rng.integers(1, 3)), int(rng.integers(0, 300)))
             for _ in range(n)]
        budget = int(rng.integers(1, 6000))
        joint = int(rng.choice([0, int(rng.integers(1, 8000))]))
        try:
            want = OP.plan(s, budget, joint)
        except OP.BudgetError:
            with pytest.raises(B.MmditError) as e:
                B.pack_plan(s, budget, joint)
            assert e.value.status == -2
            continue
        assert B.pack_plan(s, budget, joint) == want, (s, budget, joint)


def test_plan_caps_at_max_samples(B):
    assert B.pack_plan([(1, 1, 1, 0)] * 300, 10 ** 6)[0] == B.MAX_SAMPLES


def _fake_pack(B, samples):
    """A host-consistent pack struct with placeholder device pointers, for
    validation paths that return before any launch."""
    pk = B._PackT()
    ref = OP.pack(samples)
    pk.B = len(samples)
    pk.max_joint = ref["max_joint"]
    pk.n_img, pk.n_txt, pk.n_tgt = int(ref["cu_img"][-1]), int(ref["cu_txt"][-1]), int(ref["cu_tgt"][-1])
    for i in range(pk.B + 1):
        pk.h_cu_img[i], pk.h_cu_txt[i], pk.h_cu_tgt[i] = (int(ref["cu_img"][i]), int(ref["cu_txt"][i]),
                                                         int(ref["cu_tgt"][i]))
    fake = 1 << 20
    for f in ("cu_txt", "cu_img", "cu_joint", "cu_tgt", "tgt_len", "seg_img", "seg_txt", "pos_img", "tgt_row"):
        setattr(pk, f, fake)
    return pk


def _dims(B, **kw):
    from resolution_image_gen_amd import configs as CF

    d = dict(CF.B4.__dict__)
    d.update(kw)
    D = d["head_dim"]
    rope = d.get("rope", (D // 4, 3 * D // 8, 3 * D // 8))
    return B._DimsT(d["hidden"], d["heads"], d["head_dim"], d["mlp"], d["c_lat"], d["d_txt"], d["t_dim"],
                    (ctypes.c_int32 * 3)(*rope), d["rope_theta"], d["eps"], 1)


def test_validation_errors_before_launch(B):
    lib = B._lib
    pk = _fake_pack(B, [(16, 16, 1, 128), (8, 8, 2, 3)])
    P = ctypes.byref(pk)
    ok = ctypes.byref(_dims(B))
    fake = ctypes.c_void_p(1 << 20)
    w = B._BlockW(B._StreamW(*([1 << 20] * 7)), B._StreamW(*([1 << 20] * 7)))
    # head_dim outside {64, 128}
    assert lib.mmdit_block_fwd(ctypes.byref(_dims(B, heads=32, head_dim=96)), ctypes.byref(w), P, fake, fake,
                               fake, fake, 1 << 40, None) == -3
    # hidden != heads * head_dim
    assert lib.mmdit_block_fwd(ctypes.byref(_dims(B, heads=20)), ctypes.byref(w), P, fake, fake, fake, fake,
                               1 << 40, None) == -1
    # workspace too small
    need = lib.mmdit_workspace_size(ok, P)
    assert need > 0
    assert lib.mmdit_block_fwd(ok, ctypes.byref(w), P, fake, fake, fake, fake, need - 1, None) == -4
    assert b"workspace" in lib.mmdit_last_error()
    # NULL weight
    w2 = B._BlockW(B._StreamW(*([1 << 20] * 7)), B._StreamW(*([1 << 20] * 6 + [0])))
    assert lib.mmdit_block_fwd(ok, ctypes.byref(w2), P, fake, fake, fake, fake, need, None) == -1
    # misaligned pointer
    assert lib.mmdit_block_fwd(ok, ctypes.byref(w), P, ctypes.c_void_p((1 << 20) + 2), fake, fake, fake, need,
                               None) == -3
    # pack whose host mirror is inconsistent
    bad = _fake_pack(B, [(4, 4, 1, 1)])
    bad.n_img = 99
    assert lib.mmdit_block_fwd(ok, ctypes.byref(w), ctypes.byref(bad), fake, fake, fake, fake, need, None) == -1
    # rf wrapper
    assert lib.rf_euler_step(P, 1, 128, fake, 0, 5, ctypes.c_float(4.0), ctypes.c_float(1.0),
                             ctypes.c_float(0.75), fake, None, None) == -1
    assert lib.rf_euler_step(P, 1, 128, fake, 0, 1, ctypes.c_float(4.0), ctypes.c_float(1.0),
                             ctypes.c_float(0.75), fake, None, None) == -1    # different target sizes
    assert lib.rf_loss(P, 1, 128, fake, fake, fake, fake, fake, fake, 16, None) == -4
    # the documented minimum, n_tgt * 4 + 4 bytes, minus one
    n_tgt = 16 * 16 + 8 * 8
    assert lib.rf_loss(P, 1, 128, fake, fake, fake, fake, fake, fake, n_tgt * 4 + 3, None) == -4
    assert lib.rf_loss(P, 1, 128, fake, fake, fake, fake, fake, ctypes.c_void_p((1 << 20) + 4), 1 << 20, None) == -3
    assert lib.rf_make_xt(P, 1, 12, fake, fake, fake, fake, None) == -3        # C % 8
    # the workspace-free loss keeps its per-row sums in a fixed scratch of 2^22 rows
    big = ctypes.byref(_fake_pack(B, [(2048, 2048, 1, 0), (1, 1, 1, 0)]))
    assert lib.rf_loss_noalloc(big, 1, 128, fake, fake, fake, fake, fake, None) == -3
    assert b"scratch" in lib.mmdit_last_error()
    # linear shape errors
    assert lib.mmdit_linear(1, -1, 64, 64, fake, fake, fake, 0, None, 0, None, 0, None) == -1
    assert lib.mmdit_linear(1, 64, 64, 64, fake, fake, fake, 3, None, 0, None, 0, None) == -1
    # gate rows are read as 16-byte vectors: the stride must be a multiple of 4 floats
    assert lib.mmdit_linear(1, 64, 64, 64, fake, fake, fake, 3, fake, 66, fake, 0, None) == -3
    assert b"gate_stride" in lib.mmdit_last_error()
    assert lib.mmdit_linear(1, 64, 64, 64, fake, fake, fake, 3, fake, 60, fake, 0, None) == -1
    # K at 2^22: the 32-bit tile offsets cannot address it
    assert lib.mmdit_linear(1, 64, 64, 1 << 22, fake, fake, fake, 0, None, 0, None, 0, None) == -3
    assert b"2^22" in lib.mmdit_last_error()
    # pack: too many samples
    arr = (B._Sample * 300)(*[B._Sample(1, 1, 1, 0)] * 300)
    assert lib.mmdit_pack(arr, 300, ctypes.byref(B._PackT()), None) == -1
    assert lib.mmdit_workspace_size(ctypes.byref(_dims(B, head_dim=96, heads=32)), P) == 0
    # RoPE bands: even widths summing to head_dim, anything else is rejected
    for rope in ((32, 48, 50), (33, 47, 48), (-2, 66, 64), (32, 48, 46)):
        bad = _dims(B, rope=rope)
        assert lib.mmdit_qk_norm_rope(ctypes.byref(bad), 4, fake, fake, fake, fake, None) == -3, rope
        assert b"rope_dims" in lib.mmdit_last_error()
        assert lib.mmdit_block_fwd(ctypes.byref(bad), ctypes.byref(w), P, fake, fake, fake, fake, need, None) == -3
        assert lib.mmdit_workspace_size(ctypes.byref(bad), P) == 0
    for rope in ((0, 64, 64), (128, 0, 0), (64, 32, 32)):   # other even splits are computed
        assert lib.mmdit_workspace_size(ctypes.byref(_dims(B, rope=rope)), P) > 0


def test_training_calls_validate_before_launch(B):
    lib = B._lib
    pk = _fake_pack(B, [(16, 16, 1, 128), (8, 8, 2, 3)])
    P = ctypes.byref(pk)
    ok = ctypes.byref(_dims(B))
    fake = ctypes.c_void_p(1 << 20)
    w = B._BlockW(B._StreamW(*([1 << 20] * 7)), B._StreamW(*([1 << 20] * 7)))
    g = B._BlockG(B._StreamG(*([1 << 20] * 7)), B._StreamG(*([1 << 20] * 7)))
    need_ws = lib.mmdit_workspace_size(ok, P)
    saved = lib.mmdit_block_saved_size(ok, P)
    bws = lib.mmdit_block_bwd_workspace_size(ok, P)
    assert saved > 0 and bws > 0 and lib.mmdit_wrap_bwd_workspace_size(ok, P) > 0
    assert lib.mmdit_cond_bwd_workspace_size(ok, 2) > 0
    # per row: block input, both modulated norms, q/k/v after their norm and q/k before it, o, both branch
    # outputs, the residual after attention and the MLP pre-activation (mlp = 4H): 16 H bf16 values
    assert saved >= (pk.n_img + pk.n_txt) * 16 * 3072 * 2
    # saved buffer and backward workspace one byte short
    assert lib.mmdit_block_fwd_train(ok, ctypes.byref(w), P, fake, fake, fake, fake, saved - 1, fake, need_ws,
                                     None) == -4
    assert b"saved" in lib.mmdit_last_error()
    assert lib.mmdit_block_bwd(ok, ctypes.byref(w), P, fake, fake, saved, fake, fake, ctypes.byref(g), fake, fake,
                               bws - 1, None) == -4
    # a NULL gradient pointer, a NULL gradient struct, a misaligned dc
    g2 = B._BlockG(B._StreamG(*([1 << 20] * 7)), B._StreamG(*([1 << 20] * 6 + [0])))
    assert lib.mmdit_block_bwd(ok, ctypes.byref(w), P, fake, fake, saved, fake, fake, ctypes.byref(g2), fake, fake,
                               bws, None) == -1
    assert lib.mmdit_block_bwd(ok, ctypes.byref(w), P, fake, fake, saved, fake, fake, None, fake, fake, bws,
                               None) == -1
    assert lib.mmdit_block_bwd(ok, ctypes.byref(w), P, fake, fake, saved, fake, fake, ctypes.byref(g),
                               ctypes.c_void_p((1 << 20) + 4), fake, bws, None) == -3
    # wrapper backward: workspace, NULL weight gradient, sample count
    wr = lib.mmdit_wrap_bwd_workspace_size(ok, P)
    assert lib.mmdit_final_bwd(ok, fake, fake, P, fake, fake, fake, fake, fake, fake, fake, fake, wr - 1, None) == -4
    assert lib.mmdit_embed_bwd(ok, P, fake, fake, fake, fake, None, fake, fake, wr, None) == -1
    assert lib.mmdit_cond_bwd(ok, fake, fake, fake, 300, fake, fake, fake, fake, 1 << 30, None) == -1
    assert lib.rf_loss_grad(P, 1, 12, fake, fake, fake, fake, None) == -3     # C % 8


def test_gradient_struct_layout(B):
    assert ctypes.sizeof(B._BlockG) == 14 * ctypes.sizeof(ctypes.c_void_p)
    assert B._BlockG.txt.offset == 7 * ctypes.sizeof(ctypes.c_void_p)
    assert [f for f, _ in B._StreamG._fields_] == ["w_mod", "w_qkv", "g_q", "g_k", "w_o", "w_up", "w_down"]


def test_split_modulation_and_two_stream_calls_validate_before_launch(B):
    lib = B._lib
    pk = _fake_pack(B, [(16, 16, 1, 128), (8, 8, 2, 3)])
    P = ctypes.byref(pk)
    ok = ctypes.byref(_dims(B))
    fake = ctypes.c_void_p(1 << 20)
    w = B._BlockW(B._StreamW(*([1 << 20] * 7)), B._StreamW(*([1 << 20] * 7)))
    g = B._BlockG(B._StreamG(*([1 << 20] * 7)), B._StreamG(*([1 << 20] * 7)))
    need_ws = lib.mmdit_workspace_size(ok, P)
    # block_modulation: B outside [0, 256], NULL and misaligned outputs, a NULL weight
    assert lib.mmdit_block_modulation(ok, ctypes.byref(w), 257, fake, fake, None) == -1
    assert lib.mmdit_block_modulation(ok, ctypes.byref(w), -1, fake, fake, None) == -1
    assert lib.mmdit_block_modulation(ok, ctypes.byref(w), 2, fake, None, None) == -1
    assert lib.mmdit_block_modulation(ok, ctypes.byref(w), 2, fake, ctypes.c_void_p((1 << 20) + 4), None) == -3
    w0 = B._BlockW(B._StreamW(*([0] + [1 << 20] * 6)), B._StreamW(*([1 << 20] * 7)))
    assert lib.mmdit_block_modulation(ok, ctypes.byref(w0), 2, fake, fake, None) == -1
    assert lib.mmdit_block_modulation(ok, ctypes.byref(w), 0, None, None, None) == 0    # nothing to do
    # block_fwd_mod: a NULL modulation, a workspace one byte short
    assert lib.mmdit_block_fwd_mod(ok, ctypes.byref(w), P, None, fake, fake, fake, need_ws, None) == -1
    assert lib.mmdit_block_fwd_mod(ok, ctypes.byref(w), P, fake, fake, fake, fake, need_ws - 1, None) == -4
    # final_mod: NULL modulation, NULL output
    assert lib.mmdit_final_mod(ok, fake, P, None, fake, fake, fake, 1 << 30, None) == -1
    assert lib.mmdit_final_mod(ok, fake, P, fake, fake, None, fake, 1 << 30, None) == -1
    # block_bwd2 validates exactly like block_bwd
    saved = lib.mmdit_block_saved_size(ok, P)
    bws = lib.mmdit_block_bwd_workspace_size(ok, P)
    assert lib.mmdit_block_bwd2(ok, ctypes.byref(w), P, fake, fake, saved, fake, fake, ctypes.byref(g), fake, fake,
                                bws - 1, None, fake) == -4
    assert b"mmdit_block_bwd2" in lib.mmdit_last_error()
    assert lib.mmdit_block_bwd2(ok, ctypes.byref(w), P, fake, fake, saved - 1, fake, fake, ctypes.byref(g), fake,
                                fake, bws, None, fake) == -4
