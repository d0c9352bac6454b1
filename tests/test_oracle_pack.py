"""Pins for the oracle packer: hand-written fixtures and closed forms."""

import json
import os

import numpy as np
import pytest

from oracle import pack as P

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_pack_matches_hand_written_fixture():
    g = _load("pack_small.json")
    pk = P.pack(g["samples"])
    for key in ("cu_txt", "cu_img", "cu_joint", "cu_tgt", "tgt_len", "seg_txt", "seg_img",
                "pos_img", "tgt_rows"):
        np.testing.assert_array_equal(pk[key], np.asarray(g[key]), err_msg=key)
    assert pk["max_joint"] == g["max_joint"]


def test_plan_budget_arithmetic_fixture():
    g = _load("plan_native1024.json")
    got = P.plan(g["samples"], g["img_budget"])
    assert got == tuple(g["image_only"][k] for k in ("n_taken", "n_img", "n_txt", "max_joint"))
    got = P.plan(g["samples"], g["img_budget"], joint_budget=16384)
    assert got == tuple(g["joint_16384"][k] for k in ("n_taken", "n_img", "n_txt", "max_joint"))


def test_plan_oversize_first_sample_is_an_error():
    with pytest.raises(P.BudgetError):
        P.plan([(128, 128, 2, 0)], img_budget=16384)
    with pytest.raises(P.BudgetError):
        P.plan([(8, 8, 1, 100)], img_budget=64, joint_budget=100)


def test_plan_next_fit_stops_at_first_misfit():
    # 64 + 64 fit a 150 budget, the third (64) does not; the fourth (4) would,
    # but next-fit closes the pack at the first sample that does not fit.
    s = [(8, 8, 1, 1), (8, 8, 1, 1), (8, 8, 1, 1), (2, 2, 1, 1)]
    assert P.plan(s, 150)[0] == 2
    assert P.plan([], 10) == (0, 0, 0, 0)


@pytest.mark.parametrize("bad", [(0, 4, 1, 0), (4, 0, 1, 0), (4, 4, 3, 0), (4, 4, 1, -1)])
def test_invalid_sample(bad):
    with pytest.raises(ValueError):
        P.pack([bad])


@pytest.mark.parametrize("samples", [
    [(16, 16, 1, 32), (8, 8, 1, 32)],
    [(3, 5, 2, 7), (1, 1, 1, 0), (4, 2, 2, 3)],
    [(64, 64, 1, 256), (48, 84, 1, 256), (84, 48, 1, 256), (32, 128, 1, 256)],
])
def test_pack_closed_forms(samples):
    pk = P.pack(samples)
    B = len(samples)
    assert pk["cu_img"][B] == sum(f * h * w for h, w, f, _ in samples)
    assert pk["cu_txt"][B] == sum(t for *_, t in samples)
    assert pk["cu_tgt"][B] == sum(h * w for h, w, _, _ in samples)
    np.testing.assert_array_equal(pk["cu_joint"], pk["cu_txt"] + pk["cu_img"])
    for b, (h, w, f, t) in enumerate(samples):
        i0 = pk["cu_img"][b]
        rows = np.arange(f * h * w)
        # image row i0 + k*h*w + r*w + c carries (k, r, c)
        np.testing.assert_array_equal(pk["pos_img"][i0 + rows],
                                      np.stack([rows // (h * w), (rows % (h * w)) // w, rows % w], 1))
        assert np.all(pk["seg_img"][i0:i0 + f * h * w] == b)
        assert np.all(pk["seg_txt"][pk["cu_txt"][b]:pk["cu_txt"][b + 1]] == b)
        np.testing.assert_array_equal(pk["tgt_rows"][pk["cu_tgt"][b]:pk["cu_tgt"][b + 1]],
                                      i0 + np.arange(h * w))
