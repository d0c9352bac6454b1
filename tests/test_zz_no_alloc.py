"""GPU check of rf_loss_noalloc (the loss with its per-row sums in the
library's own device scratch instead of a caller workspace) against rf_loss,
through the C ABI: bit for bit, on two calls in a row (the second on a
smaller pack, so stale sums of the first call lie past the rows it reads),
then once more on the first pack."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _case(B, samples, C, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    pk = B.pack(samples)
    n_img, n_tgt = pk.n_img, pk.n_tgt
    z = torch.randn(n_img, C, device="cuda", generator=g).to(torch.bfloat16)
    eps = torch.randn(n_img, C, device="cuda", generator=g).to(torch.bfloat16)
    v = torch.randn(n_tgt, C, device="cuda", generator=g).to(torch.bfloat16)
    return pk, v, z, eps


def test_rf_loss_noalloc_matches_rf_loss():
    from resolution_image_gen_amd import binding as B

    big = [(64, 64, 1, 256), (48, 84, 2, 256), (84, 48, 1, 0), (32, 128, 1, 256)]
    small = [(5, 7, 2, 3), (16, 16, 1, 128), (1, 1, 1, 0)]
    C = 128
    cases = [_case(B, big, C, 1), _case(B, small, C, 2)]
    cases.append(cases[0])
    for i, (pk, v, z, eps) in enumerate(cases):
        print(f"rf_loss_noalloc call {i}: {pk.B} samples, {pk.n_tgt} target rows", flush=True)
        sse = torch.full((pk.B,), float("nan"), device="cuda")
        loss = torch.full((1,), float("nan"), device="cuda")
        B.rf_loss_noalloc(pk, v, z, eps, sse, loss)
        ref_sse, ref_loss = torch.empty_like(sse), torch.empty_like(loss)
        ws = torch.empty(pk.n_tgt * 4 + 256, dtype=torch.uint8, device="cuda")
        B.rf_loss(pk, v, z, eps, ref_sse, ref_loss, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(sse).all() and torch.isfinite(loss).all()
        assert torch.equal(sse, ref_sse), (i, (sse - ref_sse).abs().max().item())
        assert torch.equal(loss, ref_loss), (i, loss.item(), ref_loss.item())
