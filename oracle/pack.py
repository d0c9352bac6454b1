"""Oracle: native-resolution packing (test infrastructure only).

What the pages fix (hyper.ai 2607.19064, 方法; blog close-reading, 2.2(2)
and 5 "Native-resolution packing"): latent grids of different sizes are
flattened into variable-length token sequences and packed into one batch under
a fixed token budget; text is packed by the same principle; samples are
separated by cumulative offsets and attention stays inside each sample; every
sample keeps its own 2D RoPE positions; editing adds a frame index f to (h, w)
to tell source from target tokens.

Readings (the pages are silent on these):
  R1  the budget counts image-latent tokens; an optional second budget
      counts image + text tokens (0 disables it).
  R2  next-fit in input order; a sample that alone exceeds a budget is an
      error, never truncated.
  R3  canonical joint order inside a sample is [text, target image, source
      image]; storage is modality-major (one image buffer, one text buffer).
  R4  grids are flattened row-major: token r*w + c.
  R5  text tokens carry position (0, 0, 0).
  R6  target image tokens carry frame 0, source image tokens frame 1.

A sample is a tuple (h, w, frames, txt_len) in latent-grid units.
"""

import numpy as np


class BudgetError(ValueError):
    """A single sample does not fit the budget on its own (R2)."""


def _check_sample(s):
    h, w, frames, txt_len = (int(v) for v in s)
    if h < 1 or w < 1 or frames not in (1, 2) or txt_len < 0:
        raise ValueError(f"invalid sample {s!r}")
    return h, w, frames, txt_len


def plan(samples, img_budget, joint_budget=0):
    """Next-fit plan (R1, R2): how many leading samples go into one pack.

    Returns (n_taken, n_img, n_txt, max_joint).  Raises BudgetError if the
    first sample alone exceeds a budget.
    """
    n_img = n_txt = 0
    max_joint = 0
    taken = 0
    for s in samples:
        h, w, frames, txt_len = _check_sample(s)
        img = frames * h * w
        joint = img + txt_len
        if img > img_budget or (joint_budget > 0 and joint > joint_budget):
            if taken == 0:
                raise BudgetError(f"sample {s!r} exceeds the budget alone")
            break
        if n_img + img > img_budget:
            break
        if joint_budget > 0 and n_img + n_txt + joint > joint_budget:
            break
        n_img += img
        n_txt += txt_len
        max_joint = max(max_joint, joint)
        taken += 1
    return taken, n_img, n_txt, max_joint


def pack(samples):
    """Offsets, segment ids and 3-axis position ids of one pack.

    Written as explicit loops over samples, slots and grid cells so each id
    can be read off the definition.  Returns a dict of int64 numpy arrays:
      cu_txt, cu_img, cu_joint, cu_tgt : [B+1] cumulative offsets
      tgt_len                          : [B]   target image tokens per sample
      seg_img [n_img], seg_txt [n_txt] : sample index of every row
      pos_img [n_img, 3]               : (frame, row, col) of every image row
      tgt_rows [n_tgt]                 : image-row index of every target row
    """
    samples = [_check_sample(s) for s in samples]
    B = len(samples)
    cu_txt = np.zeros(B + 1, np.int64)
    cu_img = np.zeros(B + 1, np.int64)
    cu_tgt = np.zeros(B + 1, np.int64)
    tgt_len = np.zeros(B, np.int64)
    seg_img, seg_txt, pos_img, tgt_rows = [], [], [], []
    for b, (h, w, frames, txt_len) in enumerate(samples):
        cu_txt[b + 1] = cu_txt[b] + txt_len
        cu_img[b + 1] = cu_img[b] + frames * h * w
        tgt_len[b] = h * w
        cu_tgt[b + 1] = cu_tgt[b] + h * w
        for _ in range(txt_len):
            seg_txt.append(b)
        for k in range(frames):          # slot 0 = target, slot 1 = source (R3, R6)
            for r in range(h):           # row-major raster (R4)
                for c in range(w):
                    seg_img.append(b)
                    pos_img.append((k, r, c))
                    if k == 0:
                        tgt_rows.append(len(seg_img) - 1)
    return {
        "B": B,
        "cu_txt": cu_txt,
        "cu_img": cu_img,
        "cu_joint": cu_txt + cu_img,
        "cu_tgt": cu_tgt,
        "tgt_len": tgt_len,
        "seg_img": np.asarray(seg_img, np.int64),
        "seg_txt": np.asarray(seg_txt, np.int64),
        "pos_img": np.asarray(pos_img, np.int64).reshape(-1, 3),
        "tgt_rows": np.asarray(tgt_rows, np.int64),
        "max_joint": int(max((f * h * w + t for h, w, f, t in samples), default=0)),
    }
