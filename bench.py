#!/usr/bin/env python3
"""Benchmark of the packed NR-MMDiT hot path on one MI355X.

Headline (the default line): the 4-step packed-CFG Euler sampler at 1024^2.
One step of the benchmark = one whole 4-step pack: cond + uncond samples
(64x64 latent grid + 256 text tokens each, 8,704 tokens), 28 random-init
dual-stream blocks (hidden 3072, 24 x 128 heads, MLP 12288, bf16), guidance
4, t = 1, .75, .5, .25 -> 0; per Euler step the conditioning, every block's
adaLN vectors, the embeddings, 28 blocks, the final layer, then the CFG
combine + Euler update.  A pack is captured once as a HIP graph and
replayed; K replays are bracketed by hipEvents on the launch stream.
`value` = block-token throughput (8,704 tokens x 28 blocks x 4 steps per
pack / seconds per pack); `ms_per_step` = ms per 4-step pack.  One more pack
runs eagerly on one stream with every library launch bracketed by hipEvents
on its stream: it gives the per-kernel table and the roofline of the
dominant kernel.  The CPU oracle runs one block-step of the same pack.

Extra keys: the 256^2-stage training forward (16 x (16x16 grid + 128 text)
tokens, one block + RF loss) as `train_forward_256`, the same for the 1024^2
native-resolution pack, the 2048^2 edit pair and the tiny float32 pack
(`native1024_bf16`, `edit2048_bf16`, `tiny_f32`), the rectified-flow
kernels' bandwidth as `rf_kernels`, the RMSNorm + modulate chain against a
plain copy of its bytes as `chains_vs_copy`; optional legs behind flags (two-pass
CFG, 20-step and editing samplers, the 50k-token training step).

Prints ONE JSON line.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed MMDiT block tokens/s + TFLOP/s (% bf16 peak); ms per 4-step 1024² pack"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def kernel_work(wl, samples=None, depth=None):
    """Algorithmic work per launch of each tagged kernel of one step over
    `samples` (default: the workload's) with `depth` blocks."""
    d = wl.dims
    H, M = d.hidden, d.mlp
    samples = wl.samples if samples is None else samples
    depth = wl.depth if depth is None else depth
    n = sum(f * h * w + t for h, w, f, t in samples)
    n_tgt = sum(h * w for h, w, _, _ in samples)
    att = sum((f * h * w + t) ** 2 for h, w, f, t in samples)
    es = 2 if wl.dtype == "bf16" else 4
    return {
        "qkv_proj": ("mfma", 2.0 * n * H * 3 * H),
        "out_proj_gated": ("mfma", 2.0 * n * H * H),
        "mlp_up_gelu": ("mfma", 2.0 * n * H * M),
        "mlp_down_gated": ("mfma", 2.0 * n * M * H),
        "attn_mfma_kernel": ("mfma", 4.0 * H * att),
        # read x, write y: per block two launches over all N rows, and one
        # launch over the target rows per forward (final layer), averaged
        "rms_modulate_kernel": ("hbm", (2 * depth * (2.0 * es * H * n) + 2.0 * es * H * n_tgt) / (2 * depth + 1)),
        # read and write q and k of every row, one launch
        "qk_norm_rope_kernel": ("hbm", 4.0 * es * H * n),
        "final_out": ("mfma", 2.0 * n_tgt * H * d.c_lat),
    }


def train_kernel_work(wl):
    """Work per launch of the kernels of a training step's backward (GEMMs:
    2 M N K; attention backward kernels: the score-sized products each one
    runs, 2 d sum L_b^2 per head each: dQ 3 (S^T, dP^T, dQ), dK 3 (S, dP,
    dK), dV 2 (S, dV))."""
    d = wl.dims
    H, M = d.hidden, d.mlp
    n = sum(f * h * w + t for h, w, f, t in wl.samples)
    unit = 2.0 * H * sum((f * h * w + t) ** 2 for h, w, f, t in wl.samples)
    work = kernel_work(wl)
    work.update({
        "bwd_mlp_down_dx": ("mfma", 2.0 * n * H * M), "bwd_mlp_down_dw": ("mfma", 2.0 * n * H * M),
        "bwd_mlp_up_dx": ("mfma", 2.0 * n * H * M), "bwd_mlp_up_dw": ("mfma", 2.0 * n * H * M),
        "bwd_qkv_dx": ("mfma", 6.0 * n * H * H), "bwd_qkv_dw": ("mfma", 6.0 * n * H * H),
        "bwd_out_proj_dx": ("mfma", 2.0 * n * H * H), "bwd_out_proj_dw": ("mfma", 2.0 * n * H * H),
        "attn_bwd_dq_kernel": ("mfma", 3 * unit), "attn_bwd_dk_kernel": ("mfma", 3 * unit),
        "attn_bwd_dv_kernel": ("mfma", 2 * unit),
    })
    return work


# HBM bytes per launch of a kernel, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# scaled by a plain copy's counter reading (profiles/traffic.json); valid only
# while the kernel's sources are unchanged since the counters were taken.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_sources_sha256(sources):
    """SHA-256 over the given source files (repository-relative), in order."""
    import hashlib

    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(tag, workload):
    """HBM bytes per launch of kernel `tag` on `workload` from the committed
    counter record, or None when there is none or the record's kernel sources
    changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            recs = json.load(f)
    except (OSError, ValueError):
        return None
    for rec in recs if isinstance(recs, list) else [recs]:
        if rec.get("kernel") == tag and rec.get("workload") == workload:
            try:
                if rec.get("sources_sha256") != kernel_sources_sha256(rec.get("sources", ())):
                    return None
            except OSError:
                return None
            return rec.get("hbm_bytes_per_launch")
    return None


def step_flops(wl):
    from resolution_image_gen_amd.configs import block_flops

    d = wl.dims
    H = d.hidden
    B = len(wl.samples)
    n_img = sum(f * h * w for h, w, f, _ in wl.samples)
    n_txt = sum(t for *_, t in wl.samples)
    n_tgt = sum(h * w for h, w, _, _ in wl.samples)
    blk = block_flops(d, wl.samples)[0] * wl.depth
    wrap = 2.0 * (n_img * d.c_lat * H + n_txt * d.d_txt * H + n_tgt * H * d.c_lat
                  + B * (d.t_dim * H + H * H + 12 * H * H * wl.depth + 2 * H * H))
    return blk, wrap


class _NumpyWeights:
    """Host copies of the weights for the CPU oracle (the device copies can be freed)."""

    def __init__(self, W):
        self.np_wrap = W.np_wrap
        self.np_blocks = W.np_blocks


def cpu_baseline(wl, W, inputs, n_samples, min_seconds=10.0):
    """The oracle (float64 numpy) on the first n_samples samples of the pack,
    repeated until at least min_seconds of CPU work have been timed."""
    import numpy as np

    from oracle import flow as OF
    from oracle import pack as OP

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    samples = list(wl.samples[:n_samples])
    ref = OP.pack(samples)
    ni, nt = ref["cu_img"][-1], ref["cu_txt"][-1]
    Wd = {k: np.asarray(v, np.float64) for k, v in W.np_wrap.items()}
    Wd["blocks"] = [{s: {k: np.asarray(v, np.float64) for k, v in nb[s].items()} for s in nb}
                    for nb in W.np_blocks]
    z, eps, tau, t = inputs["z"][:ni], inputs["eps"][:ni], inputs["tau"][:nt], inputs["t"][:n_samples]
    runs, dt = 0, 0.0
    while runs == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        zt = OF.make_xt(z, eps, t, ref)
        v = OF.velocity_model(zt, tau, t, Wd, ref, wl.dims.heads)
        OF.loss(v, z, eps, ref)
        dt += time.perf_counter() - t0
        runs += 1
    tokens = (ni + nt) * runs
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_samples} of {len(wl.samples)} samples ({ni + nt} tokens) of the same step "
                      f"(noise, cond, embed, block, final, loss), float64 numpy, {runs} runs, {dt:.1f} s"}


# Further launches that finish a tagged kernel's work (the MLP down
# projection's split last round: the k parts of its remaining tiles, then the
# fixup that sums them and applies the epilogue); their time counts toward
# the tagged kernel's launches.
FIXUP_OF = {"mlp_down_gated": ("mlp_down_sk", "mlp_down_fixup")}


def _total_ms(kernels, tag):
    ms, cnt = kernels[tag]
    for fx in FIXUP_OF.get(tag, ()):
        if fx in kernels:
            ms += kernels[fx][0]
    return ms, cnt


def _roofline(kernels, work):
    """Roofline object of the dominant kernel: the tagged kernel with the
    largest total time (its fixup launches included) among those with a
    known algorithmic work; achieved = work per launch / average launch time."""
    dom = max((k for k in kernels if k in work), key=lambda k: _total_ms(kernels, k)[0])
    kind, per_launch = work[dom]
    tot, cnt = _total_ms(kernels, dom)
    avg_ms = tot / cnt
    if kind == "mfma":
        achieved = per_launch / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = per_launch / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    roof["traffic"] = None
    roof["kernel"] = dom
    roof["avg_launch_us"] = round(avg_ms * 1e3, 2)
    roof["work_per_launch"] = per_launch
    return roof


def _kernel_lines(kernels, work, per, unit):
    """Per-kernel table (total time per `unit`, launches, and the rate of
    kernels with a known work), largest first."""
    out = {}
    for k, (ms, cnt) in sorted(kernels.items(), key=lambda kv: -kv[1][0]):
        row = {f"us_per_{unit}": round(ms / per * 1e3, 1), "launches": round(cnt / per, 2)}
        if k in work:
            kd, wk = work[k]
            s = _total_ms(kernels, k)[0] / cnt * 1e-3
            row["TFLOP/s" if kd == "mfma" else "GB/s"] = round(wk / s / (1e12 if kd == "mfma" else 1e9), 1)
        out[k] = row
    return out


def sampler_inputs(wl):
    """z_1 = eps (64x64 x C) and the two text conditions of the sampler pack."""
    from resolution_image_gen_amd import synthetic as S

    d = wl.dims
    h, w, _, T = wl.samples[0]
    eps = S.normal((h * w, d.c_lat), 1.0, "bf16", wl.name, "eps")
    tau_c = S.text(T, d.d_txt, "bf16", wl.name, "tau_c")
    tau_u = S.text(T, d.d_txt, "bf16", wl.name, "tau_u")
    return eps, tau_c, tau_u


def _timed_graph(sm, steps, warmup):
    """ms per replay of the sampler's pack captured as one HIP graph."""
    import torch

    sm.capture()                          # one pack = one HIP graph (~1,600 launches at 4 steps)
    for _ in range(warmup):
        sm.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        sm.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del sm.graph
    return e0.elapsed_time(e1) / steps, wall


def bench_headline(steps, warmup):
    """The 4-step packed-CFG sampler at 1024^2 over 28 blocks: ms per pack
    from `steps` graph replays, then one eager pack on one stream with every
    launch timed (per-kernel table, roofline of the dominant kernel)."""
    import torch

    from resolution_image_gen_amd import binding as B
    from resolution_image_gen_amd import configs as CF
    from resolution_image_gen_amd import runner as R
    from resolution_image_gen_amd.configs import block_flops

    wl = CF.WORKLOADS["sampler1024_cfg_bf16"]
    W = R.Weights(wl, source="torch")            # 28 blocks drawn on the GPU (19 GB bf16)
    eps, tau_c, tau_u = sampler_inputs(wl)
    sm = R.Sampler(wl, W, eps, tau_c, tau_u)
    ms, wall = _timed_graph(sm, steps, warmup)
    assert torch.isfinite(sm.z).all()
    z_graph = sm.z.clone()
    # one eager pack, every launch on one stream, bracketed by hipEvents
    sm.overlap = False
    torch.cuda.synchronize()
    B.timing_enable(True)
    sm.run()
    kernels = B.timing_report()
    B.timing_enable(False)
    sm.overlap = R.OVERLAP
    assert torch.equal(sm.z, z_graph), "eager and graph-replayed packs disagree"
    nsteps = len(wl.schedule) - 1
    blk = block_flops(wl.dims, sm.samples)[0] * wl.depth * nsteps
    _, wrap1 = step_flops(wl)
    n = sum(hh * ww * f + t for hh, ww, f, t in sm.samples)
    work = kernel_work(wl, sm.samples, wl.depth)
    roof = _roofline(kernels, work)
    roof["traffic"] = measured_traffic(roof["kernel"], wl.name)
    return {
        "wl": wl, "W": W, "inputs": (eps, tau_c, tau_u), "samples": sm.samples,
        "ms_per_pack": ms, "wall_s_timed": wall, "block_flop_per_pack": blk, "wrap_flop_per_pack": wrap1 * nsteps,
        "block_tokens_per_pack": n * wl.depth * nsteps, "tokens_per_pack": n,
        "roofline": roof, "kernels": _kernel_lines(kernels, work, 1, "pack"),
    }


def bench_sampler_extras(W, steps, warmup):
    """Beside the headline pack, on the same 28 blocks: the same sampler with
    its two CFG branches as separate forwards (both must end on the same
    bits), one 20-step pack (uniform steps from 1 to 0), and the 4-step
    editing sampler (target + clean source of the same grid per sample),
    packed and two-pass."""
    import torch

    from resolution_image_gen_amd import configs as CF
    from resolution_image_gen_amd import runner as R
    from resolution_image_gen_amd import synthetic as S
    from resolution_image_gen_amd.configs import block_flops

    wl = CF.WORKLOADS["sampler1024_cfg_bf16"]
    d = wl.dims
    eps, tau_c, tau_u = sampler_inputs(wl)
    h, w, _, _ = wl.samples[0]
    sm = R.Sampler(wl, W, eps, tau_c, tau_u)
    ms, _ = _timed_graph(sm, steps, warmup)
    sm2 = R.Sampler(wl, W, eps, tau_c, tau_u, two_pass=True)
    ms2, _ = _timed_graph(sm2, steps, warmup)
    assert torch.isfinite(sm.z).all()
    # the packed pack's GEMMs split their last rounds differently from the
    # one-sample forwards' (MLP down's k-parts, the sub-tiles), so the two
    # agree to rounding, not bit for bit: held to the bound the sampler's
    # parity test uses against the oracle, (|1 - g| + g) x 2e-2 (the CFG
    # combine amplifies a branch's error by up to |1 - g| + g)
    g = wl.guidance
    bound = (abs(1.0 - g) + g) * 2e-2
    diff = ((sm.z - sm2.z).abs().max() / sm2.z.abs().max()).item()
    assert diff <= bound, f"packed and two-pass CFG samplers disagree ({diff:.3e} > {bound:.3e})"
    sm20 = R.Sampler(wl, W, eps, tau_c, tau_u, schedule=[1.0 - i / 20 for i in range(21)])
    ms20, _ = _timed_graph(sm20, 1, 1)
    assert torch.isfinite(sm20.z).all()
    del sm, sm2, sm20
    ewl = CF.WORKLOADS["edit_sampler1024_cfg_bf16"]
    src = S.normal((h * w, d.c_lat), 1.0, "bf16", ewl.name, "src")
    se = R.Sampler(ewl, W, eps, tau_c, tau_u, src=src)
    ms_e, _ = _timed_graph(se, steps, warmup)
    se2 = R.Sampler(ewl, W, eps, tau_c, tau_u, src=src, two_pass=True)
    ms_e2, _ = _timed_graph(se2, steps, warmup)
    assert torch.isfinite(se.z).all()
    ediff = ((se.z - se2.z).abs().max() / se2.z.abs().max()).item()
    assert ediff <= bound, f"packed and two-pass CFG edit samplers disagree ({ediff:.3e} > {bound:.3e})"
    eblk = block_flops(d, se.samples)[0] * ewl.depth * (len(ewl.schedule) - 1)
    return {"ms_per_4step_pack": round(ms, 2), "two_pass_ms_per_4step_pack": round(ms2, 2),
            "packed_speedup_vs_two_pass": round(ms2 / ms, 3), "packed_vs_two_pass_max_rel_diff": diff,
            "packed_vs_two_pass_bound": bound,
            "ms_per_20step_pack": round(ms20, 2),
            "edit": {"workload": f"{ewl.name}: {ewl.note}", "ms_per_4step_pack": round(ms_e, 2),
                     "block_tflops": round(eblk / (ms_e * 1e-3) / 1e12, 1),
                     "two_pass_ms_per_4step_pack": round(ms_e2, 2),
                     "packed_speedup_vs_two_pass": round(ms_e2 / ms_e, 3),
                     "packed_vs_two_pass_max_rel_diff": ediff}}


def _threads():
    try:
        from threadpoolctl import threadpool_info

        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline_sampler(head, min_seconds=10.0):
    """The oracle (float64 numpy) on one block-step of the headline pack: the
    conditioning, the embeddings, block 0 of the 28, the final layer, the CFG
    combine and the Euler update over the whole 8,704-token pack at t = 1,
    with the same bf16 weights and inputs; repeated until at least
    min_seconds of CPU work have been timed.  Rate in block-tokens/s (the
    headline's unit); a pack is 28 x 4 such block-steps."""
    import numpy as np
    import torch

    from oracle import flow as OF
    from oracle import pack as OP

    wl, W = head["wl"], head["W"]
    eps, tau_c, tau_u = head["inputs"]

    def host(t):
        return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)

    Wd = {k: host(v) for k, v in W.wrap.items()}
    Wd["blocks"] = [{s: {k: host(v) for k, v in W.blocks[0][s].items()} for s in ("img", "txt")}]
    samples = head["samples"]
    ref = OP.pack(samples)
    n = samples[0][0] * samples[0][1]
    e64 = np.asarray(eps, np.float64)
    tau = np.concatenate([np.asarray(tau_c, np.float64), np.asarray(tau_u, np.float64)])
    t = np.full(2, wl.schedule[0])
    runs, dt = 0, 0.0
    while runs == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        v = OF.velocity_model(np.concatenate([e64, e64]), tau, t, Wd, ref, wl.dims.heads)
        OF.euler_step(e64, OF.cfg_combine(v[:n], v[n:], wl.guidance), wl.schedule[0], wl.schedule[1])
        dt += time.perf_counter() - t0
        runs += 1
    per = dt / runs
    tok = head["tokens_per_pack"]
    nblk = head["block_tokens_per_pack"] // tok
    return {"value": round(tok / per, 1), "unit": "block-tokens/s", "cores": int(_threads()), "kind": "oracle",
            "sample": f"one block-step (cond, embed, block 0 of {wl.depth}, final layer, CFG + Euler) over the "
                      f"whole {tok}-token pack at t = 1, float64 numpy, {runs} run(s), {dt:.1f} s",
            "ms_per_4step_pack_extrapolated": round(per * nblk * 1e3, 1),
            "extrapolation": f"x{nblk} block-steps ({wl.depth} blocks x {len(wl.schedule) - 1} steps)"}


def bench_chain_vs_copy(reps=10):
    """The RMSNorm + modulate chain against a plain device copy of the same
    bytes (torch's copy_, the practical ceiling of a read-once write-once
    pass): batches of 16 back-to-back launches between two events on their
    stream (one launch queued before the first event, so the host's launch
    cost stays hidden behind the GPU's work), chain and copy batches
    interleaved, median per launch; at the 1024^2 packed-CFG pack's 8,704
    rows and the 1024^2 native pack's 17,280 rows of hidden 3,072 (bf16; two
    samples' modulation vectors)."""
    import statistics

    import torch

    from resolution_image_gen_amd import binding as B
    from resolution_image_gen_amd import configs as CF

    d = CF.B4
    H = d.hidden
    dims = B.Dims(d, "bf16")
    gen = torch.Generator(device="cuda").manual_seed(0)
    res = {}
    for rows in (8704, 17280):
        x = torch.randn(rows, H, generator=gen, device="cuda").to(torch.bfloat16)
        y, yc = torch.empty_like(x), torch.empty_like(x)
        seg = torch.zeros(rows, dtype=torch.int32, device="cuda")
        seg[rows // 2:] = 1
        mod = torch.randn(2, 6 * H, generator=gen, device="cuda")
        fns = {"chain": lambda: B.rms_modulate(dims, x, seg, mod, 0, H, y), "copy": lambda: yc.copy_(x)}
        ts = {k: [] for k in fns}
        for _ in range(3):
            for f in fns.values():
                f()
        torch.cuda.synchronize()
        for _ in range(reps):
            for k, f in fns.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                f()
                e0.record()
                for _ in range(16):
                    f()
                e1.record()
                e1.synchronize()
                ts[k].append(e0.elapsed_time(e1) * 1e3 / 16)
        nb = 2.0 * rows * H * 2
        uc, up = statistics.median(ts["chain"]), statistics.median(ts["copy"])
        res[f"rms_modulate {rows}x{H}"] = {
            "us": round(uc, 2), "GB/s": round(nb / uc / 1e3, 1), "frac_hbm": round(nb / uc / 1e3 / 8000.0, 3),
            "copy_us": round(up, 2), "copy_GB/s": round(nb / up / 1e3, 1), "of_copy": round(up / uc, 3)}
        del x, y, yc
    return res


def bench_rf_kernels(reps=20):
    """Kernel-duration bandwidth of the rectified-flow kernels (noising, loss,
    CFG combine + Euler) at their own pack shapes, where they are launch-bound,
    and at a 64 M-element shape, where they reach steady state.  Bytes are
    algorithmic: noising reads z and eps and writes z_t (3 x 2 B per element);
    the loss reads v, z and eps of every target element (3 x 2 B), the
    negative-aware loss v+, v-, z and eps (4 x 2 B); the Euler
    step reads v_c, v_u (2 x 2 B) and the float32 z, writes z and the next
    bf16 input of both CFG samples (4 + 4 + 2 x 2 B)."""
    import torch

    from resolution_image_gen_amd import binding as B
    from resolution_image_gen_amd import configs as CF

    C = CF.B4.c_lat
    gen = torch.Generator(device="cuda").manual_seed(0)

    def rnd(*shape, dtype=torch.bfloat16):
        return torch.randn(*shape, generator=gen, device="cuda", dtype=torch.float32).to(dtype)

    def timed(fn, tags):
        fn()
        B.timing_enable(True)
        for _ in range(reps):
            fn()
        rep = B.timing_report()
        B.timing_enable(False)
        return sum(rep[t][0] for t in tags if t in rep) / reps * 1e3   # us per call

    res = {}
    noise_shapes = {"256^2 pack": CF.WORKLOADS["pack256_bf16"].samples,
                    "1024^2 pack": CF.WORKLOADS["native1024_bf16"].samples,
                    "64M elements": [(128, 128, 1, 0)] * 32}
    for name, samples in noise_shapes.items():
        pk = B.pack(list(samples))
        n, nt = pk.n_img, pk.n_tgt
        z, eps, zt, v = rnd(n, C), rnd(n, C), torch.empty(n, C, dtype=torch.bfloat16, device="cuda"), rnd(nt, C)
        t = torch.rand(pk.B, generator=gen, device="cuda")
        sse = torch.empty(pk.B, dtype=torch.float32, device="cuda")
        loss = torch.empty(1, dtype=torch.float32, device="cuda")
        ws = torch.empty(nt * 4 + 4, dtype=torch.uint8, device="cuda")
        us = timed(lambda: B.rf_make_xt(pk, z, eps, t, zt), ["make_xt_kernel"])
        res[f"noise {name}"] = {"elements": n * C, "us": round(us, 2), "GB/s": round(6.0 * n * C / us / 1e3, 1)}
        us = timed(lambda: B.rf_loss(pk, v, z, eps, sse, loss, ws), ["row_sse_kernel", "loss_finalize_kernel", "loss_sample_sums_kernel", "loss_mean_kernel"])
        res[f"loss {name}"] = {"elements": nt * C, "us": round(us, 2), "GB/s": round(6.0 * nt * C / us / 1e3, 1)}
        # negative-aware loss: reads v+, v-, z and eps of every target element (4 x 2 B)
        vn = rnd(nt, C)
        r = torch.rand(pk.B, generator=gen, device="cuda")
        us = timed(lambda: B.rf_nft_loss(pk, v, vn, z, eps, r, sse, loss, ws), ["row_nft_kernel", "loss_finalize_kernel", "loss_sample_sums_kernel", "loss_mean_kernel"])
        res[f"nft loss {name}"] = {"elements": nt * C, "us": round(us, 2), "GB/s": round(8.0 * nt * C / us / 1e3, 1)}
        del z, eps, zt, v, vn
    euler_shapes = {"1024^2 CFG pack": [(64, 64, 1, 256)] * 2, "64M elements": [(512, 1024, 1, 0)] * 2}
    for name, samples in euler_shapes.items():
        pk = B.pack(list(samples))
        per = pk.n_tgt // 2
        v = rnd(pk.n_tgt, C)
        z = rnd(per, C, dtype=torch.float32)
        zt = torch.empty(pk.n_img, C, dtype=torch.bfloat16, device="cuda")
        us = timed(lambda: B.rf_euler_step(pk, v, 0, 1, 4.0, 0.75, 0.5, z, zt), ["euler_kernel"])
        res[f"cfg+euler {name}"] = {"elements": per * C, "us": round(us, 2),
                                    "GB/s": round(16.0 * per * C / us / 1e3, 1)}
        del v, z, zt
    for r in res.values():
        r["frac_hbm"] = round(r["GB/s"] / PEAK_HBM_GBS, 3)
    return res


def train_step_flops(wl, depth):
    """Algorithmic FLOPs of one training step: per block the forward
    (24 H^2 N + 4 H sum L_b^2) and the backward (twice the linears, 2.5 times
    the attention), plus the wrapper GEMMs forward and backward (three times)."""
    from resolution_image_gen_amd.configs import block_flops

    _, lin, att = block_flops(wl.dims, wl.samples)
    _, wrap = step_flops(wl)
    wrap -= 2.0 * len(wl.samples) * 12 * wl.dims.hidden ** 2 * (wl.depth - depth)   # modulation of absent blocks
    return depth * (3 * lin + 3.5 * att) + 3 * wrap


def bench_train_step(steps, warmup, depth):
    """ms per training step over the pages' per-GPU workload: one 50,048-token
    native-resolution pack, `depth` random-init blocks forward with saved
    intermediates, the RF loss, then the whole backward (every weight
    gradient, float32)."""
    import torch

    from resolution_image_gen_amd import configs as CF
    from resolution_image_gen_amd import runner as R

    wl = CF.WORKLOADS["train50k_bf16"]
    W = R.Weights(wl, source="torch", depth=depth)
    ts = R.TrainStep(wl, W, R.training_inputs(wl))
    for _ in range(warmup):
        ts.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ts.run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert torch.isfinite(ts.loss).all()
    for g in [ts.grads["wrap"]] + [gb[s] for gb in ts.grads["blocks"] for s in gb]:
        for t in g.values():
            assert torch.isfinite(t).all()
    n = sum(h * w * f + t for h, w, f, t in wl.samples)
    fl = train_step_flops(wl, depth)
    # one more step with every launch bracketed by hipEvents on its stream
    from resolution_image_gen_amd import binding as B

    ts.overlap = False          # one stream, so no launch's events span another's work
    B.timing_enable(True)
    torch.cuda.synchronize()
    ts.run()
    kernels = B.timing_report()
    B.timing_enable(False)
    ts.overlap = R.OVERLAP
    work = train_kernel_work(wl)
    dom = max((k for k in kernels if k in work), key=lambda k: kernels[k][0])
    avg_ms = kernels[dom][0] / kernels[dom][1]
    achieved = work[dom][1] / (avg_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "kernel": dom, "avg_launch_us": round(avg_ms * 1e3, 2)}
    table = {k: round(v[0] / depth * 1e3, 1) for k, v in sorted(kernels.items(), key=lambda kv: -kv[1][0])[:24]}
    return {"workload": f"{wl.name}: {wl.note}", "depth": depth, "ms_per_step": round(ms, 2), "steps_timed": steps,
            "tokens_per_s": round(n / (ms * 1e-3), 1), "tflop_per_step": round(fl / 1e12, 2),
            "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
            "pct_bf16_peak": round(100 * fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "loss": round(ts.loss.item(), 6), "roofline": roof, "kernels_us_per_block": table}


def bench_train_forward(name, steps, warmup, graph=True, weights=None):
    """One training forward per step (pack ids, gathers, RF noising, cond,
    embed, the blocks, final layer, RF loss) over workload `name`: eager ms
    per step over `steps` steps, the same step replayed from a HIP graph, and
    one more pass of `steps` steps on one stream with every launch timed.
    `weights`: device weights of another workload with the same widths, dtype
    and depth to reuse (timing does not depend on their values)."""
    import torch

    from resolution_image_gen_amd import binding as B
    from resolution_image_gen_amd import configs as CF
    from resolution_image_gen_amd import runner as R

    wl = CF.WORKLOADS[name]
    W = weights if weights is not None else R.Weights(wl)
    inputs = R.training_inputs(wl)
    tf = R.TrainForward(wl, W, inputs)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        tf.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        tf.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    graph_ms = None
    if graph:
        tf.capture()
        for _ in range(2):
            tf.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            tf.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / steps
        del tf.graph
    tf.overlap = False
    B.timing_enable(True)
    torch.cuda.synchronize()
    for _ in range(steps):
        tf.run()
    torch.cuda.synchronize()
    kernels = B.timing_report()
    B.timing_enable(False)
    tf.overlap = R.OVERLAP
    n_tokens = sum(f * h * w + t for h, w, f, t in wl.samples)
    blk, wrap = step_flops(wl)
    tflops = (blk + wrap) / (ms_step * 1e-3) / 1e12
    work = kernel_work(wl)
    roof = _roofline(kernels, work)
    roof["traffic"] = measured_traffic(roof["kernel"], wl.name)
    out = {"workload": f"{wl.name}: {wl.note}", "ms_per_step": round(ms_step, 4),
           "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
           "tokens_per_s": round(n_tokens / (ms_step * 1e-3), 1), "tflops": round(tflops, 1),
           "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
           "block_tflop_per_step": round(blk / 1e12, 4), "roofline": roof,
           "kernels_us_per_step": {k: v["us_per_step"]
                                   for k, v in _kernel_lines(kernels, work, steps, "step").items()}}
    return out, (wl, _NumpyWeights(W), inputs, W)


def _compact(res):
    """The headline figures of a bench_train_forward result (no per-kernel table)."""
    keep = ("workload", "ms_per_step", "graph_ms_per_step", "tokens_per_s", "tflops", "pct_bf16_peak",
            "block_tflop_per_step")
    out = {k: res[k] for k in keep}
    r = res["roofline"]
    out["roofline"] = {k: r.get(k) for k in ("bound", "kernel", "avg_launch_us", "achieved", "peak", "unit", "frac")}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed 4-step packs")
    ap.add_argument("--warmup", type=int, default=2, help="untimed packs before the timed ones")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernels", action="store_true", help="print the per-kernel table to stderr")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the 256^2-stage training forward and the RF-kernel legs")
    ap.add_argument("--workload", default=None,
                    help="time only the training forward of this workload (no sampler headline), e.g. "
                         "pack256_bf16, native1024_bf16, edit2048_bf16; the line then reports it")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 times) and exit; used to "
                         "scale the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--sampler-extras", action="store_true",
                    help="also time the two-pass CFG sampler, a 20-step pack and the 4-step editing sampler "
                         "(packed and two-pass) on the same 28 blocks, under 'sampler_extras'")
    ap.add_argument("--train-steps", type=int, default=0,
                    help="also time N training steps (forward + backward, every weight gradient) over one "
                         "50,048-token pack and report them under 'train_step' (0: skip)")
    ap.add_argument("--train-depth", type=int, default=28, help="blocks of the timed training step")
    ap.add_argument("--one-stream", action="store_true",
                    help="every launch on one stream (no side streams), so profiler averages of every launch "
                         "match the instrumented single-stream pass")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: packs are independent, so more GPUs would each take "
              "their own pack with no exchange in the forward pass; no multi-GPU path is built.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_mib": args.copy_calibration_mib, "launches": 3}))
        return

    from resolution_image_gen_amd import runner as R

    if args.one_stream:
        R.OVERLAP = False
    torch.cuda.set_device(0)
    common = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic: seeded N(0,1) latents, noise and text features; random-init N(0,0.02) weights"}

    if args.workload:   # one training-forward workload alone
        res, (wl, Wn, inputs, _) = bench_train_forward(args.workload, args.steps, args.warmup)
        n_tokens = sum(f * h * w + t for h, w, f, t in wl.samples)
        out = {"metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", **common,
               "ms_per_step": res["ms_per_step"], "dtype": wl.dtype,
               "config": {"workload": res["workload"], "tokens_per_step": n_tokens, "samples": len(wl.samples),
                          "hidden": wl.dims.hidden, "heads": wl.dims.heads, "head_dim": wl.dims.head_dim,
                          "mlp": wl.dims.mlp, "blocks": wl.depth},
               **{k: v for k, v in res.items() if k not in ("workload", "ms_per_step", "tokens_per_s")}}
        if args.kernels:
            for k, v in res["kernels_us_per_step"].items():
                print(f"{k:48s} {v:10.1f} us/step", file=sys.stderr)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(wl, Wn, inputs, len(wl.samples))
        print(json.dumps(out), flush=True)
        return

    head = bench_headline(args.steps, args.warmup)
    wl = head["wl"]
    ms = head["ms_per_pack"]
    tflops = head["block_flop_per_pack"] / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(head["block_tokens_per_pack"] / (ms * 1e-3), 1),
        "unit": "block-tokens/s",
        **common,
        "ms_per_step": round(ms, 3),
        "ms_per_4step_pack": round(ms, 3),
        "config": {"workload": f"{wl.name}: {wl.note}", "tokens_per_forward": head["tokens_per_pack"],
                   "samples": [list(s) for s in head["samples"]], "steps_per_pack": len(wl.schedule) - 1,
                   "schedule": list(wl.schedule), "guidance": wl.guidance, "hidden": wl.dims.hidden,
                   "heads": wl.dims.heads, "head_dim": wl.dims.head_dim, "mlp": wl.dims.mlp,
                   "blocks": wl.depth, "timed": "HIP-graph replays of the whole pack"},
        "block_tflops": round(tflops, 1),
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "block_tflop_per_pack": round(head["block_flop_per_pack"] / 1e12, 3),
        "wrapper_tflop_per_pack": round(head["wrap_flop_per_pack"] / 1e12, 3),
        "wall_s_timed": round(head["wall_s_timed"], 3),
        "roofline": head["roofline"],
        "kernels_per_pack": head["kernels"],
    }
    if args.kernels:
        for k, v in head["kernels"].items():
            print(f"{k:48s} {json.dumps(v)}", file=sys.stderr)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_sampler(head)
    if args.sampler_extras:
        out["sampler_extras"] = bench_sampler_extras(head["W"], max(2, args.steps // 3), 1)
    W = head.pop("W")
    del W, head
    torch.cuda.empty_cache()
    if not args.no_secondary:
        res, (_, _, _, W0) = bench_train_forward("pack256_bf16", 20, 5)
        out["train_forward_256"] = res
        # the other one-block configurations at their own packs (same widths:
        # the 256^2 stage's weights are reused), and the tiny float32 pack
        out["native1024_bf16"] = _compact(bench_train_forward("native1024_bf16", 10, 3, weights=W0)[0])
        out["edit2048_bf16"] = _compact(bench_train_forward("edit2048_bf16", 5, 2, weights=W0)[0])
        del W0
        tiny = _compact(bench_train_forward("tiny_f32", 20, 5)[0])
        # float32 (the plain per-element kernels): no bf16 roofline applies
        out["tiny_f32"] = {k: tiny[k] for k in ("workload", "ms_per_step", "graph_ms_per_step", "tokens_per_s")}
        torch.cuda.empty_cache()
        out["rf_kernels"] = bench_rf_kernels()
        out["chains_vs_copy"] = bench_chain_vs_copy()
        torch.cuda.empty_cache()
    if args.train_steps > 0:
        out["train_step"] = bench_train_step(args.train_steps, 1, args.train_depth)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
