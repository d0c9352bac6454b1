#!/usr/bin/env python3
"""Benchmark of the packed NR-MMDiT hot path on one MI355X.

One step = one training forward over one synthetic pack, all on the GPU:
pack ids -> gather per-sample tensors -> RF noising -> timestep conditioning
-> token embedding -> one dual-stream block -> final layer -> RF loss.
Default workload: the 256^2-stage pack, 16 samples x (16x16 latent grid +
128 text tokens), hidden 3072, 24 x 128 heads, MLP 12288, bf16.

Prints ONE JSON line.  `value` is whole-step token throughput (image + text
tokens per second) over K eagerly launched steps bracketed by hipEvents;
`graph_ms_per_step` is the same step replayed from a HIP graph.  A second pass
of K steps brackets every launch with hipEvents on its stream (that would add
~9% to the step if done in the first pass): it gives the per-kernel table and
the roofline of the dominant kernel.  The line also carries the block's
TFLOP/s against the bf16 MFMA peak and the CPU oracle timed on a bounded
sample.
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


def kernel_work(wl):
    """Algorithmic work per launch of each tagged kernel of one step."""
    d = wl.dims
    H, M = d.hidden, d.mlp
    n = sum(f * h * w + t for h, w, f, t in wl.samples)
    n_tgt = sum(h * w for h, w, _, _ in wl.samples)
    att = sum((f * h * w + t) ** 2 for h, w, f, t in wl.samples)
    es = 2 if wl.dtype == "bf16" else 4
    return {
        "qkv_proj": ("mfma", 2.0 * n * H * 3 * H),
        "out_proj_gated": ("mfma", 2.0 * n * H * H),
        "mlp_up_gelu": ("mfma", 2.0 * n * H * M),
        "mlp_down_gated": ("mfma", 2.0 * n * M * H),
        "attn_mfma_kernel": ("mfma", 4.0 * H * att),
        # read x, write y: two launches over all N rows + one over the target rows, averaged
        "rms_modulate_kernel": ("hbm", (2 * (2.0 * es * H * n) + 2.0 * es * H * n_tgt) / 3),
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


def bench_sampler(steps, warmup):
    """ms per 4-step packed-CFG pack: cond + uncond (64x64 grid + 256 text
    tokens each), 28 random-init blocks, guidance 4, t = 1, .75, .5, .25 -> 0.
    The same sampler with the two CFG branches as separate forwards is timed
    beside it, and both must end on the same bits; then one 20-step pack
    (uniform steps from 1 to 0) of the packed sampler, and the 4-step editing
    sampler (target + clean source of the same grid per sample), packed and
    two-pass, on the same blocks."""
    import torch

    from resolution_image_gen_amd import configs as CF
    from resolution_image_gen_amd import runner as R
    from resolution_image_gen_amd import synthetic as S
    from resolution_image_gen_amd.configs import block_flops

    wl = CF.WORKLOADS["sampler1024_cfg_bf16"]
    d = wl.dims
    W = R.Weights(wl, source="torch")            # 28 blocks drawn on the GPU (19 GB bf16)
    h, w, _, T = wl.samples[0]
    eps = S.normal((h * w, d.c_lat), 1.0, "bf16", wl.name, "eps")
    tau_c = S.text(T, d.d_txt, "bf16", wl.name, "tau_c")
    tau_u = S.text(T, d.d_txt, "bf16", wl.name, "tau_u")

    def timed(sm, steps=steps):
        sm.capture()                          # one pack = one HIP graph (~1,600 launches at 4 steps)
        for _ in range(warmup):
            sm.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            sm.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        del sm.graph
        return ms

    sm = R.Sampler(wl, W, eps, tau_c, tau_u)
    ms = timed(sm)
    sm2 = R.Sampler(wl, W, eps, tau_c, tau_u, two_pass=True)
    ms2 = timed(sm2)
    assert torch.isfinite(sm.z).all()
    assert torch.equal(sm.z, sm2.z), "packed and two-pass CFG samplers disagree"
    sm_samples = sm.samples
    # the base (non-distilled) sampler: 20 uniform Euler steps, packed CFG
    sm20 = R.Sampler(wl, W, eps, tau_c, tau_u, schedule=[1.0 - i / 20 for i in range(21)])
    ms20 = timed(sm20, steps=1)
    assert torch.isfinite(sm20.z).all()
    del sm, sm2, sm20
    # the 4-step editing sampler on the same blocks: each sample a noised 64x64
    # target + the clean 64x64 source (frames 0 / 1) + text; packed and two-pass
    ewl = CF.WORKLOADS["edit_sampler1024_cfg_bf16"]
    src = S.normal((h * w, d.c_lat), 1.0, "bf16", ewl.name, "src")
    se = R.Sampler(ewl, W, eps, tau_c, tau_u, src=src)
    ms_e = timed(se)
    se2 = R.Sampler(ewl, W, eps, tau_c, tau_u, src=src, two_pass=True)
    ms_e2 = timed(se2)
    assert torch.isfinite(se.z).all()
    assert torch.equal(se.z, se2.z), "packed and two-pass CFG edit samplers disagree"
    eblk = block_flops(d, se.samples)[0] * ewl.depth * (len(ewl.schedule) - 1)
    blk = block_flops(d, sm_samples)[0] * wl.depth * (len(wl.schedule) - 1)
    n = sum(hh * ww * f + t for hh, ww, f, t in sm_samples)
    return {"workload": f"{wl.name}: {wl.note}", "ms_per_4step_pack": round(ms, 2), "packs_timed": steps,
            "block_tokens_per_s": round(n * wl.depth * (len(wl.schedule) - 1) / (ms * 1e-3), 1),
            "block_tflops": round(blk / (ms * 1e-3) / 1e12, 1),
            "pct_bf16_peak": round(100 * blk / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "two_pass_ms_per_4step_pack": round(ms2, 2),
            "packed_speedup_vs_two_pass": round(ms2 / ms, 3),
            "ms_per_20step_pack": round(ms20, 2),
            "edit": {"workload": f"{ewl.name}: {ewl.note}", "ms_per_4step_pack": round(ms_e, 2),
                     "block_tflops": round(eblk / (ms_e * 1e-3) / 1e12, 1),
                     "two_pass_ms_per_4step_pack": round(ms_e2, 2),
                     "packed_speedup_vs_two_pass": round(ms_e2 / ms_e, 3)}}


def bench_rf_kernels(reps=20):
    """Kernel-duration bandwidth of the rectified-flow kernels (noising, loss,
    CFG combine + Euler) at their own pack shapes, where they are launch-bound,
    and at a 64 M-element shape, where they reach steady state.  Bytes are
    algorithmic: noising reads z and eps and writes z_t (3 x 2 B per element);
    the loss reads v, z and eps of every target element (3 x 2 B); the Euler
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
        us = timed(lambda: B.rf_loss(pk, v, z, eps, sse, loss, ws), ["row_sse_kernel", "loss_finalize_kernel"])
        res[f"loss {name}"] = {"elements": nt * C, "us": round(us, 2), "GB/s": round(6.0 * nt * C / us / 1e3, 1)}
        del z, eps, zt, v
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="pack256_bf16")
    ap.add_argument("--cpu-samples", type=int, default=16, help="samples of the pack the CPU oracle runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernels", action="store_true", help="print the per-kernel table to stderr")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 times) and exit; used to "
                         "scale the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--train-steps", type=int, default=0,
                    help="also time N training steps (forward + backward, every weight gradient) over one "
                         "50,048-token pack and report them under 'train_step' (0: skip)")
    ap.add_argument("--train-depth", type=int, default=28, help="blocks of the timed training step")
    ap.add_argument("--one-stream", action="store_true",
                    help="every launch on one stream (no side streams), so profiler averages of every launch "
                         "match the instrumented single-stream pass")
    ap.add_argument("--sampler-packs", type=int, default=0,
                    help="also time N packs of the 4-step packed-CFG sampler (28 blocks) and report them "
                         "under 'sampler' (0: skip)")
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

    from resolution_image_gen_amd import binding as B
    from resolution_image_gen_amd import configs as CF
    from resolution_image_gen_amd import runner as R

    if args.one_stream:
        R.OVERLAP = False
    wl = CF.WORKLOADS[args.workload]
    if wl.steps:
        raise SystemExit("the sampler workloads are timed with --sampler-packs N next to a training-forward "
                         "workload")
    torch.cuda.set_device(0)
    W = R.Weights(wl)
    W_np = _NumpyWeights(W)
    inputs = R.training_inputs(wl)
    tf = R.TrainForward(wl, W, inputs)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        tf.run()
    torch.cuda.synchronize()

    # timed region (hipEvents on the launch stream bracket the whole region)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        tf.run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps

    # the same step replayed from a HIP graph (launch overhead removed)
    graph_ms = None
    if not args.no_graph:
        tf.capture()
        for _ in range(2):
            tf.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            tf.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / args.steps
        del tf.graph

    # per-kernel times: every launch bracketed by hipEvents on its stream,
    # all on one stream so no launch's events span another's work
    tf.overlap = False
    B.timing_enable(True)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        tf.run()
    torch.cuda.synchronize()
    kernels = B.timing_report()
    B.timing_enable(False)
    tf.overlap = R.OVERLAP

    n_tokens = sum(f * h * w + t for h, w, f, t in wl.samples)
    blk, wrap = step_flops(wl)
    tflops = (blk + wrap) / (ms_step * 1e-3) / 1e12
    work = kernel_work(wl)
    # dominant kernel: largest total time among kernels with a known algorithmic work
    dom = max((k for k in kernels if k in work), key=lambda k: kernels[k][0])
    kind, per_launch = work[dom]
    avg_ms = kernels[dom][0] / kernels[dom][1]
    if kind == "mfma":
        achieved = per_launch / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}
    else:
        achieved = per_launch / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    roof["kernel"] = dom
    roof["avg_launch_us"] = round(avg_ms * 1e3, 2)
    roof["traffic"] = measured_traffic(dom, wl.name)

    table = {k: {"ms_per_step": round(v[0] / args.steps, 4), "launches_per_step": v[1] / args.steps}
             for k, v in sorted(kernels.items(), key=lambda kv: -kv[1][0])}
    if args.kernels:
        for k, v in table.items():
            extra = ""
            if k in work:
                kd, wk = work[k]
                per = v["ms_per_step"] / v["launches_per_step"] * 1e-3
                extra = (f"  {wk / per / 1e12:8.1f} TFLOP/s" if kd == "mfma" else f"  {wk / per / 1e9:8.1f} GB/s")
            print(f"{k:48s} {v['ms_per_step'] * 1e3:10.1f} us/step  x{v['launches_per_step']:.0f}{extra}",
                  file=sys.stderr)

    out = {
        "metric": METRIC,
        "value": round(n_tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: seeded N(0,1) latents, noise and text features; random-init N(0,0.02) weights",
        "config": {"workload": f"{wl.name}: {wl.note}", "tokens_per_step": n_tokens,
                   "samples": len(wl.samples), "hidden": wl.dims.hidden, "heads": wl.dims.heads,
                   "head_dim": wl.dims.head_dim, "mlp": wl.dims.mlp, "blocks": wl.depth},
        "tflops": round(tflops, 1),
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "block_tflop_per_step": round(blk / 1e12, 4),
        "wall_s_timed": round(wall, 3),
        "graph_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "roofline": roof,
        "kernels_us_per_step": {k: round(v["ms_per_step"] * 1e3, 1) for k, v in table.items()},
    }
    out["rf_kernels"] = bench_rf_kernels()
    if args.sampler_packs > 0 or args.train_steps > 0:
        del tf, W
        torch.cuda.empty_cache()
    if args.sampler_packs > 0:
        out["sampler"] = bench_sampler(args.sampler_packs, 1)
        torch.cuda.empty_cache()
    if args.train_steps > 0:
        out["train_step"] = bench_train_step(args.train_steps, 1, args.train_depth)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, W_np, inputs, args.cpu_samples)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
