"""Whole-path drivers over the C ABI: the training forward with the RF loss
and the packed-CFG Euler sampler.  Marshalling and buffer ownership only:
every arithmetic step is a libmmdit kernel launch on the given stream.
"""

import os

import numpy as np
import torch

from . import binding as B
from . import synthetic as S


def _dev(a, dtype, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dtype)


class Weights:
    """Device weights of a workload: wrapper matrices + `depth` blocks."""

    def __init__(self, wl, device="cuda", recipe="default", depth=None, source="numpy", seed_blocks=None):
        self.wl = wl
        self.dims = B.Dims(wl.dims, wl.dtype)
        dt = self.dims.torch_dtype
        depth = wl.depth if depth is None else depth
        self.np_wrap = S.wrapper_weights(wl.dims, wl.dtype, wl.name, recipe) if source == "numpy" else None
        if source == "numpy":
            self.wrap = {k: _dev(v, dt, device) for k, v in self.np_wrap.items()}
        else:
            self.wrap = _torch_wrap(wl, dt, device)
        self.np_blocks = []
        self.blocks = []
        for i in range(depth):
            blk = seed_blocks[i] if seed_blocks is not None else i
            if source == "numpy":
                nb = S.block_weights(wl.dims, wl.dtype, wl.name, blk, recipe)
                self.np_blocks.append(nb)
                tb = {s: {k: _dev(v, torch.float32 if k in ("g_q", "g_k") else dt, device)
                          for k, v in nb[s].items()} for s in nb}
            else:
                tb = _torch_block(wl, dt, device, blk)
            self.blocks.append(tb)
        self.bw = [B.block_weights(tb) for tb in self.blocks]


def _torch_gen(device, *key):
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([0] + S._key(*key)).generate_state(1)[0]))
    return g


def _torch_normal(shape, std, dt, device, *key):
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=_torch_gen(device, *key))
    return t.to(dt)


def _torch_wrap(wl, dt, device):
    d = wl.dims
    H = d.hidden
    k = (wl.name, "torch", "wrap")
    return {"w_t1": _torch_normal((H, d.t_dim), 0.02, dt, device, *k, "w_t1"),
            "w_t2": _torch_normal((H, H), 0.02, dt, device, *k, "w_t2"),
            "w_in": _torch_normal((H, d.c_lat), 0.02, dt, device, *k, "w_in"),
            "w_txt": _torch_normal((H, d.d_txt), 0.02, dt, device, *k, "w_txt"),
            "w_fmod": _torch_normal((2 * H, H), 0.02, dt, device, *k, "w_fmod"),
            "w_out": _torch_normal((d.c_lat, H), 0.02, dt, device, *k, "w_out")}


def _torch_block(wl, dt, device, blk):
    """Device-side seeded weights for deep stacks (same distributions as the
    numpy recipe, drawn by torch's generator on the GPU for speed)."""
    d = wl.dims
    H, M = d.hidden, d.mlp
    out = {}
    for s in ("img", "txt"):
        k = (wl.name, "torch", "block", blk, s)
        out[s] = {"w_mod": _torch_normal((6 * H, H), 0.02, dt, device, *k, "w_mod"),
                  "w_qkv": _torch_normal((3 * H, H), 0.02, dt, device, *k, "w_qkv"),
                  "g_q": torch.ones(d.head_dim, dtype=torch.float32, device=device),
                  "g_k": torch.ones(d.head_dim, dtype=torch.float32, device=device),
                  "w_o": _torch_normal((H, H), 0.02, dt, device, *k, "w_o"),
                  "w_up": _torch_normal((M, H), 0.02, dt, device, *k, "w_up"),
                  "w_down": _torch_normal((H, M), 0.02, dt, device, *k, "w_down")}
    return out


def training_inputs(wl, samples=None):
    """Packed synthetic inputs (numpy): z, eps [n_img, C]; tau [n_txt, d_txt]; t [B]."""
    samples = wl.samples if samples is None else samples
    d = wl.dims
    n_img = sum(f * h * w for h, w, f, _ in samples)
    n_txt = sum(t for *_, t in samples)
    return {"z": S.latents(n_img, d.c_lat, wl.dtype, wl.name, "z"),
            "eps": S.latents(n_img, d.c_lat, wl.dtype, wl.name, "eps"),
            "tau": S.text(n_txt, d.d_txt, wl.dtype, wl.name, "tau"),
            "t": S.timesteps(len(samples), wl.name)}


# Default for new runners: side streams on (conditioning and adaLN vectors
# beside the embeddings; the backward's weight gradients beside its input
# gradients).  False puts every launch on the caller's stream.
OVERLAP = True
# The packed sampler computes every step's adaLN vectors in one pass over the
# weights when they fit one weight-streaming product; MMDIT_SAMPLER_ALL_STEPS=0
# computes them per step (the same bits).
ALL_STEP_VECTORS = os.environ.get("MMDIT_SAMPLER_ALL_STEPS", "1") != "0"


class _SideMods:
    """The conditioning and the adaLN vectors of every block and of the final
    layer, on a side stream.  They depend on t and the weights only, so these
    weight-streaming (HBM-bound) launches run while the main stream gathers,
    noises and embeds (MFMA-bound); the main stream waits for block i's
    vectors right before block i.  Same kernels, so the same bits as the
    single-stream calls.  Default-priority stream; events without timing."""

    def __init__(self, W, n_samples, device, steps=0):
        H, dt = W.dims.c.hidden, W.dims.torch_dtype
        es = 2 if dt == torch.bfloat16 else 4
        nb = len(W.bw)
        self.n_samples = n_samples
        self.mods = torch.empty(nb, 2, n_samples, 6 * H, dtype=torch.float32, device=device)
        self.modf = torch.empty(n_samples, 2 * H, dtype=torch.float32, device=device)
        self.ws = torch.empty(n_samples * (W.dims.c.t_dim + H) * es + 1024, dtype=torch.uint8, device=device)
        if steps:   # launch_steps: every step's vectors at once
            rows = steps * n_samples
            self.c_all = torch.empty(rows, H, dtype=dt, device=device)
            self.ws_all = torch.empty(rows * (W.dims.c.t_dim + H) * es + 1024, dtype=torch.uint8, device=device)
            self.mods_all = torch.empty(2, rows, 6 * H, dtype=torch.float32, device=device)
            self.modf_all = torch.empty(rows, 2 * H, dtype=torch.float32, device=device)
            self.mods_steps = torch.empty(steps, nb, 2, n_samples, 6 * H, dtype=torch.float32, device=device)
        self.stream = torch.cuda.Stream(device=device)
        self.ev_start = torch.cuda.Event()
        self.ev_mod = [torch.cuda.Event() for _ in range(nb)]
        self.ev_modf = torch.cuda.Event()

    def launch(self, W, dm, t, c, main, overlap=True):
        """cond, then every block's vectors and the final layer's, after main's
        current point (on main itself when overlap is False)."""
        side = self.stream if overlap else main
        self.ev_start.record(main)
        side.wait_event(self.ev_start)
        B.cond(dm, W.wrap["w_t1"], W.wrap["w_t2"], t, c, self.ws, side)
        for i, bw in enumerate(W.bw):
            B.block_modulation(dm, bw, c, self.mods[i], side)
            self.ev_mod[i].record(side)
        B.modulation(dm, W.wrap["w_fmod"], 2, c, self.modf, side)
        self.ev_modf.record(side)

    def launch_steps(self, W, dm, t_all, main, overlap=True):
        """The vectors of every step of a sampler pack in one pass over the
        weights: cond and every block's and the final layer's vectors for all
        S steps' rows at once (t_all [S * B], step-major; S * B <= 16, the
        rows the weight-streaming GEMV takes in one product, each row's
        arithmetic the same as alone), then each block's [2][S][B][6H] copied
        into per-step [2][B][6H] slots (mods_steps[k][i]); one event per
        block as in launch."""
        side = self.stream if overlap else main
        S = t_all.shape[0] // self.n_samples
        self.ev_start.record(main)
        side.wait_event(self.ev_start)
        c_all = self.c_all[:S * self.n_samples]
        B.cond(dm, W.wrap["w_t1"], W.wrap["w_t2"], t_all, c_all, self.ws_all, side)
        B.modulation(dm, W.wrap["w_fmod"], 2, c_all, self.modf_all[:S * self.n_samples], side)
        H6 = self.mods.shape[-1]
        for i, bw in enumerate(W.bw):
            m = self.mods_all[:, :S * self.n_samples]
            B.block_modulation(dm, bw, c_all, m, side)
            with torch.cuda.stream(side):
                self.mods_steps[:S, i].copy_(m.view(2, S, self.n_samples, H6).permute(1, 0, 2, 3))
            self.ev_mod[i].record(side)
        self.ev_modf.record(side)

    def blocks_and_final_step(self, W, dm, pk, k, x_img, x_txt, ws, v, main):
        """Step k's blocks and final layer with the vectors of launch_steps
        (each block waits for its own vectors only on the first step)."""
        for i, bw in enumerate(W.bw):
            if k == 0:
                main.wait_event(self.ev_mod[i])
            B.block_fwd_mod(dm, bw, pk, self.mods_steps[k, i], x_img, x_txt, ws, main)
        if k == 0:
            main.wait_event(self.ev_modf)
        nb = self.n_samples
        B.final_mod(dm, W.wrap["w_out"], pk, self.modf_all[k * nb:(k + 1) * nb], x_img, v, ws, main)

    def blocks_and_final(self, W, dm, pk, x_img, x_txt, ws, v, main, loss=None):
        """Every block, then the final layer; with loss = (z, eps, sse, loss)
        the final layer and the RF loss in one call (rf_final_loss)."""
        for i, bw in enumerate(W.bw):
            main.wait_event(self.ev_mod[i])
            B.block_fwd_mod(dm, bw, pk, self.mods[i], x_img, x_txt, ws, main)
        main.wait_event(self.ev_modf)
        if loss is None:
            B.final_mod(dm, W.wrap["w_out"], pk, self.modf, x_img, v, ws, main)
        else:
            z, eps, sse, lo = loss
            B.rf_final_loss(dm, W.wrap["w_out"], pk, self.modf, x_img, z, eps, v, sse, lo, ws, main)


class TrainForward:
    """One training forward over a pack: gather per-sample tensors, noise,
    condition, embed, run the blocks, final layer and RF loss."""

    def __init__(self, wl, W, inputs, device="cuda", samples=None, img_budget=None):
        self.wl, self.W = wl, W
        self.samples = list(wl.samples if samples is None else samples)
        budget = wl.img_budget if img_budget is None else img_budget
        n_taken = B.pack_plan(self.samples, budget)[0]
        if n_taken != len(self.samples):
            raise ValueError(f"workload does not fit one pack ({n_taken} of {len(self.samples)})")
        d = wl.dims
        self.dims = W.dims
        dt = self.dims.torch_dtype
        self.device = device
        self.pk = B.pack(self.samples, device)
        pk = self.pk
        cu_img, cu_txt = pk.host("h_cu_img"), pk.host("h_cu_txt")
        z = _dev(inputs["z"], dt, device)
        eps = _dev(inputs["eps"], dt, device)
        tau = _dev(inputs["tau"], dt, device)
        # per-sample tensors: the path starts from separate samples and packs them
        self.z_s = [z[cu_img[b]:cu_img[b + 1]].clone() for b in range(pk.B)]
        self.eps_s = [eps[cu_img[b]:cu_img[b + 1]].clone() for b in range(pk.B)]
        self.tau_s = [tau[cu_txt[b]:cu_txt[b + 1]].clone() for b in range(pk.B)]
        self.t = torch.from_numpy(inputs["t"]).to(device)
        e = dict(dtype=dt, device=device)
        ni, nt, ng = max(pk.n_img, 1), max(pk.n_txt, 1), max(pk.n_tgt, 1)
        self.z = torch.empty(ni, d.c_lat, **e)
        self.eps = torch.empty(ni, d.c_lat, **e)
        self.tau = torch.empty(nt, d.d_txt, **e)
        self.zt = torch.empty(ni, d.c_lat, **e)
        self.c = torch.empty(pk.B, d.hidden, **e)
        self.x_img = torch.empty(ni, d.hidden, **e)
        self.x_txt = torch.empty(nt, d.hidden, **e)
        self.v = torch.empty(ng, d.c_lat, **e)
        self.sse = torch.empty(max(pk.B, 1), dtype=torch.float32, device=device)
        self.loss = torch.empty(1, dtype=torch.float32, device=device)
        self.ws = torch.empty(B.workspace_size(self.dims, pk), dtype=torch.uint8, device=device)
        self.side = _SideMods(W, pk.B, device)
        # False: every launch on the one stream (per-kernel timing wants
        # launches that do not overlap)
        self.overlap = OVERLAP

    def run(self, stream=None, repack=True):
        W, pk, dm = self.W, self.pk, self.dims
        main = stream if stream is not None else torch.cuda.current_stream()
        if repack:
            pk = self._repack(main)
        self.side.launch(W, dm, self.t, self.c, main, self.overlap)
        B.pack_gather(pk, 0, self.z_s, self.z, main)
        B.pack_gather(pk, 0, self.eps_s, self.eps, main)
        B.pack_gather(pk, 1, self.tau_s, self.tau, main)
        # noising folded into the image embedding, the loss's row sums into
        # the final layer
        B.rf_embed(dm, W.wrap["w_in"], W.wrap["w_txt"], pk, self.z, self.eps, self.t, self.tau, self.x_img,
                   self.x_txt, self.zt, main)
        self.side.blocks_and_final(W, dm, pk, self.x_img, self.x_txt, self.ws, self.v, main,
                                   loss=(self.z, self.eps, self.sse, self.loss))

    def capture(self):
        """Record one whole training forward (every launch) as a HIP graph."""
        self.run()                           # first call sets kernel attributes
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run()
        torch.cuda.synchronize()
        return self.graph

    def replay(self):
        self.graph.replay()
        return self.loss

    def _repack(self, stream):
        # rebuild the ids of the pack in place (same buffers, same samples)
        pk = self.pk
        B._ck(B._lib.mmdit_pack(B._samples(self.samples), len(self.samples), pk.ref, B._stream(stream)))
        return pk


WRAP_KEYS = ("w_t1", "w_t2", "w_in", "w_txt", "w_fmod", "w_out")


class TrainStep(TrainForward):
    """One training step over a pack: the forward of TrainForward with every
    block's intermediates kept (one saved buffer per block), then the whole
    backward: loss gradient, final layer, the blocks in reverse order, the
    embeddings and the conditioning.  Every weight gradient lands in
    self.grads (float32, the shape of its weight): self.grads["wrap"][name]
    and self.grads["blocks"][i]["img" | "txt"][name]."""

    def __init__(self, wl, W, inputs, device="cuda", samples=None, img_budget=None):
        super().__init__(wl, W, inputs, device, samples, img_budget)
        pk, dm = self.pk, self.dims
        d = wl.dims
        f32 = dict(dtype=torch.float32, device=device)
        nsv = B.block_saved_size(dm, pk)
        self.saved = [torch.empty(nsv, dtype=torch.uint8, device=device) for _ in W.bw]
        self.ws_bwd = torch.empty(max(B.block_bwd_workspace_size(dm, pk), B.wrap_bwd_workspace_size(dm, pk),
                                      B.cond_bwd_workspace_size(dm, pk.B), 256), dtype=torch.uint8, device=device)
        e = dict(dtype=dm.torch_dtype, device=device)
        self.dv = torch.empty(max(pk.n_tgt, 1), d.c_lat, **e)
        self.dx_img = torch.empty(max(pk.n_img, 1), d.hidden, **e)
        self.dx_txt = torch.empty(max(pk.n_txt, 1), d.hidden, **e)
        self.dc = torch.empty(max(pk.B, 1), d.hidden, **f32)
        self.modf = torch.empty(max(pk.B, 1), 2 * d.hidden, **f32)
        self.grads = {"wrap": {k: torch.empty(tuple(W.wrap[k].shape), **f32) for k in WRAP_KEYS},
                      "blocks": [{s: {k: torch.empty(tuple(blk[s][k].shape), **f32) for k in B.GRAD_KEYS}
                                  for s in ("img", "txt")} for blk in W.blocks]}
        self.bg = [B.block_grads(g) for g in self.grads["blocks"]]
        # the blocks' weight gradients run on their own stream beside the
        # input-gradient chain (mmdit_block_bwd2); default priority
        self.wstream = torch.cuda.Stream(device=device)

    def run(self, stream=None, repack=True):
        W, pk, dm = self.W, self.pk, self.dims
        if repack:
            pk = self._repack(stream)
        B.pack_gather(pk, 0, self.z_s, self.z, stream)
        B.pack_gather(pk, 0, self.eps_s, self.eps, stream)
        B.pack_gather(pk, 1, self.tau_s, self.tau, stream)
        B.cond(dm, W.wrap["w_t1"], W.wrap["w_t2"], self.t, self.c, self.ws, stream)
        B.rf_embed(dm, W.wrap["w_in"], W.wrap["w_txt"], pk, self.z, self.eps, self.t, self.tau, self.x_img,
                   self.x_txt, self.zt, stream)
        for bw, sv in zip(W.bw, self.saved):
            B.block_fwd_train(dm, bw, pk, self.c, self.x_img, self.x_txt, sv, self.ws, stream)
        B.modulation(dm, W.wrap["w_fmod"], 2, self.c, self.modf, stream)
        B.rf_final_loss(dm, W.wrap["w_out"], pk, self.modf, self.x_img, self.z, self.eps, self.v, self.sse,
                        self.loss, self.ws, stream)
        # backward
        g = self.grads["wrap"]
        self.dc.zero_()
        B.rf_loss_grad(pk, self.v, self.z, self.eps, self.dv, stream)
        B.final_bwd(dm, W.wrap["w_fmod"], W.wrap["w_out"], pk, self.c, self.x_img, self.dv, self.dx_img,
                    g["w_fmod"], g["w_out"], self.dc, self.ws_bwd, stream)
        self.dx_txt.zero_()
        for i in range(len(W.bw) - 1, -1, -1):
            B.block_bwd(dm, W.bw[i], pk, self.c, self.saved[i], self.dx_img, self.dx_txt, self.bg[i], self.dc,
                        self.ws_bwd, stream, stream_w=self.wstream if self.overlap else None)
        B.embed_bwd(dm, pk, self.zt, self.tau, self.dx_img, self.dx_txt, g["w_in"], g["w_txt"], self.ws_bwd, stream)
        B.cond_bwd(dm, W.wrap["w_t1"], W.wrap["w_t2"], self.t, self.dc, g["w_t1"], g["w_t2"], self.ws_bwd, stream)


class Sampler:
    """Packed-CFG Euler sampler: one pack [cond, uncond] of the same grid,
    `steps` forwards through the block stack, CFG combine + Euler per step.

    two_pass=True samples the unpacked way, as the comparison point for
    packing: per step one forward over the conditional sample and one over
    the unconditional sample (each a one-sample pack), writing the two
    velocities into the halves of the same buffer, then the same CFG combine
    + Euler launch.  Every row's arithmetic is the same in both forms, so the
    two give the same bits.

    src (the clean source latent [h*w, C] of an edit) makes both samples
    editing samples: image rows [target (frame 0); source (frame 1)], the
    source rows written once per pack and never updated; the velocity, the
    CFG combine and the Euler step touch the target rows only."""

    def __init__(self, wl, W, eps, tau_c, tau_u, device="cuda", guidance=None, schedule=None,
                 two_pass=False, src=None):
        self.wl, self.W = wl, W
        d = wl.dims
        self.dims = W.dims
        dt = self.dims.torch_dtype
        h, w = wl.samples[0][0], wl.samples[0][1]
        f = 1 if src is None else 2
        self.samples = [(h, w, f, len(tau_c)), (h, w, f, len(tau_u))]
        self.pk = B.pack(self.samples, device)
        self.g = float(wl.guidance if guidance is None else guidance)
        self.schedule = list(wl.schedule if schedule is None else schedule)
        e = dict(dtype=dt, device=device)
        self.eps = torch.from_numpy(np.ascontiguousarray(eps, np.float32)).to(device)
        self.z = torch.empty_like(self.eps)
        self.tau = torch.cat([_dev(tau_c, dt, device), _dev(tau_u, dt, device)])
        n = self.pk.n_img
        self.zt = torch.empty(n, d.c_lat, **e)
        self.c = torch.empty(2, d.hidden, **e)
        self.x_img = torch.empty(n, d.hidden, **e)
        self.x_txt = torch.empty(self.pk.n_txt, d.hidden, **e)
        self.v = torch.empty(self.pk.n_tgt, d.c_lat, **e)
        self.tsched = torch.tensor([[t, t] for t in self.schedule[:-1]], dtype=torch.float32, device=device)
        self.ws = torch.empty(B.workspace_size(self.dims, self.pk), dtype=torch.uint8, device=device)
        # an edit sample's image rows at z_1 = eps: [eps; source], both in dtype
        self.img_rows = None if src is None else torch.cat([_dev(eps, dt, device), _dev(src, dt, device)])
        self.two_pass = two_pass
        nsteps = len(self.schedule) - 1
        # every step's adaLN vectors in one pass over the weights when the
        # steps' rows fit one weight-streaming product (4 steps x 2 samples)
        self.all_steps = ALL_STEP_VECTORS and not two_pass and 2 * nsteps <= 16
        self.side = _SideMods(W, 2, device, steps=nsteps if self.all_steps else 0)
        self.t_all = self.tsched.reshape(-1).contiguous()
        self.overlap = OVERLAP
        if two_pass:   # one-sample packs; the two-sample workspace covers each
            self.pk_one = [B.pack(self.samples[:1], device), B.pack(self.samples[1:], device)]

    def capture(self):
        """Record one whole pack (every launch of the 4 steps) as a HIP graph.

        The library allocates nothing and records no memset, so the graph
        replays the same launches on the same buffers."""
        self.run()                           # first call sets kernel attributes
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run()
        torch.cuda.synchronize()
        return self.graph

    def replay(self):
        self.graph.replay()
        return self.z

    def _two_pass_forward(self, i, stream):
        """Velocities of step i as two forwards: cond rows, then uncond rows."""
        W, dm = self.W, self.dims
        ib = it = iv = 0
        for pk in self.pk_one:
            ni, nt, nv = pk.n_img, pk.n_txt, pk.n_tgt
            B.cond(dm, W.wrap["w_t1"], W.wrap["w_t2"], self.tsched[i, :1], self.c[:1], self.ws, stream)
            B.embed(dm, W.wrap["w_in"], W.wrap["w_txt"], pk, self.zt[ib:ib + ni], self.tau[it:it + nt],
                    self.x_img[:ni], self.x_txt[:nt], stream)
            for bw in W.bw:
                B.block_fwd(dm, bw, pk, self.c[:1], self.x_img[:ni], self.x_txt[:nt], self.ws, stream)
            B.final(dm, W.wrap["w_fmod"], W.wrap["w_out"], pk, self.c[:1], self.x_img[:ni],
                    self.v[iv:iv + nv], self.ws, stream)
            ib, it, iv = ib + ni, it + nt, iv + nv

    def run(self, stream=None, on_step=None):
        W, pk, dm = self.W, self.pk, self.dims
        self.z.copy_(self.eps)               # z_1 = eps
        if self.img_rows is not None:         # source rows of both samples (targets too, as eps)
            B.pack_gather(pk, 0, [self.img_rows, self.img_rows], self.zt, stream)
        B.rf_pack_latent(pk, self.z, 0, 1, self.zt, stream)
        main = stream if stream is not None else torch.cuda.current_stream()
        if self.all_steps:
            self.side.launch_steps(W, dm, self.t_all, main, self.overlap)
        for i in range(len(self.schedule) - 1):
            if self.two_pass:
                self._two_pass_forward(i, stream)
            elif self.all_steps:
                B.embed(dm, W.wrap["w_in"], W.wrap["w_txt"], pk, self.zt, self.tau, self.x_img, self.x_txt,
                        main)
                self.side.blocks_and_final_step(W, dm, pk, i, self.x_img, self.x_txt, self.ws, self.v, main)
            else:
                self.side.launch(W, dm, self.tsched[i], self.c, main, self.overlap)
                B.embed(dm, W.wrap["w_in"], W.wrap["w_txt"], pk, self.zt, self.tau, self.x_img, self.x_txt,
                        main)
                self.side.blocks_and_final(W, dm, pk, self.x_img, self.x_txt, self.ws, self.v, main)
            if on_step is not None:
                on_step(i, self)
            B.rf_euler_step(pk, self.v, 0, 1, self.g, self.schedule[i], self.schedule[i + 1], self.z,
                            self.zt, stream)
        return self.z
