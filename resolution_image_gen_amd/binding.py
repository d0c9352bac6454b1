"""Python binding of libmmdit (HIP, gfx950): argument marshalling only.

Every step of the path runs in the library's kernels.  PyTorch supplies
device memory (tensors) and streams; the binding passes raw pointers and
sizes through the C ABI declared in include/mmdit.h and raises MmditError on
any non-zero status.  Importing this module loads libmmdit.so and fails
loudly if it has not been built.
"""

import ctypes
import os

__all__ = [
    "MmditError", "Pack", "Dims", "lib_path", "pack_plan", "pack", "pack_gather",
    "workspace_size", "workspace_layout", "cond", "modulation", "embed", "block_fwd",
    "rms_modulate", "qk_norm_rope", "attention", "linear", "final", "rf_make_xt", "rf_embed", "rf_final_loss",
    "rf_loss", "rf_loss_noalloc", "rf_nft_loss", "rf_euler_step", "rf_pack_latent", "EPI_STORE", "EPI_STORE_F32", "EPI_GELU",
    "EPI_GATED_RES", "MAX_SAMPLES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmmdit.so")

MAX_SAMPLES = 256
F32, BF16 = 0, 1
EPI_STORE, EPI_STORE_F32, EPI_GELU, EPI_GATED_RES = 0, 1, 2, 3

_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t


class MmditError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libmmdit status {status}: {msg}")
        self.status = status


class _Sample(ctypes.Structure):
    _fields_ = [("h", _i32), ("w", _i32), ("frames", _i32), ("txt_len", _i32)]


class _PackT(ctypes.Structure):
    _fields_ = [
        ("B", _i32), ("max_joint", _i32), ("n_img", _i64), ("n_txt", _i64), ("n_tgt", _i64),
        ("cu_txt", _vp), ("cu_img", _vp), ("cu_joint", _vp), ("cu_tgt", _vp), ("tgt_len", _vp),
        ("seg_img", _vp), ("seg_txt", _vp), ("pos_img", _vp), ("tgt_row", _vp),
        ("h_cu_txt", _i32 * (MAX_SAMPLES + 1)), ("h_cu_img", _i32 * (MAX_SAMPLES + 1)),
        ("h_cu_tgt", _i32 * (MAX_SAMPLES + 1)), ("h_frames", _i32 * MAX_SAMPLES),
    ]


class _DimsT(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("heads", _i32), ("head_dim", _i32), ("mlp", _i32),
                ("c_lat", _i32), ("d_txt", _i32), ("t_dim", _i32), ("rope_dims", _i32 * 3),
                ("rope_theta", _f32), ("eps", _f32), ("dtype", _i32)]


class _StreamW(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("w_mod", "w_qkv", "g_q", "g_k", "w_o", "w_up", "w_down")]


class _BlockW(ctypes.Structure):
    _fields_ = [("img", _StreamW), ("txt", _StreamW)]


GRAD_KEYS = ("w_mod", "w_qkv", "g_q", "g_k", "w_o", "w_up", "w_down")


class _StreamG(ctypes.Structure):
    _fields_ = [(k, _vp) for k in GRAD_KEYS]


class _BlockG(ctypes.Structure):
    _fields_ = [("img", _StreamG), ("txt", _StreamG)]


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is missing: build it with `python -m resolution_image_gen_amd.build`")
    lib = ctypes.CDLL(lib_path)
    P, D = ctypes.POINTER(_PackT), ctypes.POINTER(_DimsT)
    sig = {
        "mmdit_last_error": (ctypes.c_char_p, []),
        "mmdit_version": (ctypes.c_char_p, []),
        "mmdit_pack_plan": (_i32, [ctypes.POINTER(_Sample), _i32, _i64, _i64, ctypes.POINTER(_i32),
                                   ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.POINTER(_i32)]),
        "mmdit_pack": (_i32, [ctypes.POINTER(_Sample), _i32, P, _vp]),
        "mmdit_pack_gather": (_i32, [P, _i32, ctypes.POINTER(_vp), _i32, _i32, _vp, _vp]),
        "mmdit_workspace_size": (_sz, [D, P]),
        "mmdit_workspace_layout": (_i32, [D, P, ctypes.POINTER(_sz)]),
        "mmdit_cond": (_i32, [D, _vp, _vp, _vp, _i32, _vp, _vp, _sz, _vp]),
        "mmdit_modulation": (_i32, [D, _vp, _i32, _i32, _vp, _vp, _vp]),
        "mmdit_embed": (_i32, [D, _vp, _vp, P, _vp, _vp, _vp, _vp, _vp]),
        "mmdit_block_fwd": (_i32, [D, ctypes.POINTER(_BlockW), P, _vp, _vp, _vp, _vp, _sz, _vp]),
        "mmdit_block_modulation": (_i32, [D, ctypes.POINTER(_BlockW), _i32, _vp, _vp, _vp]),
        "mmdit_block_fwd_mod": (_i32, [D, ctypes.POINTER(_BlockW), P, _vp, _vp, _vp, _vp, _sz, _vp]),
        "mmdit_block_saved_size": (_sz, [D, P]),
        "rf_loss_grad": (_i32, [P, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
        "mmdit_wrap_bwd_workspace_size": (_sz, [D, P]),
        "mmdit_final_bwd": (_i32, [D, _vp, _vp, P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "mmdit_embed_bwd": (_i32, [D, P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "mmdit_cond_bwd_workspace_size": (_sz, [D, _i32]),
        "mmdit_cond_bwd": (_i32, [D, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
        "mmdit_block_fwd_train": (_i32, [D, ctypes.POINTER(_BlockW), P, _vp, _vp, _vp, _vp, _sz, _vp, _sz, _vp]),
        "mmdit_block_bwd_workspace_size": (_sz, [D, P]),
        "mmdit_block_bwd": (_i32, [D, ctypes.POINTER(_BlockW), P, _vp, _vp, _sz, _vp, _vp, ctypes.POINTER(_BlockG),
                                   _vp, _vp, _sz, _vp]),
        "mmdit_block_bwd2": (_i32, [D, ctypes.POINTER(_BlockW), P, _vp, _vp, _sz, _vp, _vp, ctypes.POINTER(_BlockG),
                                   _vp, _vp, _sz, _vp, _vp]),
        "mmdit_rms_modulate": (_i32, [D, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _vp]),
        "mmdit_qk_norm_rope": (_i32, [D, _i64, _vp, _vp, _vp, _vp, _vp]),
        "mmdit_attention": (_i32, [D, P, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "mmdit_attention_workspace_size": (_sz, [D, P]),
        "mmdit_linear": (_i32, [_i32, _i64, _i32, _i32, _vp, _vp, _vp, _i32, _vp, _i64, _vp, _i32, _vp]),
        "mmdit_final": (_i32, [D, _vp, _vp, P, _vp, _vp, _vp, _vp, _sz, _vp]),
        "mmdit_final_mod": (_i32, [D, _vp, P, _vp, _vp, _vp, _vp, _sz, _vp]),
        "rf_make_xt": (_i32, [P, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
        "rf_embed": (_i32, [D, _vp, _vp, P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
        "rf_final_loss": (_i32, [D, _vp, P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "rf_loss": (_i32, [P, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "rf_loss_noalloc": (_i32, [P, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
        "rf_nft_loss": (_i32, [P, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "rf_euler_step": (_i32, [P, _i32, _i32, _vp, _i32, _i32, _f32, _f32, _f32, _vp, _vp, _vp]),
        "rf_pack_latent": (_i32, [P, _i32, _i32, _vp, _i32, _i32, _vp, _vp]),
        "mmdit_timing_enable": (_i32, [_i32]),
        "mmdit_timing_report": (_i32, [_i32, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(_i64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _ck(status):
    if status != 0:
        raise MmditError(status, _lib.mmdit_last_error().decode())


def _stream(stream):
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t):
    import torch

    return BF16 if t.dtype == torch.bfloat16 else F32


class Dims:
    """Model widths + compute dtype ("bf16" or "f32")."""

    def __init__(self, d, dtype):
        self.d = d
        self.dtype = dtype
        self.c = _DimsT(d.hidden, d.heads, d.head_dim, d.mlp, d.c_lat, d.d_txt, d.t_dim,
                        (_i32 * 3)(*d.bands), d.rope_theta, d.eps, BF16 if dtype == "bf16" else F32)

    @property
    def torch_dtype(self):
        import torch

        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


class Pack:
    """A built pack: the ctypes struct plus the int32 device tensors it points to."""

    def __init__(self, samples, device):
        import torch

        self.samples = [tuple(int(v) for v in s) for s in samples]
        B = len(self.samples)
        n_img = sum(f * h * w for h, w, f, _ in self.samples)
        n_txt = sum(t for *_, t in self.samples)
        n_tgt = sum(h * w for h, w, _, _ in self.samples)
        z = dict(dtype=torch.int32, device=device)
        self.t = {
            "cu_txt": torch.zeros(B + 1, **z), "cu_img": torch.zeros(B + 1, **z),
            "cu_joint": torch.zeros(B + 1, **z), "cu_tgt": torch.zeros(B + 1, **z),
            "tgt_len": torch.zeros(max(B, 1), **z), "seg_img": torch.zeros(max(n_img, 1), **z),
            "seg_txt": torch.zeros(max(n_txt, 1), **z), "pos_img": torch.zeros(max(n_img, 1) * 3, **z),
            "tgt_row": torch.zeros(max(n_tgt, 1), **z),
        }
        self.c = _PackT()
        for k, v in self.t.items():
            setattr(self.c, k, v.data_ptr())
        self.ref = ctypes.byref(self.c)

    @property
    def B(self):
        return self.c.B

    @property
    def n_img(self):
        return self.c.n_img

    @property
    def n_txt(self):
        return self.c.n_txt

    @property
    def n_tgt(self):
        return self.c.n_tgt

    @property
    def max_joint(self):
        return self.c.max_joint

    def host(self, name):
        n = self.B + 1
        return list(getattr(self.c, name)[:n])


def _samples(samples):
    arr = (_Sample * max(len(samples), 1))()
    for i, s in enumerate(samples):
        arr[i] = _Sample(*[int(v) for v in s])
    return arr


def pack_plan(samples, img_budget, joint_budget=0):
    """Next-fit plan (host only): (n_taken, n_img, n_txt, max_joint)."""
    nt, ni, nx, mj = _i32(), _i64(), _i64(), _i32()
    _ck(_lib.mmdit_pack_plan(_samples(samples), len(samples), int(img_budget), int(joint_budget),
                             ctypes.byref(nt), ctypes.byref(ni), ctypes.byref(nx), ctypes.byref(mj)))
    return nt.value, ni.value, nx.value, mj.value


def pack(samples, device="cuda", stream=None):
    pk = Pack(samples, device)
    _ck(_lib.mmdit_pack(_samples(samples), len(samples), pk.ref, _stream(stream)))
    return pk


def pack_gather(pk, which, srcs, out, stream=None):
    """which: 0 image rows, 1 text rows, 2 target rows; srcs: per-sample tensors."""
    arr = (_vp * max(len(srcs), 1))(*[s.data_ptr() for s in srcs])
    _ck(_lib.mmdit_pack_gather(pk.ref, which, arr, out.shape[-1], _dt(out), _p(out), _stream(stream)))


def workspace_size(dims, pk):
    return int(_lib.mmdit_workspace_size(ctypes.byref(dims.c), pk.ref))


def workspace_layout(dims, pk):
    out = (_sz * 8)()
    n = _lib.mmdit_workspace_layout(ctypes.byref(dims.c), pk.ref, out)
    if n != 6:
        raise MmditError(-1, _lib.mmdit_last_error().decode())
    return dict(zip(("mod_img", "mod_txt", "h", "qkv", "o", "u"), list(out[:6])))


def cond(dims, w_t1, w_t2, t, c, ws, stream=None):
    _ck(_lib.mmdit_cond(ctypes.byref(dims.c), _p(w_t1), _p(w_t2), _p(t), t.numel(), _p(c), _p(ws),
                        ws.numel() * ws.element_size(), _stream(stream)))


def modulation(dims, w, chunks, c, mod, stream=None):
    _ck(_lib.mmdit_modulation(ctypes.byref(dims.c), _p(w), chunks, c.shape[0], _p(c), _p(mod),
                              _stream(stream)))


def embed(dims, w_in, w_txt, pk, zt, tau, x_img, x_txt, stream=None):
    _ck(_lib.mmdit_embed(ctypes.byref(dims.c), _p(w_in), _p(w_txt), pk.ref, _p(zt), _p(tau),
                         _p(x_img), _p(x_txt), _stream(stream)))


def _stream_w(w):
    return _StreamW(*[w[k].data_ptr() for k in ("w_mod", "w_qkv", "g_q", "g_k", "w_o", "w_up", "w_down")])


def block_weights(wb):
    """ctypes struct for {"img": {...}, "txt": {...}} dicts of device tensors (keep wb alive)."""
    return _BlockW(_stream_w(wb["img"]), _stream_w(wb["txt"]))


def block_fwd(dims, wb, pk, c, x_img, x_txt, ws, stream=None):
    bw = wb if isinstance(wb, _BlockW) else block_weights(wb)
    _ck(_lib.mmdit_block_fwd(ctypes.byref(dims.c), ctypes.byref(bw), pk.ref, _p(c), _p(x_img),
                             _p(x_txt), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def block_modulation(dims, wb, c, mod, stream=None):
    """Both streams' adaLN vectors of a block into mod (float32 [2, B, 6H])."""
    bw = wb if isinstance(wb, _BlockW) else block_weights(wb)
    _ck(_lib.mmdit_block_modulation(ctypes.byref(dims.c), ctypes.byref(bw), c.shape[0], _p(c), _p(mod),
                                    _stream(stream)))


def block_fwd_mod(dims, wb, pk, mod, x_img, x_txt, ws, stream=None):
    """block_fwd with the adaLN vectors from block_modulation."""
    bw = wb if isinstance(wb, _BlockW) else block_weights(wb)
    _ck(_lib.mmdit_block_fwd_mod(ctypes.byref(dims.c), ctypes.byref(bw), pk.ref, _p(mod), _p(x_img),
                                 _p(x_txt), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def block_saved_size(dims, pk):
    return int(_lib.mmdit_block_saved_size(ctypes.byref(dims.c), pk.ref))


def block_bwd_workspace_size(dims, pk):
    return int(_lib.mmdit_block_bwd_workspace_size(ctypes.byref(dims.c), pk.ref))


def block_fwd_train(dims, wb, pk, c, x_img, x_txt, saved, ws, stream=None):
    bw = wb if isinstance(wb, _BlockW) else block_weights(wb)
    _ck(_lib.mmdit_block_fwd_train(ctypes.byref(dims.c), ctypes.byref(bw), pk.ref, _p(c), _p(x_img), _p(x_txt),
                                   _p(saved), saved.numel() * saved.element_size(), _p(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)))


def block_grads(g):
    """ctypes struct for {"img": {...}, "txt": {...}} dicts of float32 gradient tensors (keep g alive)."""
    return _BlockG(*[_StreamG(*[g[s][k].data_ptr() for k in GRAD_KEYS]) for s in ("img", "txt")])


def block_bwd(dims, wb, pk, c, saved, dx_img, dx_txt, grads, dc, ws, stream=None, stream_w=None):
    """dx_img, dx_txt: dL/dx_out in, dL/dx_in out; grads overwritten; dc accumulated.
    stream_w: run the weight gradients on this second stream (mmdit_block_bwd2)."""
    bw = wb if isinstance(wb, _BlockW) else block_weights(wb)
    bg = grads if isinstance(grads, _BlockG) else block_grads(grads)
    if stream_w is None:
        _ck(_lib.mmdit_block_bwd(ctypes.byref(dims.c), ctypes.byref(bw), pk.ref, _p(c), _p(saved),
                                 saved.numel() * saved.element_size(), _p(dx_img), _p(dx_txt), ctypes.byref(bg),
                                 _p(dc), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))
    else:
        _ck(_lib.mmdit_block_bwd2(ctypes.byref(dims.c), ctypes.byref(bw), pk.ref, _p(c), _p(saved),
                                  saved.numel() * saved.element_size(), _p(dx_img), _p(dx_txt), ctypes.byref(bg),
                                  _p(dc), _p(ws), ws.numel() * ws.element_size(), _stream(stream),
                                  _stream(stream_w)))


def rf_loss_grad(pk, v, z, eps, dv, stream=None):
    _ck(_lib.rf_loss_grad(pk.ref, _dt(v), v.shape[-1], _p(v), _p(z), _p(eps), _p(dv), _stream(stream)))


def wrap_bwd_workspace_size(dims, pk):
    return int(_lib.mmdit_wrap_bwd_workspace_size(ctypes.byref(dims.c), pk.ref))


def final_bwd(dims, w_fmod, w_out, pk, c, x_img, dv, dx_img, dw_fmod, dw_out, dc, ws, stream=None):
    _ck(_lib.mmdit_final_bwd(ctypes.byref(dims.c), _p(w_fmod), _p(w_out), pk.ref, _p(c), _p(x_img), _p(dv),
                             _p(dx_img), _p(dw_fmod), _p(dw_out), _p(dc), _p(ws), ws.numel() * ws.element_size(),
                             _stream(stream)))


def embed_bwd(dims, pk, zt, tau, dx_img, dx_txt, dw_in, dw_txt, ws, stream=None):
    _ck(_lib.mmdit_embed_bwd(ctypes.byref(dims.c), pk.ref, _p(zt), _p(tau), _p(dx_img), _p(dx_txt), _p(dw_in),
                             _p(dw_txt), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def cond_bwd_workspace_size(dims, B):
    return int(_lib.mmdit_cond_bwd_workspace_size(ctypes.byref(dims.c), B))


def cond_bwd(dims, w_t1, w_t2, t, dc, dw_t1, dw_t2, ws, stream=None):
    _ck(_lib.mmdit_cond_bwd(ctypes.byref(dims.c), _p(w_t1), _p(w_t2), _p(t), t.numel(), _p(dc), _p(dw_t1),
                            _p(dw_t2), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def rms_modulate(dims, x, seg, mod, shift_off, scale_off, y, row_map=None, stream=None):
    n = y.shape[0]
    _ck(_lib.mmdit_rms_modulate(ctypes.byref(dims.c), n, _p(x), _p(row_map), _p(seg), _p(mod),
                                mod.shape[-1], shift_off, scale_off, _p(y), _stream(stream)))


def qk_norm_rope(dims, qkv, pos, g_q, g_k, stream=None):
    _ck(_lib.mmdit_qk_norm_rope(ctypes.byref(dims.c), qkv.shape[0], _p(qkv), _p(pos), _p(g_q),
                                _p(g_k), _stream(stream)))


def attention(dims, pk, qkv_img, qkv_txt, o_img, o_txt, ws=None, stream=None):
    """Joint attention; allocates the V^T staging buffer when ws is not given."""
    if ws is None:
        import torch

        n = int(_lib.mmdit_attention_workspace_size(ctypes.byref(dims.c), pk.ref))
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=qkv_img.device)
    _ck(_lib.mmdit_attention(ctypes.byref(dims.c), pk.ref, _p(qkv_img), _p(qkv_txt), _p(o_img),
                             _p(o_txt), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def linear(A, W, Y, epilogue=EPI_STORE, gate=None, gate_stride=0, seg=None, a_silu=False, stream=None):
    M, K = A.shape
    N = W.shape[0]
    _ck(_lib.mmdit_linear(_dt(A), M, N, K, _p(A), _p(W), _p(Y), epilogue, _p(gate), gate_stride,
                          _p(seg), 1 if a_silu else 0, _stream(stream)))


def final(dims, w_fmod, w_out, pk, c, x_img, v, ws, stream=None):
    _ck(_lib.mmdit_final(ctypes.byref(dims.c), _p(w_fmod), _p(w_out), pk.ref, _p(c), _p(x_img), _p(v),
                         _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def final_mod(dims, w_out, pk, modf, x_img, v, ws, stream=None):
    """final with its adaLN vectors from modulation(w_fmod, 2, c)."""
    _ck(_lib.mmdit_final_mod(ctypes.byref(dims.c), _p(w_out), pk.ref, _p(modf), _p(x_img), _p(v),
                             _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def rf_embed(dims, w_in, w_txt, pk, z, eps, t, tau, x_img, x_txt, zt, stream=None):
    _ck(_lib.rf_embed(ctypes.byref(dims.c), _p(w_in), _p(w_txt), pk.ref, _p(z), _p(eps), _p(t), _p(tau),
                      _p(x_img), _p(x_txt), _p(zt), _stream(stream)))


def rf_final_loss(dims, w_out, pk, modf, x_img, z, eps, v, sse, loss, ws, stream=None):
    _ck(_lib.rf_final_loss(ctypes.byref(dims.c), _p(w_out), pk.ref, _p(modf), _p(x_img), _p(z), _p(eps), _p(v),
                           _p(sse), _p(loss), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def rf_make_xt(pk, z, eps, t, zt, stream=None):
    _ck(_lib.rf_make_xt(pk.ref, _dt(z), z.shape[-1], _p(z), _p(eps), _p(t), _p(zt), _stream(stream)))


def rf_loss(pk, v, z, eps, sse, loss, ws, stream=None):
    _ck(_lib.rf_loss(pk.ref, _dt(v), v.shape[-1], _p(v), _p(z), _p(eps), _p(sse), _p(loss), _p(ws),
                     ws.numel() * ws.element_size(), _stream(stream)))


def rf_loss_noalloc(pk, v, z, eps, sse, loss, stream=None):
    _ck(_lib.rf_loss_noalloc(pk.ref, _dt(v), v.shape[-1], _p(v), _p(z), _p(eps), _p(sse), _p(loss),
                             _stream(stream)))


def rf_nft_loss(pk, v_pos, v_neg, z, eps, r, sse, loss, ws, stream=None):
    _ck(_lib.rf_nft_loss(pk.ref, _dt(v_pos), v_pos.shape[-1], _p(v_pos), _p(v_neg), _p(z), _p(eps), _p(r),
                         _p(sse), _p(loss), _p(ws), ws.numel() * ws.element_size(), _stream(stream)))


def rf_euler_step(pk, v, cond_b, uncond_b, guidance, t_cur, t_next, z, zt_next=None, stream=None):
    _ck(_lib.rf_euler_step(pk.ref, _dt(v), v.shape[-1], _p(v), cond_b, uncond_b, guidance, t_cur,
                           t_next, _p(z), _p(zt_next), _stream(stream)))


def rf_pack_latent(pk, z, b0, b1, zt, stream=None):
    _ck(_lib.rf_pack_latent(pk.ref, _dt(zt), z.shape[-1], _p(z), b0, b1, _p(zt), _stream(stream)))


def timing_enable(on=True):
    _ck(_lib.mmdit_timing_enable(1 if on else 0))


def timing_report(max_entries=128):
    """{kernel name: (total ms, launches)} since timing_enable(True); syncs the device."""
    names = ctypes.create_string_buffer(64 * max_entries)
    ms = (ctypes.c_double * max_entries)()
    cnt = (_i64 * max_entries)()
    n = _lib.mmdit_timing_report(max_entries, names, ms, cnt)
    if n < 0:
        raise MmditError(-5, _lib.mmdit_last_error().decode())
    raw = names.raw
    out = {}
    for i in range(n):
        nm = raw[64 * i:64 * (i + 1)].split(b"\0", 1)[0].decode()
        out[nm] = (ms[i], cnt[i])
    return out


def version():
    return _lib.mmdit_version().decode()
