"""ctypes binding of libvt.so: argument marshalling only.

Every function here has the name of the C entry point it calls and passes
torch tensors as raw device pointers, the current HIP stream as the stream.
All computation happens in the HIP kernels of the library; there is no
fallback: if ``libvt.so`` is missing the import raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvt.so")

VT_OK, VT_ERR_INVALID_ARG, VT_ERR_UNSUPPORTED, VT_ERR_WORKSPACE, VT_ERR_HIP = range(5)
VT_BF16, VT_FP32 = 0, 1
VT_ORDER_WINDOW, VT_ORDER_RASTER = 0, 1
VT_EPI_BF16, VT_EPI_GELU_TANH_BF16, VT_EPI_GELU_ERF_BF16, VT_EPI_RESID_F32, VT_EPI_F32 = range(5)
VT_EPI_SPLITK_PARTIALS_F32 = 5
VT_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

EXPORTED = ("vt_config_default", "vt_status_string", "vt_last_error", "vt_version",
            "vt_tower_workspace_size", "vt_block_workspace_size", "vt_build_metadata",
            "vt_patch_embed", "vt_attention_varlen", "vt_block_forward", "vt_merge_project",
            "vt_tower_forward", "vt_plan_patches", "vt_pack_items", "vt_mean_pool",
            "vt_linear_workspace_size", "vt_linear", "vt_layer_norm", "vt_attention_backward",
            "vt_attention_backward_workspace_size", "vt_block_backward",
            "vt_block_backward_workspace_size", "vt_tower_backward",
            "vt_tower_backward_workspace_size", "vt_clock_probe", "vt_attention_varlen_noalloc",
            "vt_linear_residual_ln", "vt_attention_pack", "vt_attention_packed")


class VtError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


class vt_grid_thw(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32)]


class vt_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("layers", "hidden", "heads", "head_dim", "mlp",
                                              "patch", "t_patch", "merge", "proj_hidden",
                                              "proj_out")] + [
        ("ln_eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
        ("rope_pairs", ctypes.c_int32 * 3), ("rope_shared_ladder", ctypes.c_int32),
        ("gelu_erf_projector", ctypes.c_int32)]


_P = ctypes.c_void_p


class vt_block_weights(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g",
                                  "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2")]


class vt_block_grads(ctypes.Structure):
    _fields_ = list(vt_block_weights._fields_)


class vt_tower_grads(ctypes.Structure):
    _fields_ = [("w_patch", _P), ("b_patch", _P), ("blocks", ctypes.POINTER(vt_block_grads))]


class vt_projector_weights(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("w1", "b1", "w2", "b2", "w3", "b3", "w4", "b4")]


class vt_tower_weights(ctypes.Structure):
    _fields_ = [("w_patch", _P), ("b_patch", _P), ("blocks", ctypes.POINTER(vt_block_weights)),
                ("proj", vt_projector_weights)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m vision_transformer_encoder_tiled_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    C, I32, SZ = ctypes.c_char_p, ctypes.c_int32, ctypes.c_size_t
    cfgp, gridp = ctypes.POINTER(vt_config), ctypes.POINTER(vt_grid_thw)
    sig = {
        "vt_config_default": (None, [cfgp]),
        "vt_status_string": (C, [ctypes.c_int]),
        "vt_last_error": (C, []),
        "vt_version": (C, []),
        "vt_tower_workspace_size": (SZ, [cfgp, gridp, I32]),
        "vt_block_workspace_size": (SZ, [cfgp, I32, I32, I32]),
        "vt_build_metadata": (ctypes.c_int, [gridp, I32, _P, _P, _P, _P]),
        "vt_patch_embed": (ctypes.c_int, [cfgp, _P, gridp, I32, _P, _P, _P, _P, SZ, _P]),
        "vt_attention_varlen": (ctypes.c_int, [cfgp, _P, _P, _P, I32, I32, I32, _P, ctypes.c_int,
                                               _P, SZ, _P]),
        "vt_attention_varlen_noalloc": (ctypes.c_int, [cfgp, _P, _P, _P, I32, I32, I32, _P, ctypes.c_int,
                                                       _P]),
        "vt_attention_pack": (ctypes.c_int, [cfgp, _P, _P, _P, I32, I32, I32, _P, SZ, _P]),
        "vt_attention_packed": (ctypes.c_int, [cfgp, I32, I32, I32, _P, _P, ctypes.c_int, _P, SZ, _P]),
        "vt_attention_backward": (ctypes.c_int, [cfgp, _P, _P, _P, I32, I32, I32, _P, _P,
                                                 ctypes.c_int, _P, SZ, _P]),
        "vt_attention_backward_workspace_size": (SZ, [cfgp, I32, I32, I32]),
        "vt_block_backward": (ctypes.c_int, [cfgp, _P, ctypes.POINTER(vt_block_weights), _P, _P, I32,
                                             I32, I32, _P, ctypes.POINTER(vt_block_grads), _P, SZ, _P]),
        "vt_block_backward_workspace_size": (SZ, [cfgp, I32, I32, I32]),
        "vt_block_forward": (ctypes.c_int, [cfgp, _P, ctypes.POINTER(vt_block_weights), _P, _P,
                                            I32, I32, I32, _P, SZ, _P]),
        "vt_merge_project": (ctypes.c_int, [cfgp, _P, ctypes.c_int, gridp, I32,
                                            ctypes.POINTER(vt_projector_weights), _P, _P, _P, SZ,
                                            _P]),
        "vt_tower_forward": (ctypes.c_int, [cfgp, _P, gridp, I32, ctypes.POINTER(vt_tower_weights),
                                            _P, _P, _P, _P, SZ, _P]),
        "vt_tower_backward": (ctypes.c_int, [cfgp, _P, gridp, I32, ctypes.POINTER(vt_tower_weights), _P,
                                             ctypes.POINTER(vt_tower_grads), _P, SZ, _P]),
        "vt_tower_backward_workspace_size": (SZ, [cfgp, gridp, I32]),
        "vt_linear_workspace_size": (SZ, [I32, I32, I32]),
        "vt_linear": (ctypes.c_int, [_P, I32, I32, _P, I32, _P, ctypes.c_int, _P, _P, SZ, _P]),
        "vt_layer_norm": (ctypes.c_int, [_P, I32, I32, _P, _P, ctypes.c_float, _P, _P]),
        "vt_linear_residual_ln": (ctypes.c_int, [_P, I32, I32, _P, I32, _P, _P, _P, _P, ctypes.c_float, _P,
                                                 _P, SZ, _P]),
        "vt_mean_pool": (ctypes.c_int, [_P, _P, I32, I32, _P, _P]),
        "vt_plan_patches": (ctypes.c_int, [_P, ctypes.c_size_t, I32, ctypes.c_int64, _P, _P]),
        "vt_pack_items": (ctypes.c_int, [_P, _P, I32, ctypes.c_size_t, _P, _P]),
        "vt_clock_probe": (ctypes.c_int, [ctypes.c_int64, _P, ctypes.POINTER(ctypes.c_int64), _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def _status_name(s):
    return LIB.vt_status_string(int(s)).decode()


def last_error() -> str:
    return LIB.vt_last_error().decode()


def _check(status):
    if status != VT_OK:
        raise VtError(status, last_error())


# ------------------------------------------------------------------ marshalling helpers
def _ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _grid(grids):
    arr = (vt_grid_thw * len(grids))()
    for i, (t, h, w) in enumerate(grids):
        arr[i].t, arr[i].h, arr[i].w = int(t), int(h), int(w)
    return arr, len(grids)


def config(**overrides) -> vt_config:
    c = vt_config()
    LIB.vt_config_default(ctypes.byref(c))
    for k, v in overrides.items():
        if k == "rope_pairs":
            for i in range(3):
                c.rope_pairs[i] = int(v[i])
        else:
            setattr(c, k, v)
    return c


def vt_config_default() -> vt_config:
    return config()


def vt_version() -> str:
    return LIB.vt_version().decode()


def vt_tower_workspace_size(cfg, grids) -> int:
    g, n = _grid(grids)
    return int(LIB.vt_tower_workspace_size(ctypes.byref(cfg), g, n))


def vt_block_workspace_size(cfg, total_tokens, n_img, max_seqlen) -> int:
    return int(LIB.vt_block_workspace_size(ctypes.byref(cfg), total_tokens, n_img, max_seqlen))


def vt_linear_workspace_size(M, N, K) -> int:
    return int(LIB.vt_linear_workspace_size(M, N, K))


def vt_build_metadata(grids, cu_seqlens, pos_thw, raster_index=None, stream=None):
    g, n = _grid(grids)
    _check(LIB.vt_build_metadata(g, n, _ptr(cu_seqlens), _ptr(pos_thw), _ptr(raster_index),
                                 _stream(stream)))


def vt_patch_embed(cfg, pixels, grids, w_patch, b_patch, resid_out, ws, stream=None):
    g, n = _grid(grids)
    _check(LIB.vt_patch_embed(ctypes.byref(cfg), _ptr(pixels), g, n, _ptr(w_patch), _ptr(b_patch),
                              _ptr(resid_out), _ptr(ws), ws.numel() if ws is not None else 0,
                              _stream(stream)))


def vt_attention_varlen(cfg, qkv, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen, out,
                        out_dtype, ws, stream=None):
    _check(LIB.vt_attention_varlen(ctypes.byref(cfg), _ptr(qkv), _ptr(cu_seqlens), _ptr(pos_thw),
                                   n_img, total_tokens, max_seqlen, _ptr(out), out_dtype, _ptr(ws),
                                   ws.numel() if ws is not None else 0, _stream(stream)))


def vt_attention_pack(cfg, qkv, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen, ws, stream=None):
    _check(LIB.vt_attention_pack(ctypes.byref(cfg), _ptr(qkv), _ptr(cu_seqlens), _ptr(pos_thw), n_img,
                                 total_tokens, max_seqlen, _ptr(ws), ws.numel() if ws is not None else 0,
                                 _stream(stream)))


def vt_attention_packed(cfg, n_img, total_tokens, max_seqlen, out, out_dtype, ws, stream=None, host_seqlens=None):
    """host_seqlens: optional list of the images' token counts (a host-side hint)."""
    hs = None
    if host_seqlens is not None:
        hs = (ctypes.c_int32 * len(host_seqlens))(*[int(v) for v in host_seqlens])
    _check(LIB.vt_attention_packed(ctypes.byref(cfg), n_img, total_tokens, max_seqlen, hs, _ptr(out), out_dtype,
                                   _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def vt_attention_varlen_noalloc(cfg, qkv, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen, out,
                                out_dtype, stream=None):
    _check(LIB.vt_attention_varlen_noalloc(ctypes.byref(cfg), _ptr(qkv), _ptr(cu_seqlens), _ptr(pos_thw),
                                           n_img, total_tokens, max_seqlen, _ptr(out), out_dtype,
                                           _stream(stream)))


def vt_attention_backward_workspace_size(cfg, total_tokens, n_img, max_seqlen) -> int:
    return int(LIB.vt_attention_backward_workspace_size(ctypes.byref(cfg), total_tokens, n_img,
                                                        max_seqlen))


def vt_attention_backward(cfg, qkv, cu_seqlens, pos_thw, n_img, total_tokens, max_seqlen, dout,
                          dqkv, dqkv_dtype, ws, stream=None):
    _check(LIB.vt_attention_backward(ctypes.byref(cfg), _ptr(qkv), _ptr(cu_seqlens), _ptr(pos_thw),
                                     n_img, total_tokens, max_seqlen, _ptr(dout), _ptr(dqkv),
                                     dqkv_dtype, _ptr(ws), ws.numel() if ws is not None else 0,
                                     _stream(stream)))


def block_grads(g: dict) -> vt_block_grads:
    """vt_block_grads from a dict of fp32 device tensors keyed like the weights
    (missing entries -> NULL, not formed)."""
    b = vt_block_grads()
    keep = []
    for name, _ in vt_block_grads._fields_:
        t = g.get(name)
        setattr(b, name, None if t is None else t.data_ptr())
        keep.append(t)
    b._tensors = keep
    return b


def vt_block_backward_workspace_size(cfg, total_tokens, n_img, max_seqlen) -> int:
    return int(LIB.vt_block_backward_workspace_size(ctypes.byref(cfg), total_tokens, n_img, max_seqlen))


def vt_block_backward(cfg, resid_in, bw: vt_block_weights, cu_seqlens, pos_thw, n_img, total_tokens,
                      max_seqlen, dresid, grads: vt_block_grads, ws, stream=None):
    _check(LIB.vt_block_backward(ctypes.byref(cfg), _ptr(resid_in), ctypes.byref(bw), _ptr(cu_seqlens),
                                 _ptr(pos_thw), n_img, total_tokens, max_seqlen, _ptr(dresid),
                                 ctypes.byref(grads), _ptr(ws), ws.numel() if ws is not None else 0,
                                 _stream(stream)))


def block_weights(w: dict, prefix: str = "") -> vt_block_weights:
    """vt_block_weights from a dict of device tensors (missing biases -> NULL).
    The struct keeps references to the tensors it points to."""
    b = vt_block_weights()
    keep = []
    for name, _ in vt_block_weights._fields_:
        t = w.get(prefix + name)
        setattr(b, name, None if t is None else t.data_ptr())
        keep.append(t)
    b._tensors = keep
    return b


def projector_weights(w: dict) -> vt_projector_weights:
    p = vt_projector_weights()
    keep = []
    for name, _ in vt_projector_weights._fields_:
        t = w.get("p_" + name)
        setattr(p, name, None if t is None else t.data_ptr())
        keep.append(t)
    p._tensors = keep
    return p


def vt_block_forward(cfg, resid, bw: vt_block_weights, cu_seqlens, pos_thw, n_img, total_tokens,
                     max_seqlen, ws, stream=None):
    _check(LIB.vt_block_forward(ctypes.byref(cfg), _ptr(resid), ctypes.byref(bw), _ptr(cu_seqlens),
                                _ptr(pos_thw), n_img, total_tokens, max_seqlen, _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream(stream)))


def vt_merge_project(cfg, tower, order, grids, pw: vt_projector_weights, merged_raw, out, ws,
                     stream=None):
    g, n = _grid(grids)
    _check(LIB.vt_merge_project(ctypes.byref(cfg), _ptr(tower), order, g, n,
                                ctypes.byref(pw) if pw is not None else None, _ptr(merged_raw),
                                _ptr(out), _ptr(ws), ws.numel() if ws is not None else 0,
                                _stream(stream)))


class TowerWeights:
    """Keeps the ctypes structs of a tower weight set alive (device tensors in ``w``)."""

    def __init__(self, w: dict, n_layers: int):
        self.w = w
        self.blocks = (vt_block_weights * max(1, n_layers))()
        for i in range(n_layers):
            self.blocks[i] = block_weights(w, f"l{i}.")
        self.struct = vt_tower_weights()
        self.struct.w_patch = w["patch_w"].data_ptr()
        bp = w.get("patch_b")
        self.struct.b_patch = None if bp is None else bp.data_ptr()
        self.struct.blocks = ctypes.cast(self.blocks, ctypes.POINTER(vt_block_weights))
        if "p_w1" in w:
            self.struct.proj = projector_weights(w)


def vt_tower_forward(cfg, pixels, grids, tw: TowerWeights, tower_out, merged_raw, out, ws,
                     stream=None):
    g, n = _grid(grids)
    _check(LIB.vt_tower_forward(ctypes.byref(cfg), _ptr(pixels), g, n, ctypes.byref(tw.struct),
                                _ptr(tower_out), _ptr(merged_raw), _ptr(out), _ptr(ws),
                                ws.numel() if ws is not None else 0, _stream(stream)))


class TowerGrads:
    """Keeps the ctypes structs of a tower gradient set alive: ``g`` maps
    "patch_w", "patch_b" and "l<i>.<name>" to fp32 device tensors (missing
    entries are not formed)."""

    def __init__(self, g: dict, n_layers: int):
        self.g = g
        self.blocks = (vt_block_grads * max(1, n_layers))()
        for i in range(n_layers):
            p = f"l{i}."
            self.blocks[i] = block_grads({k[len(p):]: v for k, v in g.items() if k.startswith(p)})
        self.struct = vt_tower_grads()
        for name in ("w_patch", "b_patch"):
            t = g.get("patch_" + name[0])
            setattr(self.struct, name, None if t is None else t.data_ptr())
        self.struct.blocks = ctypes.cast(self.blocks, ctypes.POINTER(vt_block_grads))


def vt_tower_backward_workspace_size(cfg, grids) -> int:
    g, n = _grid(grids)
    return int(LIB.vt_tower_backward_workspace_size(ctypes.byref(cfg), g, n))


def vt_tower_backward(cfg, pixels, grids, tw: TowerWeights, d_tower, tg: TowerGrads, ws, stream=None):
    g, n = _grid(grids)
    _check(LIB.vt_tower_backward(ctypes.byref(cfg), _ptr(pixels), g, n, ctypes.byref(tw.struct),
                                 _ptr(d_tower), ctypes.byref(tg.struct), _ptr(ws),
                                 ws.numel() if ws is not None else 0, _stream(stream)))


def vt_linear(x, M, K, w, N, bias, epi, out, ws=None, stream=None):
    _check(LIB.vt_linear(_ptr(x), M, K, _ptr(w), N, _ptr(bias), epi, _ptr(out), _ptr(ws),
                         ws.numel() if ws is not None else 0, _stream(stream)))


def vt_linear_residual_ln(x, M, K, w, N, bias, R, g, beta, eps, out, ws=None, stream=None):
    _check(LIB.vt_linear_residual_ln(_ptr(x), M, K, _ptr(w), N, _ptr(bias), _ptr(R), _ptr(g), _ptr(beta),
                                     ctypes.c_float(eps), _ptr(out), _ptr(ws),
                                     ws.numel() if ws is not None else 0, _stream(stream)))


def vt_plan_patches(cfg, budget_bytes, n_img=1, max_pixels=0):
    """(patches, wanted): see include/vt.h."""
    p, w = ctypes.c_int64(), ctypes.c_int64()
    _check(LIB.vt_plan_patches(ctypes.byref(cfg), int(budget_bytes), n_img, int(max_pixels),
                               ctypes.byref(p), ctypes.byref(w)))
    return p.value, w.value


def vt_pack_items(cfg, grids, budget_bytes):
    """Call index of each item, greedy in list order (see include/vt.h)."""
    g, n = _grid(grids)
    batch = (ctypes.c_int32 * n)()
    nb = ctypes.c_int32()
    _check(LIB.vt_pack_items(ctypes.byref(cfg), g, n, int(budget_bytes), batch, ctypes.byref(nb)))
    return list(batch), nb.value


def vt_mean_pool(tower, cu_seqlens, n_img, hidden, out, stream=None):
    _check(LIB.vt_mean_pool(_ptr(tower), _ptr(cu_seqlens), n_img, hidden, _ptr(out), _stream(stream)))


def vt_clock_probe(wait_us, out, stream=None) -> int:
    """Enqueue the core-clock probe on ``stream`` (out: 4 int64 on the device);
    returns the real-time counter rate in Hz.  The core clock is
    (out[1] - out[0]) / (out[3] - out[2]) * rate once the probe has ended."""
    hz = ctypes.c_int64(0)
    _check(LIB.vt_clock_probe(int(wait_us), _ptr(out), ctypes.byref(hz), _stream(stream)))
    return hz.value


def vt_layer_norm(x, rows, width, g, b, eps, out, stream=None):
    _check(LIB.vt_layer_norm(_ptr(x), rows, width, _ptr(g), _ptr(b), float(eps), _ptr(out),
                             _stream(stream)))


# ------------------------------------------------------------------ device helpers
def to_device_bits(a: np.ndarray, device="cuda"):
    """Upload uint16 bf16 bits as an int16 tensor (same bytes)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


def bits_to_numpy(t) -> np.ndarray:
    """Download an int16/bf16 tensor holding bf16 bits as uint16."""
    import torch
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint16)


def workspace(nbytes: int, device="cuda"):
    """A 256-byte aligned uint8 workspace tensor (torch's allocator aligns to 512 B)."""
    import torch
    t = torch.empty(max(1, int(nbytes)), dtype=torch.uint8, device=device)
    assert t.data_ptr() % 256 == 0
    return t
