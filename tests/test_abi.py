"""Host-side checks of the C-ABI library: it loads, exports every declared
symbol, sizes its workspace linearly in the token count, and rejects invalid
arguments before launching anything.  No GPU needed: every call here fails
validation (or only computes sizes), so no HIP work is enqueued."""
import ctypes
import os
import re

import pytest
import torch

import vision_transformer_encoder_tiled_amd as vt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vt.h")

# Fake but aligned device addresses: validation must reject the call before
# any of them is dereferenced.  Used only where no GPU is present, so that a
# validation bug cannot turn into a device access.
needs_no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                                  reason="fake-pointer validation tests run on hosts without a GPU")
FAKE = 0x100000


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vt_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    declared = header_functions()
    assert len(declared) == 29
    assert sorted(vt.EXPORTED) == declared
    lib = ctypes.CDLL(vt.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert vt.vt_version().startswith("vt ")


def header_signatures():
    """{name: (return type, parameter count)} of every declaration in vt.h."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for ret, name, params in re.findall(
            r"\b(vt_status|size_t|void|const char\*|int32_t|int)\s+(vt_[a-z_0-9]+)\s*\(([^;]*?)\)\s*;", src, flags=re.S):
        p = params.strip()
        out[name] = (ret, 0 if p in ("", "void") else p.count(",") + 1)
    return out


def test_binding_signatures_match_the_header():
    """Every ctypes prototype of the binding has the parameter count and
    return type the header declares (a binding that passed one argument too
    few or too many would shift every argument after it)."""
    sigs = header_signatures()
    assert sorted(sigs) == header_functions()
    ret_types = {"vt_status": ctypes.c_int, "size_t": ctypes.c_size_t, "const char*": ctypes.c_char_p,
                 "void": None, "int32_t": ctypes.c_int32, "int": ctypes.c_int}
    for name, (ret, n) in sigs.items():
        fn = getattr(vt.LIB, name)
        assert fn.argtypes is not None and len(fn.argtypes) == n, (name, n, fn.argtypes)
        assert fn.restype == ret_types[ret], (name, ret, fn.restype)


def test_default_config_is_the_minimax_m3_shape():
    c = vt.vt_config_default()
    assert (c.layers, c.hidden, c.heads, c.head_dim, c.mlp) == (32, 1280, 16, 80, 5120)
    assert (c.patch, c.t_patch, c.merge, c.proj_hidden, c.proj_out) == (14, 2, 2, 6144, 6144)
    assert list(c.rope_pairs) == [8, 16, 16]
    assert c.ln_eps == pytest.approx(1e-6) and c.rope_theta == 10000.0


def test_workspace_is_affine_in_tokens():
    cfg = vt.config()
    # large square images: affine in the tokens, up to the GEMM partial-sum
    # area (at most 64 MiB: 256 tiles of 256 x 256 fp32), which a call has or
    # has not depending on how its tiles fill the CUs' rounds
    sizes = [vt.vt_tower_workspace_size(cfg, [(1, 64, 64)] * k) for k in (8, 16, 24, 32)]
    d1 = sizes[1] - sizes[0]
    part = 256 * 256 * 256 * 4
    # (a second difference can see the area appear in one step and go in the next)
    assert abs((sizes[2] - sizes[1]) - d1) <= 2 * part + 4096
    assert abs((sizes[3] - sizes[2]) - d1) <= 2 * part + 4096
    per_token = (sizes[3] - sizes[0]) / (24 * 64 * 64)
    assert per_token < 64 * 1024          # tens of KB per token ...
    # ... so a 2016x2016 image (20,736 patches) needs well under a GB of scratch,
    # against ~13.8 GB for one layer's untiled fp16 [16, n, n] score tensor.
    ws2016 = vt.vt_tower_workspace_size(cfg, [(1, 144, 144)])
    assert ws2016 < 1.5e9
    assert 16 * 20736 ** 2 * 2 > 13.7e9
    blk = [vt.vt_block_workspace_size(cfg, n, 1, n) for n in (4096, 8192, 16384)]
    assert abs((blk[2] - blk[1]) - 2 * (blk[1] - blk[0])) <= part + 4096


def test_workspace_size_reports_invalid_grids():
    cfg = vt.config()
    assert vt.vt_tower_workspace_size(cfg, [(1, 3, 4)]) == 0
    assert "even" in vt.last_error()
    assert vt.vt_tower_workspace_size(cfg, [(0, 4, 4)]) == 0
    assert "positive" in vt.last_error()
    # a clip of t temporal patches is sized like any item of t*h*w tokens, up to
    # the RoPE table (40 (cos, sin) pairs per position, positions < max(t, h, w))
    a = vt.vt_tower_workspace_size(cfg, [(4, 8, 8)])
    b = vt.vt_tower_workspace_size(cfg, [(1, 16, 16)])
    assert a > 0 and abs(a - b) <= 40 * 8 * 16
    bad = vt.config(head_dim=64, hidden=1024, rope_pairs=(0, 16, 16))
    assert vt.vt_tower_workspace_size(bad, [(1, 4, 4)]) == 0
    assert "head_dim 80" in vt.last_error()


def _call_metadata(grids):
    g, n = vt._lib._grid(grids)
    return vt.LIB.vt_build_metadata(g, n, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None, None)


@needs_no_gpu
def test_metadata_rejects_bad_grids_before_launch():
    assert _call_metadata([(1, 3, 4)]) == vt.VT_ERR_INVALID_ARG
    assert _call_metadata([(1, 4, 0)]) == vt.VT_ERR_INVALID_ARG
    assert _call_metadata([(-1, 4, 4)]) == vt.VT_ERR_INVALID_ARG
    g, _ = vt._lib._grid([(1, 4, 4)])
    assert vt.LIB.vt_build_metadata(g, 0, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None,
                                    None) == vt.VT_ERR_INVALID_ARG
    assert vt.LIB.vt_build_metadata(g, 1, None, ctypes.c_void_p(FAKE), None,
                                    None) == vt.VT_ERR_INVALID_ARG


def _attn(cfg, qkv=FAKE, out=FAKE, n_img=1, total=64, max_seq=64, ws=FAKE, ws_bytes=None,
          dtype=vt.VT_BF16):
    if ws_bytes is None:
        ws_bytes = vt.vt_block_workspace_size(cfg, total, n_img, max_seq)
    P = lambda v: None if v is None else ctypes.c_void_p(v)
    return vt.LIB.vt_attention_varlen(ctypes.byref(cfg), P(qkv), P(FAKE), P(FAKE), n_img, total,
                                      max_seq, P(out), dtype, P(ws), ws_bytes, None)


@needs_no_gpu
def test_attention_validation():
    cfg = vt.config()
    need = vt.vt_block_workspace_size(cfg, 64, 1, 64)
    assert need > 0
    assert _attn(cfg, ws_bytes=need - 1) == vt.VT_ERR_WORKSPACE
    assert "too small" in vt.last_error()
    assert _attn(cfg, qkv=None) == vt.VT_ERR_INVALID_ARG
    assert _attn(cfg, qkv=FAKE + 8) == vt.VT_ERR_INVALID_ARG          # misaligned
    assert "aligned" in vt.last_error()
    assert _attn(cfg, ws=FAKE + 64) == vt.VT_ERR_INVALID_ARG          # workspace not 256-B aligned
    assert _attn(cfg, max_seq=65) == vt.VT_ERR_INVALID_ARG            # max_seqlen > total
    assert _attn(cfg, n_img=0) == vt.VT_ERR_INVALID_ARG
    assert _attn(cfg, dtype=7) == vt.VT_ERR_INVALID_ARG
    assert _attn(vt.config(head_dim=64, hidden=1024, rope_pairs=(0, 16, 16))) == vt.VT_ERR_UNSUPPORTED
    assert _attn(vt.config(rope_pairs=(8, 12, 20))) == vt.VT_ERR_UNSUPPORTED
    assert _attn(vt.config(rope_pairs=(8, 16, 8))) == vt.VT_ERR_INVALID_ARG


@needs_no_gpu
def test_attention_two_part_validation():
    """vt_attention_pack validates as vt_attention_varlen (less out and its
    dtype); vt_attention_packed validates the sizes, out, dtype, ws and the
    optional host-side lengths (the workspace's contents are device data and
    are not checked)."""
    cfg = vt.config()
    P = lambda v: None if v is None else ctypes.c_void_p(v)
    need = vt.vt_block_workspace_size(cfg, 64, 1, 64)

    def pack(cfg=cfg, qkv=FAKE, cu=FAKE, n_img=1, total=64, max_seq=64, ws=FAKE, ws_bytes=need):
        return vt.LIB.vt_attention_pack(ctypes.byref(cfg), P(qkv), P(cu), P(FAKE), n_img, total, max_seq,
                                        P(ws), ws_bytes, None)

    def packed(cfg=cfg, n_img=1, total=64, max_seq=64, out=FAKE, dtype=vt.VT_BF16, ws=FAKE, ws_bytes=need,
               lens=None):
        hs = None if lens is None else (ctypes.c_int32 * len(lens))(*lens)
        return vt.LIB.vt_attention_packed(ctypes.byref(cfg), n_img, total, max_seq, hs, P(out), dtype, P(ws),
                                          ws_bytes, None)

    assert pack(ws_bytes=need - 1) == vt.VT_ERR_WORKSPACE
    assert pack(qkv=None) == vt.VT_ERR_INVALID_ARG
    assert pack(cu=None) == vt.VT_ERR_INVALID_ARG
    assert pack(max_seq=65) == vt.VT_ERR_INVALID_ARG
    assert pack(ws=FAKE + 64) == vt.VT_ERR_INVALID_ARG
    assert pack(vt.config(rope_pairs=(8, 12, 20))) == vt.VT_ERR_UNSUPPORTED
    assert packed(ws_bytes=need - 1) == vt.VT_ERR_WORKSPACE
    assert packed(ws=None) == vt.VT_ERR_WORKSPACE
    assert packed(out=None) == vt.VT_ERR_INVALID_ARG
    assert packed(out=FAKE + 8) == vt.VT_ERR_INVALID_ARG
    assert packed(dtype=7) == vt.VT_ERR_INVALID_ARG
    assert packed(n_img=0) == vt.VT_ERR_INVALID_ARG
    assert packed(max_seq=65) == vt.VT_ERR_INVALID_ARG
    assert packed(vt.config(head_dim=64, hidden=1024, rope_pairs=(0, 16, 16))) == vt.VT_ERR_UNSUPPORTED
    assert packed(lens=[63]) == vt.VT_ERR_INVALID_ARG                 # does not add up to total_tokens
    assert "add up" in vt.last_error()
    assert packed(lens=[65]) == vt.VT_ERR_INVALID_ARG                 # beyond max_seqlen
    assert packed(n_img=2, max_seq=40, lens=[0, 64]) == vt.VT_ERR_INVALID_ARG
    assert packed(ws_bytes=need - 1, lens=[64]) == vt.VT_ERR_WORKSPACE


def _attn_bwd(cfg, qkv=FAKE, dout=FAKE, dqkv=FAKE, n_img=1, total=64, max_seq=64, ws=FAKE,
              ws_bytes=None, dtype=vt.VT_FP32):
    if ws_bytes is None:
        ws_bytes = vt.vt_attention_backward_workspace_size(cfg, total, n_img, max_seq)
    P = lambda v: None if v is None else ctypes.c_void_p(v)
    return vt.LIB.vt_attention_backward(ctypes.byref(cfg), P(qkv), P(FAKE), P(FAKE), n_img, total,
                                        max_seq, P(dout), P(dqkv), dtype, P(ws), ws_bytes, None)


@needs_no_gpu
def test_attention_backward_validation():
    cfg = vt.config()
    need = vt.vt_attention_backward_workspace_size(cfg, 64, 1, 64)
    assert need > vt.vt_block_workspace_size(cfg, 64, 1, 64) // 2
    assert _attn_bwd(cfg, ws_bytes=need - 1) == vt.VT_ERR_WORKSPACE
    assert _attn_bwd(cfg, dout=None) == vt.VT_ERR_INVALID_ARG
    assert _attn_bwd(cfg, dqkv=FAKE + 4) == vt.VT_ERR_INVALID_ARG
    assert _attn_bwd(cfg, n_img=0) == vt.VT_ERR_INVALID_ARG
    assert _attn_bwd(cfg, dtype=5) == vt.VT_ERR_INVALID_ARG
    assert _attn_bwd(vt.config(head_dim=64, hidden=1024, rope_pairs=(0, 16, 16))) == vt.VT_ERR_UNSUPPORTED
    assert vt.vt_attention_backward_workspace_size(cfg, 0, 1, 1) == 0


@needs_no_gpu
def test_block_backward_validation():
    cfg = vt.config()
    P = ctypes.c_void_p
    need = vt.vt_block_backward_workspace_size(cfg, 64, 1, 64)
    assert need > vt.vt_attention_backward_workspace_size(cfg, 64, 1, 64)
    bw = vt.vt_block_weights()
    for name, _ in vt.vt_block_weights._fields_:
        setattr(bw, name, FAKE)
    g = vt.vt_block_grads()

    def call(cfg=cfg, resid=FAKE, dresid=FAKE, grads=g, ws_bytes=need, n_img=1, bw=bw):
        return vt.LIB.vt_block_backward(ctypes.byref(cfg), P(resid), ctypes.byref(bw), P(FAKE), P(FAKE),
                                        n_img, 64, 64, P(dresid),
                                        ctypes.byref(grads) if grads is not None else None, P(FAKE),
                                        ws_bytes, None)
    assert call(ws_bytes=need - 1) == vt.VT_ERR_WORKSPACE
    assert call(resid=None) == vt.VT_ERR_INVALID_ARG
    assert call(dresid=FAKE + 4) == vt.VT_ERR_INVALID_ARG
    assert call(grads=None) == vt.VT_ERR_INVALID_ARG
    assert call(n_img=0) == vt.VT_ERR_INVALID_ARG
    g2 = vt.vt_block_grads()
    g2.w_o = FAKE + 8
    assert call(grads=g2) == vt.VT_ERR_INVALID_ARG
    bw2 = vt.vt_block_weights()
    assert call(bw=bw2) == vt.VT_ERR_INVALID_ARG                       # NULL weights
    wide = vt.config(hidden=2560, heads=32)
    assert call(cfg=wide, ws_bytes=1 << 40) == vt.VT_ERR_UNSUPPORTED   # hidden > 2048


@needs_no_gpu
def test_tower_backward_validation():
    cfg = vt.config(layers=2)
    P = ctypes.c_void_p
    grids = [(1, 4, 4)]
    need = vt.vt_tower_backward_workspace_size(cfg, grids)
    assert need > 0
    blocks = (vt.vt_block_weights * 2)()
    for b in blocks:
        for name, _ in vt.vt_block_weights._fields_:
            setattr(b, name, FAKE)
    tw = vt.vt_tower_weights()
    tw.w_patch = FAKE
    tw.blocks = ctypes.cast(blocks, ctypes.POINTER(vt.vt_block_weights))
    bg = (vt.vt_block_grads * 2)()
    tg = vt.vt_tower_grads()
    tg.blocks = ctypes.cast(bg, ctypes.POINTER(vt.vt_block_grads))

    def call(grids=grids, d_tower=FAKE, tg=tg, ws_bytes=need, tw=tw, cfg=cfg):
        g, n = vt._lib._grid(grids)
        return vt.LIB.vt_tower_backward(ctypes.byref(cfg), P(FAKE), g, n, ctypes.byref(tw), P(d_tower),
                                        ctypes.byref(tg) if tg is not None else None, P(FAKE), ws_bytes,
                                        None)
    assert call(ws_bytes=need - 1) == vt.VT_ERR_WORKSPACE
    assert call(d_tower=None) == vt.VT_ERR_INVALID_ARG
    assert call(tg=None) == vt.VT_ERR_INVALID_ARG
    assert call(grids=[(1, 3, 4)]) == vt.VT_ERR_INVALID_ARG
    tg2 = vt.vt_tower_grads()                                       # blocks missing
    assert call(tg=tg2) == vt.VT_ERR_INVALID_ARG
    bg[1].w_o = FAKE + 4                                            # misaligned gradient
    assert call() == vt.VT_ERR_INVALID_ARG
    assert "block 1" in vt.last_error()
    bg[1].w_o = None
    tw2 = vt.vt_tower_weights()
    tw2.w_patch = FAKE
    assert call(tw=tw2) == vt.VT_ERR_INVALID_ARG                    # blocks NULL
    assert vt.vt_tower_backward_workspace_size(cfg, [(1, 3, 3)]) == 0


def test_attention_backward_workspace_is_affine():
    cfg = vt.config()
    s = [vt.vt_attention_backward_workspace_size(cfg, n, 1, n) for n in (4096, 8192, 16384)]
    assert abs((s[2] - s[1]) - 2 * (s[1] - s[0])) <= 4096
    assert (s[1] - s[0]) / 4096 < 40 * 1024       # about 36 KB per token at 16 heads
    b = [vt.vt_block_backward_workspace_size(cfg, n, 1, n) for n in (4096, 8192, 16384)]
    # up to the GEMMs' partial-sum area (at most 64 MiB), present or not by shape
    assert abs((b[2] - b[1]) - 2 * (b[1] - b[0])) <= 256 * 256 * 256 * 4 + 4096
    assert (b[1] - b[0]) / 4096 < 128 * 1024      # about 115 KB per token


@needs_no_gpu
def test_linear_and_layer_norm_validation():
    P = ctypes.c_void_p
    L = vt.LIB
    assert L.vt_linear(P(FAKE), 16, 100, P(FAKE), 64, None, 0, P(FAKE), None, 0, None) == vt.VT_ERR_UNSUPPORTED
    assert L.vt_linear(P(FAKE), 16, 64, P(FAKE), 96, None, 0, P(FAKE), None, 0, None) == vt.VT_ERR_UNSUPPORTED
    assert L.vt_linear(P(FAKE), 0, 64, P(FAKE), 64, None, 0, P(FAKE), None, 0, None) == vt.VT_ERR_INVALID_ARG
    assert L.vt_linear(P(FAKE), 16, 64, P(FAKE), 64, P(FAKE + 2), 0, P(FAKE), None, 0, None) == vt.VT_ERR_INVALID_ARG
    assert L.vt_linear(P(FAKE), 16, 64, P(FAKE), 64, None, 9, P(FAKE), None, 0, None) == vt.VT_ERR_INVALID_ARG
    # small M with a long K plans a split-K: the partial buffer must be supplied
    need = vt.vt_linear_workspace_size(256, 6144, 24576)
    assert need > 0
    assert L.vt_linear(P(FAKE), 256, 24576, P(FAKE), 6144, None, 0, P(FAKE), None, 0, None) == vt.VT_ERR_WORKSPACE
    assert L.vt_layer_norm(P(FAKE), 4, 1000, P(FAKE), P(FAKE), 1e-6, P(FAKE), None) == vt.VT_ERR_UNSUPPORTED
    assert L.vt_layer_norm(P(FAKE), 4, 1280, P(FAKE), P(FAKE), 0.0, P(FAKE), None) == vt.VT_ERR_INVALID_ARG
    assert L.vt_layer_norm(None, 4, 1280, P(FAKE), P(FAKE), 1e-6, P(FAKE), None) == vt.VT_ERR_INVALID_ARG


@needs_no_gpu
def test_clock_probe_validation():
    P = ctypes.c_void_p
    hz = ctypes.c_int64(0)
    L = vt.LIB
    assert L.vt_clock_probe(0, P(FAKE), ctypes.byref(hz), None) == vt.VT_ERR_INVALID_ARG
    assert L.vt_clock_probe(10_000_001, P(FAKE), ctypes.byref(hz), None) == vt.VT_ERR_INVALID_ARG
    assert L.vt_clock_probe(1000, P(FAKE + 4), ctypes.byref(hz), None) == vt.VT_ERR_INVALID_ARG
    assert L.vt_clock_probe(1000, None, ctypes.byref(hz), None) == vt.VT_ERR_INVALID_ARG
    assert L.vt_clock_probe(1000, P(FAKE), None, None) == vt.VT_ERR_INVALID_ARG


@needs_no_gpu
def test_tower_validation():
    cfg = vt.config(layers=0)
    g, n = vt._lib._grid([(1, 4, 4)])
    tw = vt.vt_tower_weights()
    tw.w_patch = FAKE
    P = ctypes.c_void_p
    need = vt.vt_tower_workspace_size(cfg, [(1, 4, 4)])
    L = vt.LIB
    # no output requested
    assert L.vt_tower_forward(ctypes.byref(cfg), P(FAKE), g, n, ctypes.byref(tw), None, None, None,
                              P(FAKE), need, None) == vt.VT_ERR_INVALID_ARG
    # projector requested without projector weights
    assert L.vt_tower_forward(ctypes.byref(cfg), P(FAKE), g, n, ctypes.byref(tw), None, None,
                              P(FAKE), P(FAKE), need, None) == vt.VT_ERR_INVALID_ARG
    assert "projector" in vt.last_error()
    # workspace one byte short
    assert L.vt_tower_forward(ctypes.byref(cfg), P(FAKE), g, n, ctypes.byref(tw), P(FAKE), None,
                              None, P(FAKE), need - 1, None) == vt.VT_ERR_WORKSPACE
    # layers > 0 with no block array
    cfg1 = vt.config(layers=1)
    assert L.vt_tower_forward(ctypes.byref(cfg1), P(FAKE), g, n, ctypes.byref(tw), P(FAKE), None,
                              None, P(FAKE), need, None) == vt.VT_ERR_INVALID_ARG
    assert vt.LIB.vt_status_string(3) == b"VT_ERR_WORKSPACE"


def test_package_fails_loudly_without_library(tmp_path):
    """A copy of the package without libvt.so refuses to import (no CPU
    fallback exists to route to)."""
    import shutil
    import subprocess
    import sys
    src = os.path.dirname(vt.__file__)
    dst = tmp_path / "vision_transformer_encoder_tiled_amd"
    dst.mkdir()
    for f in os.listdir(src):
        if f.endswith(".py"):
            shutil.copy(os.path.join(src, f), dst / f)
    r = subprocess.run([sys.executable, "-c", "import vision_transformer_encoder_tiled_amd"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=120,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "libvt.so is missing" in r.stderr


def test_package_does_not_load_the_oracle():
    """Importing the library binding loads no oracle module: the product path
    never reaches the CPU oracle."""
    import subprocess
    import sys
    code = ("import sys, vision_transformer_encoder_tiled_amd; "
            "print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "[]"


def test_noalloc_scratch_size_matches_the_header():
    m = re.search(r"#define\s+VT_NOALLOC_SCRATCH_BYTES\s+\((\d+)u \* (\d+)u \* (\d+)u\)", open(HEADER).read())
    assert m and int(m[1]) * int(m[2]) * int(m[3]) == vt.VT_NOALLOC_SCRATCH_BYTES


@needs_no_gpu
def test_attention_noalloc_validation():
    """Rejections happen on the host before the fixed array's address is
    looked up: sizes whose attention scratch exceeds the array, and the
    argument errors of vt_attention_varlen."""
    cfg = vt.config()
    P = lambda v: None if v is None else ctypes.c_void_p(v)

    def call(qkv=FAKE, out=FAKE, n_img=1, total=64, max_seq=64, dtype=vt.VT_BF16, cfg=cfg):
        return vt.LIB.vt_attention_varlen_noalloc(ctypes.byref(cfg), P(qkv), P(FAKE), P(FAKE), n_img, total,
                                                  max_seq, P(out), dtype, None)
    assert call(total=8192, max_seq=8192) == vt.VT_ERR_WORKSPACE       # one image of 8,192 tokens
    assert "fixed array" in vt.last_error()
    assert call(n_img=8, total=8192, max_seq=1024) == vt.VT_ERR_WORKSPACE   # eight 448x448 images
    assert call(qkv=None) == vt.VT_ERR_INVALID_ARG
    assert call(out=FAKE + 8) == vt.VT_ERR_INVALID_ARG
    assert call(n_img=0) == vt.VT_ERR_INVALID_ARG
    assert call(max_seq=65) == vt.VT_ERR_INVALID_ARG
    assert call(dtype=7) == vt.VT_ERR_INVALID_ARG
    assert call(cfg=vt.config(head_dim=64, hidden=1024, rope_pairs=(0, 16, 16))) == vt.VT_ERR_UNSUPPORTED
