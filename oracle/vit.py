"""Oracle functions, one per step of the tower's forward pass.

Every function works on plain numpy arrays.  The tower entry points compute in
float32 (matmuls are ``np.matmul``); the per-step functions keep the dtype they
are given, so the pin tests can also run them in float64.

Sources (page titles of the reference material):

* "MiniMax-M3-Vision README", Architecture table: layer count and widths,
  patch 14, Conv3d patch embed, 3D RoPE, GELU, 2x2 merge, temporal patch 2,
  the projector Linear(1280,6144) GELU Linear(6144,6144), flatten four
  6144-wide patches, Linear(24576,6144) GELU Linear(6144,6144); the paragraph
  under it gives the 1280 / 5120 / 6144 output widths.
* "v2_loaders FINDINGS", section 3 (MiniMax-M3 vision tower): temporal dim
  padded to 2 by repeating the frame, ``grid_thw = [[1, h, w]]``, 3D RoPE with
  theta 10000.
* "v2_loaders FINDINGS", section 1 (MoonViT): native-resolution patches
  unfolded to (N, 3, 14, 14) with a per-image ``grid_hws``.
* "init.rs (VisionEncoder::new)": bf16 decode by shifting the 16 bits into the
  high half of an fp32; the vision RoPE inverse-frequency ladder
  ``theta^(-2k/dim)``.

Readings where the pages are silent (each is also listed in the design notes):
attention scale 1/sqrt(80); RoPE rotate-half pairing (x_j, x_{j+40}); pairs
[0,8) -> t, [8,24) -> h, [24,40) -> w with a per-axis ladder
``theta^(-2k/(2 n_axis))``; positions are integer patch coordinates per image
(t, row, col), t = 0 for a still image; LayerNorm with biased variance and eps inside the sqrt;
GELU(tanh) in the blocks and the projector; W_qkv rows are [Q | K | V], each
head-major 16 x 80; attention is block-diagonal per image, non-causal; tokens
in raster order inside an image; merged token m = (r, c) gathers the 2x2 block
in order k = 2*dr + dc.

Parity pins (tests/test_oracle_*.py): every function below is pinned by at
least one check that does not re-type its formula -- brute force in float64,
closed forms, invariants or values printed on the pages.  The full 32-layer
tower has no external numerical reference (no real weights exist here): its
composition is pinned only through its pinned parts ("parity unpinned" for
the end-to-end numbers against any external implementation).
"""
from __future__ import annotations

import math

import numpy as np

PATCH = 14
T_PATCH = 2


# ------------------------------------------------------------------ decoding
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> fp32 upcast: the 16 bits become the high half of the fp32
    word ("init.rs (VisionEncoder::new)", pos-embed download)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------ metadata
def cu_seqlens(grids) -> np.ndarray:
    """Offsets of each image's tokens in the packed sequence: cu[i+1] = cu[i] + t*h*w."""
    cu = [0]
    for t, h, w in grids:
        cu.append(cu[-1] + t * h * w)
    return np.asarray(cu, dtype=np.int32)


def positions(grids) -> np.ndarray:
    """Per-token (t, row, col) integer patch coordinates, raster order inside
    each image, restarting at 0 for every image ("v2_loaders FINDINGS" s.3,
    ``grid_thw``; mixed grids as in s.1)."""
    out = []
    for t, h, w in grids:
        for tt in range(t):
            for r in range(h):
                for c in range(w):
                    out.append((tt, r, c))
    return np.asarray(out, dtype=np.int32).reshape(-1, 3)


def merge_map(grids) -> np.ndarray:
    """[N/4, 4] global raster token indices gathered into each merged token.

    Merged token m = (tt, r, c) of an image (raster over the (t, h/2, w/2)
    grid) takes patches (tt, 2r+dr, 2c+dc) in slot k = 2*dr + dc (2x2
    spatial merge, MiniMax-M3-Vision README, Architecture table; the merge is
    spatial, so each temporal slice is merged on its own)."""
    out = []
    base = 0
    for t, h, w in grids:
        for tt in range(t):
            for r in range(h // 2):
                for c in range(w // 2):
                    out.append([base + tt * h * w + (2 * r + dr) * w + (2 * c + dc)
                                for dr in (0, 1) for dc in (0, 1)])
        base += t * h * w
    return np.asarray(out, dtype=np.int64).reshape(-1, 4)


# ------------------------------------------------------------------ patchify
def frames_of(t: int) -> int:
    """Frames stored per item: a still image (t = 1) is one frame, repeated
    to fill the temporal patch of 2 ("v2_loaders FINDINGS" s.3); a clip with
    t temporal patches is 2t frames (README Architecture: temporal patch 2)."""
    return 1 if t == 1 else 2 * t


def patchify(pix: np.ndarray) -> np.ndarray:
    """[3, 14h, 14w] (still image) or [2t, 3, 14h, 14w] (clip) -> rows in
    raster patch order over (temporal patch, row, col).

    Row layout is (channel, tau, py, px), i.e. a Conv3d weight
    [1280, 3, 2, 14, 14] flattened, so that ``X @ W.T`` is the Conv3d with
    kernel = stride = (2, 14, 14) (README Architecture: Conv3d patch embed);
    temporal patch tt covers frames 2tt and 2tt+1.  A still image's single
    frame is repeated ("v2_loaders FINDINGS" s.3)."""
    frames = pix[None] if pix.ndim == 3 else pix
    if frames.shape[0] == 1:
        frames = np.concatenate([frames, frames], axis=0)
    F, c, H, W = frames.shape
    assert F % T_PATCH == 0
    t, h, w = F // T_PATCH, H // PATCH, W // PATCH
    p = frames.reshape(t, T_PATCH, c, h, PATCH, w, PATCH)
    p = p.transpose(0, 3, 5, 2, 1, 4, 6)  # t, h, w, c, tau, py, px
    return np.ascontiguousarray(p.reshape(t * h * w, c * T_PATCH * PATCH * PATCH))


def unpatchify(x: np.ndarray, h: int, w: int) -> np.ndarray:
    """Inverse of :func:`patchify` for a still image, using the tau = 0 slice."""
    p = x.reshape(h, w, 3, T_PATCH, PATCH, PATCH)[:, :, :, 0]
    return np.ascontiguousarray(p.transpose(2, 0, 3, 1, 4).reshape(3, h * PATCH, w * PATCH))


# ------------------------------------------------------------------ basic ops
def linear(x: np.ndarray, w: np.ndarray, b=None) -> np.ndarray:
    """PyTorch Linear: y = x @ W^T + b, W stored [out, in]."""
    y = np.matmul(x, w.T)
    if b is not None:
        y = y + b
    return y


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """Textbook LayerNorm over the last axis: biased variance, eps inside the sqrt, then affine."""
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    return xc / np.sqrt(var + x.dtype.type(eps)) * g + b


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    dt = x.dtype.type
    k = dt(math.sqrt(2.0 / math.pi))
    return dt(0.5) * x * (dt(1.0) + np.tanh(k * (x + dt(0.044715) * x * x * x)))


def gelu_erf(x: np.ndarray) -> np.ndarray:
    """GELU, exact form: 0.5 x (1 + erf(x / sqrt 2)) (erf from the math library)."""
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return (0.5 * x.astype(np.float64) * (1.0 + erf(x.astype(np.float64) / math.sqrt(2.0)))).astype(x.dtype)


# ------------------------------------------------------------------ 3D RoPE
def rope_tables(head_dim=80, sections=(8, 16, 16), theta=10000.0, shared_ladder=False):
    """(axis[j], inv_freq[j]) for the head_dim/2 rotation pairs.

    Pairs are split over the (t, h, w) axes by ``sections`` in that order.
    Per-axis ladder (default): pair k of an axis with n pairs turns at
    theta^(-2k / (2n)), the vision ladder theta^(-2k/dim) of
    "init.rs (VisionEncoder::new)" applied with dim = 2n for each axis.
    Shared ladder: pair j turns at theta^(-2j/head_dim) whatever its axis."""
    half = head_dim // 2
    assert sum(sections) == half
    axis = np.concatenate([np.full(n, a, dtype=np.int32) for a, n in enumerate(sections)])
    if shared_ladder:
        inv = np.array([theta ** (-2.0 * j / head_dim) for j in range(half)], dtype=np.float64)
    else:
        inv = np.concatenate([[theta ** (-2.0 * k / (2 * n)) for k in range(n)] for n in sections])
    return axis, inv.astype(np.float64)


def apply_rope(x: np.ndarray, pos: np.ndarray, axis: np.ndarray, inv_freq: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on [n, heads, head_dim] with per-token 3D positions [n, 3].

    Pair j = (x_j, x_{j+half}) turns by angle pos[axis[j]] * inv_freq[j]:
    x'_j = x_j cos - x_{j+half} sin,  x'_{j+half} = x_{j+half} cos + x_j sin.
    Angles are formed in float64 and rounded to x's dtype."""
    half = x.shape[-1] // 2
    ang = pos[:, axis].astype(np.float64) * inv_freq[None, :]          # [n, half]
    cos = np.cos(ang).astype(x.dtype)[:, None, :]
    sin = np.sin(ang).astype(x.dtype)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


# ------------------------------------------------------------------ attention
def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Exact row softmax exp(s - rowmax) / sum."""
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention_image(q, k, v, scale=None, rows=None, chunk=512):
    """Non-causal softmax attention of one image, one head group.

    q, k, v: [n, heads, hd].  Returns [len(rows), heads, hd] for the query
    rows ``rows`` (default: all).  Scores are formed for full rows, a chunk of
    queries at a time (exact softmax, not online)."""
    n, H, hd = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(hd)
    scale = q.dtype.type(scale)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    out = np.empty((len(rows), H, hd), dtype=q.dtype)
    kt = np.ascontiguousarray(k.transpose(1, 2, 0))   # H, hd, n
    vh = np.ascontiguousarray(v.transpose(1, 0, 2))   # H, n, hd
    for s0 in range(0, len(rows), chunk):
        r = rows[s0:s0 + chunk]
        qh = np.ascontiguousarray(q[r].transpose(1, 0, 2))      # H, m, hd
        p = softmax_rows(np.matmul(qh, kt) * scale)             # H, m, n
        out[s0:s0 + len(r)] = np.matmul(p, vh).transpose(1, 0, 2)
    return out


def attention_varlen(q, k, v, cu, scale=None):
    """Block-diagonal attention over packed images: image i attends only to
    tokens cu[i]..cu[i+1] (no cross-image attention)."""
    out = np.empty_like(q)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        out[a:b] = attention_image(q[a:b], k[a:b], v[a:b], scale)
    return out


# ------------------------------------------------------------------ model
class Config:
    """Tower shape (README Architecture table) and the readings listed above."""

    def __init__(self, hidden=1280, heads=16, head_dim=80, mlp=5120, layers=32,
                 proj=6144, ln_eps=1e-6, rope_theta=10000.0, rope_sections=(8, 16, 16),
                 rope_shared_ladder=False, gelu_proj="tanh"):
        self.hidden, self.heads, self.head_dim, self.mlp = hidden, heads, head_dim, mlp
        self.layers, self.proj, self.ln_eps = layers, proj, ln_eps
        self.rope_theta, self.rope_sections = rope_theta, tuple(rope_sections)
        self.rope_shared_ladder, self.gelu_proj = rope_shared_ladder, gelu_proj


def weights_f32(bits: dict) -> dict:
    """Decode every bf16 tensor of a weight dict to fp32."""
    return {k: bf16_to_f32(v) for k, v in bits.items()}


def block_forward(R, W, pos, cu, cfg: Config, prefix="l0.", return_attn=False):
    """One pre-LN block on the fp32 residual R [N, d]:
    x = LN1(R); q,k,v = x W_qkv^T + b; RoPE(q), RoPE(k); A = attention;
    R += A W_o^T + b_o; R += GELU(LN2(R) W_1^T + b_1) W_2^T + b_2."""
    N, d = R.shape
    H, hd = cfg.heads, cfg.head_dim
    g = lambda name: W[prefix + name]
    x = layer_norm(R, g("ln1_g"), g("ln1_b"), cfg.ln_eps)
    qkv = linear(x, g("w_qkv"), g("b_qkv")).reshape(N, 3, H, hd)
    axis, inv = rope_tables(hd, cfg.rope_sections, cfg.rope_theta, cfg.rope_shared_ladder)
    q = apply_rope(qkv[:, 0], pos, axis, inv)
    k = apply_rope(qkv[:, 1], pos, axis, inv)
    v = np.ascontiguousarray(qkv[:, 2])
    a = attention_varlen(q, k, v, cu).reshape(N, d)
    R = R + linear(a, g("w_o"), g("b_o"))
    x = layer_norm(R, g("ln2_g"), g("ln2_b"), cfg.ln_eps)
    R = R + linear(gelu_tanh(linear(x, g("w_fc1"), g("b_fc1"))), g("w_fc2"), g("b_fc2"))
    if return_attn:
        return R, a
    return R


def patch_embed(images, W, grids):
    """Patchify every item (raster order over (t, row, col)) and apply the
    Conv3d-as-Linear embed."""
    X = np.concatenate([patchify(img) for img in images], axis=0)
    b = W.get("patch_b")
    return linear(X, W["patch_w"], b)


def split_pixels(flat, grids):
    """Cut the concatenated items out of one flat array: [3, 14h, 14w] for a
    still image (t = 1), [2t, 3, 14h, 14w] for a clip."""
    out, o = [], 0
    for t, h, w in grids:
        F = frames_of(t)
        n = F * 3 * PATCH * h * PATCH * w
        a = flat[o:o + n].reshape(F, 3, PATCH * h, PATCH * w)
        out.append(a[0] if F == 1 else a)
        o += n
    return out


def merge_gather(Y, grids):
    """[N, C] -> [N/4, 4C]: merged token m is the concatenation of its 2x2 patches, slot k = 2dr+dc."""
    mm = merge_map(grids)
    return Y[mm].reshape(mm.shape[0], 4 * Y.shape[1])


def projector(T, W, grids, cfg: Config):
    """Y2 = GELU(T W1^T + b1) W2^T + b2 per token; Z = 2x2 gather of Y2;
    Out = GELU(Z W3^T + b3) W4^T + b4 (README Architecture, Projector row)."""
    act = gelu_tanh if cfg.gelu_proj == "tanh" else gelu_erf
    y = linear(act(linear(T, W["p_w1"], W["p_b1"])), W["p_w2"], W["p_b2"])
    z = merge_gather(y, grids)
    return linear(act(linear(z, W["p_w3"], W["p_b3"])), W["p_w4"], W["p_b4"])


def mean_pool(T: np.ndarray, grids) -> np.ndarray:
    """[n_img, d]: the mean of each item's tower tokens -- the sequence
    mean-pooled to (1, 1280) per image ("v2_loaders FINDINGS" s.3,
    preprocessing line).  Token order inside an item does not matter."""
    cu = cu_seqlens(grids)
    return np.stack([T[cu[i]:cu[i + 1]].mean(axis=0, dtype=np.float64) for i in range(len(grids))]
                    ).astype(T.dtype)


def tower_forward(pixels_bits, grids, weight_bits, cfg: Config = None, n_layers=None,
                  keep_layers=False, projector_on=True, dtype=np.float32):
    """Full forward pass, fp32 by default.  Returns a dict with
    ``tower`` [N, d] (last_hidden_state, raster order), ``merged_raw`` [N/4, 4d],
    ``out`` [N/4, proj] (if the projector runs) and ``layers`` (list of the
    residual after each block, if requested).

    Block l reads the weights named ``l{l}.*``; the projector takes the last
    block's output.  ``dtype`` = np.float64 runs the same steps on the exactly
    decoded bf16 values in float64 (used to pin this composition against an
    independent float64 implementation)."""
    cfg = cfg or Config()
    W = {k: v.astype(dtype, copy=False) for k, v in weights_f32(weight_bits).items()}
    L = cfg.layers if n_layers is None else n_layers
    imgs = [x.astype(dtype, copy=False) for x in split_pixels(bf16_to_f32(pixels_bits), grids)]
    pos = positions(grids)
    cu = cu_seqlens(grids)
    R = patch_embed(imgs, W, grids).astype(dtype)
    layers = []
    for i in range(L):
        R = block_forward(R, W, pos, cu, cfg, prefix=f"l{i}.")
        if keep_layers:
            layers.append(R.copy())
    res = {"tower": R, "merged_raw": merge_gather(R, grids), "layers": layers}
    if projector_on:
        res["out"] = projector(R, W, grids, cfg)
    return res
