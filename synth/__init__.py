"""Seeded synthetic inputs for the vision tower: weights, pixels and image grids.

This module is the only code shared by the oracle side and the HIP side of the
tests and the benchmark.  It holds none of the tower's arithmetic: it draws
random numbers, rounds the fp32 draws to bfloat16 bit patterns (round to
nearest, ties to even) and names the tensors.  Both sides receive the same
uint16 bit patterns.

Workload recipe (MiniMax-M3 vision tower shape, MiniMax-M3-Vision README,
"Architecture" table):

* weights: ``numpy.random.SeedSequence(seed)`` spawns one child per tensor in
  the canonical order of :func:`weight_names`; matrices are
  ``PCG64(child).standard_normal(float32) * 0.02`` rounded to bf16; biases are
  0, LayerNorm gamma 1 and beta 0 (``affine="canonical"``).  The variant
  ``affine="random"`` draws biases ~N(0, 0.02), gammas 1+N(0, 0.1) and betas
  ~N(0, 0.1) so that every bias and affine path carries a non-zero value.
* pixels: ``PCG64(seed).random(float32)`` ~ U[0, 1) of shape [3, 14h, 14w],
  rounded to bf16.
* grids: fixed per workload; the mixed-resolution workload draws (h, w) even
  in [16, 96] from ``PCG64(4)``.
"""
from __future__ import annotations

import dataclasses

import numpy as np

PATCH = 14
HIDDEN = 1280
HEADS = 16
HEAD_DIM = 80
MLP = 5120
LAYERS = 32
PROJ = 6144
PATCH_DIM = 3 * 2 * PATCH * PATCH  # channels x temporal patch x 14 x 14 = 1176


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bfloat16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- tensor names
BLOCK_TENSORS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
                 "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2")
PROJ_TENSORS = ("p_w1", "p_b1", "p_w2", "p_b2", "p_w3", "p_b3", "p_w4", "p_b4")


def block_shapes(d=HIDDEN, mlp=MLP):
    return {
        "ln1_g": (d,), "ln1_b": (d,),
        "w_qkv": (3 * d, d), "b_qkv": (3 * d,),
        "w_o": (d, d), "b_o": (d,),
        "ln2_g": (d,), "ln2_b": (d,),
        "w_fc1": (mlp, d), "b_fc1": (mlp,),
        "w_fc2": (d, mlp), "b_fc2": (d,),
    }


def proj_shapes(d=HIDDEN, p=PROJ):
    return {
        "p_w1": (p, d), "p_b1": (p,),
        "p_w2": (p, p), "p_b2": (p,),
        "p_w3": (p, 4 * p), "p_b3": (p,),
        "p_w4": (p, p), "p_b4": (p,),
    }


def weight_names(n_layers: int, projector: bool = True):
    """Canonical tensor order: patch embed, then each block, then the projector."""
    names = ["patch_w", "patch_b"]
    for i in range(n_layers):
        names += [f"l{i}.{t}" for t in BLOCK_TENSORS]
    if projector:
        names += list(PROJ_TENSORS)
    return names


def _shape_of(name, d, mlp, p):
    if name == "patch_w":
        return (d, PATCH_DIM)
    if name == "patch_b":
        return (d,)
    if name.startswith("l"):
        return block_shapes(d, mlp)[name.split(".", 1)[1]]
    return proj_shapes(d, p)[name]


def _kind(name):
    base = name.split(".")[-1]
    if base.startswith("ln") and base.endswith("_g"):
        return "gamma"
    if base.startswith("ln") and base.endswith("_b"):
        return "beta"
    if base.startswith("w_") or base in ("patch_w",) or base.startswith("p_w"):
        return "matrix"
    return "bias"


def make_weights(n_layers: int = LAYERS, projector: bool = True, seed: int = 0,
                 affine: str = "canonical", d: int = HIDDEN, mlp: int = MLP,
                 p: int = PROJ) -> dict:
    """Return {name: uint16 bf16 bits} for the tower (and projector).

    The draw for a tensor depends only on (seed, its index in the canonical
    order), so a one-block model uses exactly the patch embed and layer 0 of
    the full tower's draw.
    """
    names = weight_names(LAYERS if n_layers <= LAYERS else n_layers, projector)
    children = np.random.SeedSequence(seed).spawn(len(names))
    keep = set(weight_names(n_layers, projector))
    out = {}
    for name, child in zip(names, children):
        if name not in keep:
            continue
        shape = _shape_of(name, d, mlp, p)
        kind = _kind(name)
        if kind == "matrix":
            g = np.random.Generator(np.random.PCG64(child))
            out[name] = bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(0.02))
        elif affine == "canonical":
            val = 1.0 if kind == "gamma" else 0.0
            out[name] = bf16_bits(np.full(shape, val, dtype=np.float32))
        elif affine == "random":
            g = np.random.Generator(np.random.PCG64(child))
            z = g.standard_normal(shape, dtype=np.float32)
            if kind == "gamma":
                v = 1.0 + np.float32(0.1) * z
            elif kind == "beta":
                v = np.float32(0.1) * z
            else:
                v = np.float32(0.02) * z
            out[name] = bf16_bits(v)
        else:
            raise ValueError(f"unknown affine mode {affine!r}")
    return out


def make_pixels(h: int, w: int, seed: int) -> np.ndarray:
    """bf16 bits of one image, [3, 14h, 14w], values ~U[0, 1)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return bf16_bits(g.random((3, PATCH * h, PATCH * w), dtype=np.float32))


def make_clip(t: int, h: int, w: int, seed: int) -> np.ndarray:
    """bf16 bits of one clip of 2t frames, [2t, 3, 14h, 14w], values ~U[0, 1)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return bf16_bits(g.random((2 * t, 3, PATCH * h, PATCH * w), dtype=np.float32))


# ---------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    grids: tuple          # ((t, h, w), ...)
    seeds: tuple          # pixel seed per image
    layers: int
    projector: bool
    description: str

    @property
    def tokens(self):
        return sum(t * h * w for t, h, w in self.grids)

    @property
    def n_img(self):
        return len(self.grids)


def mixed_grids(n: int = 8, seed: int = 4):
    """(h, w) patch grids, both even and uniform over the 41 even values in [16, 96]."""
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        h = 2 * int(g.integers(8, 49))
        w = 2 * int(g.integers(8, 49))
        out.append((1, h, w))
    return tuple(out)


WORKLOADS = {
    "block_224": Workload("block_224", ((1, 16, 16),), (1,), 1, False,
                          "one ViT block, one 224x224 image (16x16 patches)"),
    "tower_448": Workload("tower_448", ((1, 32, 32),), (2,), LAYERS, True,
                          "32-layer tower + 2x2 merge + projector, one 448x448 image"),
    "tower_448x16": Workload("tower_448x16", tuple((1, 32, 32) for _ in range(16)),
                             tuple(3000 + i for i in range(16)), LAYERS, True,
                             "16 images of 448x448 packed varlen through the tower + projector"),
    "tower_mixed8": Workload("tower_mixed8", mixed_grids(), tuple(4000 + i for i in range(8)),
                             LAYERS, True,
                             "8 native-resolution images, seeded even grids in [16, 96]"),
    "tower_2016": Workload("tower_2016", ((1, 144, 144),), (5,), LAYERS, True,
                           "one 2016x2016 image (144x144 patches) through the tower + projector"),
    "tower_clip16": Workload("tower_clip16", ((8, 32, 32),), (6,), LAYERS, True,
                             "one 16-frame 448x448 clip (8 temporal patches of 32x32) through the "
                             "tower + projector"),
    "tower_4096": Workload("tower_4096", ((1, 256, 256),), (7,), LAYERS, True,
                           "one 4096x4096 image (256x256 patches, 65,536 tokens) through the tower + "
                           "projector"),
}


def make_batch_pixels(wl: Workload) -> np.ndarray:
    """All items of a workload, flattened and concatenated (bf16 bits): one
    frame per still image (t = 1), 2t frames per clip."""
    return np.concatenate([(make_pixels(h, w, s) if t == 1 else make_clip(t, h, w, s)).reshape(-1)
                           for (t, h, w), s in zip(wl.grids, wl.seeds)])
