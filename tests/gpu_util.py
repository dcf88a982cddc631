"""Helpers shared by the GPU parity tests: device upload of the seeded inputs,
comparison metrics, and the token-order permutation between the library's
2x2-window order and the oracle's raster order (taken from the oracle's own
integer maps, never from the GPU)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def window_to_raster(grids) -> np.ndarray:
    """perm[j] = raster index of the library's token j (window order), from the
    oracle's merge map: merged token m's four patches in slot order are the
    window-order tokens 4m .. 4m+3."""
    return oracle.merge_map(grids).reshape(-1)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def cosine_rows(a, b) -> np.ndarray:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return (a * b).sum(-1) / np.maximum(np.linalg.norm(a, axis=-1) * np.linalg.norm(b, axis=-1), 1e-30)


def bf16_f32(bits):
    return oracle.bf16_to_f32(bits)


def dev_bits(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def host_bits(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def upload_weights(w_bits: dict, torch) -> dict:
    return {k: dev_bits(v, torch) for k, v in w_bits.items()}


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def random_bf16(shape, seed, scale=1.0):
    return synth.bf16_bits(rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(scale))


def item_pixels(grids, seeds) -> np.ndarray:
    """Flat bf16 pixels of a list of items: a still image for t == 1
    ([3, 14h, 14w]), a clip of 2t frames otherwise."""
    return np.concatenate([(synth.make_pixels(h, w, s) if t == 1 else synth.make_clip(t, h, w, s)).reshape(-1)
                           for (t, h, w), s in zip(grids, seeds)])
