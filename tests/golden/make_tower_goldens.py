"""Write the oracle's expected values for the two workloads whose full oracle
pass takes too long to run inside a GPU test: the 2016x2016 image (144 x 144
patches, 20,736 tokens) and the eight seeded native-resolution grids.

Every number stored here comes from ``oracle.tower_forward`` (numpy fp32) on
the seeded inputs of ``synth`` -- nothing from the HIP library.  The tests
that read the files recompute the same seeds, sampled row indices and input
bits, and compare the library's outputs at those rows.

    python tests/golden/make_tower_goldens.py [--only 2016|mixed8] [--procs 8]

Outputs (numpy ``.npz``, no pickled objects):

* ``tower_2016_oracle.npz``: ``layer_rows`` [32, 16, 1280] -- the fp32
  residual after each block at 16 sampled raster rows (``layer_row_idx``);
  ``tower`` [64, 1280] at ``tower_row_idx``; ``out`` [16, 6144], the projected
  tokens at merged raster rows ``out_row_idx``; ``layer_norms`` [32], the
  L2 norm of each full residual.
* ``tower_mixed8_oracle.npz``: per image i, ``tower_i`` [32, 1280] at
  ``tower_row_idx_i`` (raster rows of that image) and ``out_i`` [4, 6144] at
  ``out_row_idx_i`` (merged raster rows of that image).  Each image is run
  through the oracle on its own: attention is block-diagonal and every other
  step works per token or per image, so an image's outputs are those of the
  packed batch (the varlen invariant pinned in tests/test_oracle_pins.py).

Workloads (MiniMax-M3-Vision README, Architecture table: 32 layers, hidden
1280, projector; v2_loaders FINDINGS section 1: native-resolution grids):
the seeds, grids and weight draw of ``synth.WORKLOADS``.
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

ROW_SEED = 2016


def sample(n: int, edge: int, extra: int, seed: int) -> np.ndarray:
    """Sorted distinct indices in [0, n): the first and last ``edge`` plus
    ``extra`` seeded draws."""
    g = np.random.Generator(np.random.PCG64(seed))
    idx = np.r_[0:min(edge, n), max(0, n - edge):n, g.integers(0, n, extra)]
    return np.unique(idx).astype(np.int64)


def rows_2016():
    N, M = 20736, 5184
    return (sample(N, 4, 8, ROW_SEED), sample(N, 8, 48, ROW_SEED + 1), sample(M, 2, 12, ROW_SEED + 2))


def rows_mixed8(i: int, n: int):
    return sample(n, 4, 24, 4000 + 10 * i), sample(n // 4, 1, 2, 4001 + 10 * i)


def log(msg):
    print(time.strftime("%H:%M:%S"), msg, flush=True)


def make_2016(weights):
    wl = synth.WORKLOADS["tower_2016"]
    px = synth.make_batch_pixels(wl)
    lrow, trow, orow = rows_2016()
    log("oracle tower 2016x2016 (20,736 tokens, 32 layers, projector)")
    t0 = time.perf_counter()
    ref = oracle.tower_forward(px, list(wl.grids), weights, keep_layers=True)
    log(f"  done in {time.perf_counter() - t0:.0f} s")
    np.savez_compressed(
        os.path.join(HERE, "tower_2016_oracle.npz"),
        layer_rows=np.stack([L[lrow] for L in ref["layers"]]).astype(np.float32),
        layer_row_idx=lrow,
        layer_norms=np.array([np.linalg.norm(L.astype(np.float64)) for L in ref["layers"]]),
        tower=ref["tower"][trow].astype(np.float32), tower_row_idx=trow,
        out=ref["out"][orow].astype(np.float32), out_row_idx=orow)


_WEIGHTS = None  # set before the worker processes fork, read by them


def _mixed_one(i):
    weights = _WEIGHTS
    from threadpoolctl import threadpool_limits
    wl = synth.WORKLOADS["tower_mixed8"]
    t, h, w = wl.grids[i]
    px = synth.make_pixels(h, w, wl.seeds[i]).reshape(-1)
    with threadpool_limits(1):
        t0 = time.perf_counter()
        ref = oracle.tower_forward(px, [(t, h, w)], weights)
    trow, orow = rows_mixed8(i, t * h * w)
    log(f"  image {i} ({h}x{w}) done in {time.perf_counter() - t0:.0f} s")
    return i, ref["tower"][trow].astype(np.float32), trow, ref["out"][orow].astype(np.float32), orow


def make_mixed8(weights, procs):
    import multiprocessing as mp
    global _WEIGHTS
    _WEIGHTS = weights
    wl = synth.WORKLOADS["tower_mixed8"]
    log(f"oracle tower on the 8 mixed grids {wl.grids}, one process per image")
    # largest images first so that the pool finishes together
    order = sorted(range(8), key=lambda i: -wl.grids[i][1] * wl.grids[i][2])
    with mp.get_context("fork").Pool(procs) as pool:
        res = pool.map(_mixed_one, order, chunksize=1)
    out = {}
    for i, tw, tr, ow, orr in res:
        out[f"tower_{i}"], out[f"tower_row_idx_{i}"] = tw, tr
        out[f"out_{i}"], out[f"out_row_idx_{i}"] = ow, orr
    np.savez_compressed(os.path.join(HERE, "tower_mixed8_oracle.npz"), **out)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", choices=["2016", "mixed8"], default=None)
    ap.add_argument("--procs", type=int, default=8)
    a = ap.parse_args()
    weights = synth.make_weights(32, projector=True)
    if a.only in (None, "mixed8"):
        make_mixed8(weights, a.procs)
    if a.only in (None, "2016"):
        make_2016(weights)
    log("written")


if __name__ == "__main__":
    main()
