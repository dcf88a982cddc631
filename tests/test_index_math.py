"""CPU emulations of the index arithmetic of three device code paths, checked
before the kernels ran on a GPU and kept as regression checks of the
mappings they establish.  Each function below restates the kernel's index
expressions (named in its docstring) and checks that every access stays in
bounds and every output element is written exactly once."""
import itertools

import numpy as np
import pytest


def mfma_slot16(k):
    return (k & ~15) | (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1)


# ---------------------------------------------------------------- QKV pack epilogue
def qkv_feature(n, d, BN):
    """gemm.hip qkv_feature: output column -> W_qkv row (pair-major q/k tiles)."""
    if n >= 2 * d:
        return n
    part = 1 if n >= d else 0
    local = n - part * d
    c = local % BN
    p = (local - c) // 2 + c % (BN // 2)
    return part * d + (p // 40) * 80 + p % 40 + 40 * (c // (BN // 2))


@pytest.mark.parametrize("BN", [128, 256])
def test_qkv_feature_is_a_pair_major_bijection(BN):
    d = 1280
    f = [qkv_feature(n, d, BN) for n in range(3 * d)]
    assert sorted(f) == list(range(3 * d))
    for n0 in range(0, 2 * d, BN):
        part = 1 if n0 >= d else 0
        p0 = (n0 - part * d) // 2
        for q in range(BN // 16):            # chunk q and its partner chunk BN/16 + q
            for e in range(8):
                p = p0 + 8 * q + e
                assert f[n0 + 8 * q + e] == part * d + (p // 40) * 80 + p % 40
                assert f[n0 + BN // 2 + 8 * q + e] == part * d + (p // 40) * 80 + p % 40 + 40
            assert (p0 + 8 * q) // 40 == (p0 + 8 * q + 7) // 40   # a chunk never straddles heads
    for n in range(0, 2 * d, 4):  # the bias is read as 4 consecutive features
        assert f[n + 3] == f[n] + 3


def pack_store_counts(grids, BM, BN, d=1280, H=16):
    """gemm.hip qkv_pack_store with attention.hip attn_image_init_kernel's
    kslot: counts of the writes to Q and to the tile images."""
    N = sum(t * h * w for t, h, w in grids)
    cu = np.cumsum([0] + [t * h * w for t, h, w in grids])
    kts = np.cumsum([0] + [(cu[i + 1] - cu[i] + 63) // 64 for i in range(len(grids))])
    max_kt = (N + 63) // 64 + len(grids)
    kslot = np.full(N, -1)
    for i in range(len(grids)):
        for T in range(kts[i], kts[i + 1]):
            first = cu[i] + (T - kts[i]) * 64
            for s in range(min(64, cu[i + 1] - first)):
                kslot[first + s] = T * 64 + s
    assert (kslot >= 0).all()
    IMG, KOFF = 24576 // 2, 64 * 88
    q = np.zeros(N * 1280, int)
    kv = np.zeros(max_kt * H * IMG, int)
    for m0, n0 in itertools.product(range(0, N, BM), range(0, 3 * d, BN)):
        rows = range(m0, min(N, m0 + BM))
        if n0 < 2 * d:
            part = 1 if n0 >= d else 0
            p0 = (n0 - part * d) // 2
            for tok, qc in itertools.product(rows, range(BN // 16)):
                p = p0 + 8 * qc
                head, j0 = p // 40, p % 40
                for off in (0, 40):
                    sl = slice(j0 + off, j0 + off + 8)
                    if part == 0:
                        base = (tok * H + head) * 80
                        q[base + sl.start:base + sl.stop] += 1
                    else:
                        ks = kslot[tok]
                        assert (ks & 63) * 88 + sl.stop <= KOFF
                        base = ((ks >> 6) * H + head) * IMG + (ks & 63) * 88
                        kv[base + sl.start:base + sl.stop] += 1
        else:
            for tok in rows:
                ks = kslot[tok]
                for c in range(BN):
                    head, dim = (n0 - 2 * d + c) // 80, (n0 - 2 * d + c) % 80
                    assert KOFF + dim * 72 + 63 < IMG
                    kv[((ks >> 6) * H + head) * IMG + KOFF + dim * 72 + mfma_slot16(ks & 63)] += 1
    want = np.zeros_like(kv)
    for tok in range(N):
        T, s = kslot[tok] >> 6, kslot[tok] & 63
        for head in range(H):
            base = (T * H + head) * IMG
            want[base + s * 88: base + s * 88 + 80] += 1
            for dim in range(80):
                want[base + KOFF + dim * 72 + mfma_slot16(s)] += 1
    return q, kv, want


@pytest.mark.parametrize("BM,BN", [(128, 128), (256, 256)])
def test_qkv_pack_store_writes_every_operand_once(BM, BN):
    # a still image, a ragged one and a clip: key tiles start inside the
    # GEMM's row tiles (4 + 60 + 48 tokens)
    q, kv, want = pack_store_counts([(1, 2, 2), (1, 6, 10), (2, 4, 6)], BM, BN)
    assert (q == 1).all()
    assert (kv == want).all()


# ---------------------------------------------------------------- GEMM epilogue staging
def pass_rows(bm, row_bytes, ring):
    r = bm
    while r > 1 and r * row_bytes > ring:
        r //= 2
    return r


@pytest.mark.parametrize("BM,BN,GWM,GWN,NST,BK,CW", [
    (128, 128, 4, 2, 3, 64, 0), (128, 128, 4, 2, 4, 32, 0), (128, 160, 4, 1, 3, 64, 4),
    (128, 192, 4, 1, 3, 64, 4), (256, 256, 2, 4, 4, 32, 0)])
@pytest.mark.parametrize("f32", [False, True])
def test_gemm_epilogue_staging_is_a_bijection(BM, BN, GWM, GWN, NST, BK, CW, f32):
    """gemm.hip gemm_dl_kernel epilogue: the multiplying wavefronts write the
    accumulators of the current pass into the idle LDS ring (chunk-rotated
    rows), then every wavefront, copy-only ones included, reads 16-byte chunks
    back after the barrier and stores them.  Every LDS word is written once per
    pass and every output element is read back by exactly one thread, from the
    word that holds its own (row, column)."""
    NW, NWC = GWM * GWN, GWM * GWN + CW
    WM, WN = BM // GWM, BN // GWN
    ESZ = 4 if f32 else 2
    ROWB, RING = BN * ESZ, NST * (BM + BN) * 2 * BK
    CHUNKS, EPC = ROWB // 16, 16 // ESZ
    PR = pass_rows(BM, ROWB, RING)
    assert CHUNKS >= 16 and PR % WM == 0 and BM % PR == 0 and PR * ROWB <= RING
    done = {}
    for p in range(BM // PR):
        lds = {}
        for wave, lane in itertools.product(range(NW), range(64)):
            wm, wn = wave // GWN, wave % GWN
            if wm * WM // PR != p:
                continue
            fr, h = lane & 31, lane >> 5
            for t, f, g in itertools.product(range(WM // 32), range(WN // 32), range(4)):
                r = wm * WM + 32 * t + fr - p * PR
                c = (wn * WN + 32 * f + 8 * g) // EPC
                if f32:
                    off = r * ROWB + ((c + h + (r & 15)) % CHUNKS) * 16
                else:
                    off = r * ROWB + ((c + (r & 15)) % CHUNKS) * 16 + 8 * h
                for e in range(4):
                    assert off + e * ESZ not in lds
                    lds[off + e * ESZ] = (p * PR + r, wn * WN + 32 * f + 8 * g + 4 * h + e)
        for tid in range(64 * NWC):
            for i in range(tid, PR * CHUNKS, 64 * NWC):
                r, c = i // CHUNKS, i % CHUNKS
                for e in range(EPC):
                    row_col = lds[r * ROWB + ((c + (r & 15)) % CHUNKS) * 16 + e * ESZ]
                    assert row_col == (p * PR + r, c * EPC + e)
                    assert row_col not in done
                    done[row_col] = tid
    assert len(done) == BM * BN
