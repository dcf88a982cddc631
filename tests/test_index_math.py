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


@pytest.mark.parametrize("BM,BN,NW,CW,CO,BK", [
    (128, 160, 4, 4, True, 64), (128, 192, 4, 4, True, 64), (128, 128, 8, 0, False, 64),
    (128, 128, 8, 0, False, 32), (256, 256, 8, 0, False, 32)])
def test_gemm_copy_groups_fill_each_stage_once(BM, BN, NW, CW, CO, BK):
    """gemm.hip gemm_dl_kernel copy assignment: a K step is G = (BM + BN) / RPG
    groups of RPG rows (1 KB, one copy instruction); copying wavefront cw
    (with CO only the CW copy-only wavefronts, cw = wave - NW; else every
    wavefront, cw = wave) copies groups cw + NCP j for j < CP_LO, and one more
    (j = CP_LO) when cw < G % NCP, into LDS bytes 1024 cw + 1024 NCP j of the
    stage.  Every group lands once, at 1024 g, and each of its lanes fetches
    the row and chunk whose LDS bytes it writes (A rows first, then B rows)."""
    NWC = NW + CW
    NCP = CW if CO else NWC
    RB = 2 * BK
    CH, RPG = RB // 16, 1024 // RB
    GA, G = BM // RPG, (BM + BN) // RPG
    CP_HI, CP_LO = -(-G // NCP), G // NCP
    seen = {}
    for wave in range(NWC):
        mw = CW == 0 or wave < NW
        if CO and mw:
            continue                                  # issue() returns at once
        cw = max(wave - NW, 0) if CO else wave
        hi = cw < G % NCP
        for j in range(CP_HI):
            if j == CP_LO and not (CP_HI > CP_LO and hi):
                continue
            g = min(cw + NCP * j, G - 1)
            dst = 1024 * cw + 1024 * NCP * j
            assert dst == 1024 * g and g not in seen
            seen[g] = wave
            for lane in range(64):
                row = RPG * g + lane // CH            # stage row: A rows, then B rows
                assert (row < BM) == (g < GA)
                assert dst + 16 * lane == RB * row + 16 * (lane % CH)  # row r at byte RB r
    assert sorted(seen) == list(range(G))


# ---------------------------------------------------------------- lean attention split tail
def tail_pieces(n_items_keys, heads, S, min_tiles=8):
    """attention.hip tail_plan, the piece walk of attention_lean_kernel and
    the record lookup of attn_tail_merge_kernel.  n_items_keys[qt] = key
    tiles of q-tile qt (the schedule's order).  Returns the (qt, head, j0, j1,
    slot) pieces of every block and the merge's (item -> records) map."""
    nq = len(n_items_keys)
    qkpre = np.concatenate([[0], np.cumsum(n_items_keys)]).astype(np.int64)
    n_items = nq * heads
    nw = (n_items // S) * S // heads * heads
    T = heads * (qkpre[nq] - qkpre[nw // heads]) if nw < n_items else 0
    if T < S * min_tiles or (nw < n_items and n_items_keys[nw // heads] < 64):
        nw, T = n_items, 0
    pieces = [(i // heads, i % heads, 0, n_items_keys[i // heads], -1) for i in range(nw)]
    if T == 0:
        return pieces, {}, nw, T
    qt_tail = nw // heads
    tbase = qkpre[qt_tail]
    assert T < 2 ** 31
    for k in range(S):
        lo, hi = k * T // S, (k + 1) * T // S
        pos = lo
        a, z = qt_tail, nq - 1
        while a < z:
            mid = (a + z + 1) >> 1
            if heads * (qkpre[mid] - tbase) <= lo:
                a = mid
            else:
                z = mid - 1
        qt = a
        while pos < hi:
            while heads * (qkpre[qt + 1] - tbase) <= pos:
                qt += 1
            n = qkpre[qt + 1] - qkpre[qt]
            off = pos - heads * (qkpre[qt] - tbase)
            head, j0 = off // n, off % n
            j1 = min(n, j0 + (hi - pos))
            slot = -1 if (j0 == 0 and j1 == n) else (2 * k if pos == lo else 2 * k + 1)
            pieces.append((qt, head, j0, j1, slot))
            pos += j1 - j0
    merge = {}
    for u in range(S + heads):                  # the merge kernel's grid
        item = nw + u
        if item >= n_items:
            continue
        qt, head = item // heads, item % heads
        n = qkpre[qt + 1] - qkpre[qt]
        P0 = heads * (qkpre[qt] - tbase) + head * n
        wg_of = lambda p: ((p + 1) * S - 1) // T
        kA, kB = wg_of(P0), wg_of(P0 + n - 1)
        if kA == kB:
            continue
        merge[(qt, head)] = [2 * k if k * T // S >= P0 else 2 * k + 1 for k in range(kA, kB + 1)]
    return pieces, merge, nw, T


def q_tiles(grids, WQ):
    """Key tiles per q-tile in the schedule's order (largest image first)."""
    sizes = sorted((t * h * w for t, h, w in grids), reverse=True)
    return [(-(-n // 64)) for n in sizes for _ in range(-(-n // WQ))]


@pytest.mark.parametrize("grids,WQ,S", [
    ([(1, 144, 144)], 256, 512),                 # 2016x2016: 1,296 items, 2.53 rounds
    ([(1, 112, 112)], 256, 512),
    ([(1, 128, 128)], 256, 512),                 # exactly two rounds: no tail
    ([(1, 256, 256)], 256, 512),
    ([(1, 32, 32)] * 16, 256, 512),
    ([(1, 48, 48)], 128, 768),
    ([(1, 96, 96), (1, 16, 18), (1, 40, 22), (1, 64, 64), (1, 2, 2), (1, 90, 60)], 256, 512),
    ([(1, 96, 96), (1, 16, 18), (1, 40, 22), (1, 64, 64), (1, 2, 2), (1, 90, 60)], 128, 768),
    ([(1, 60, 80), (1, 20, 24)], 128, 700),      # a resident count that is no multiple of the heads
])
def test_lean_split_tail_covers_every_key_tile_once(grids, WQ, S):
    heads = 16
    nk = q_tiles(grids, WQ)
    pieces, merge, nw, T = tail_pieces(nk, heads, S)
    seen = {}
    slots = {}
    for qt, head, j0, j1, slot in pieces:
        assert 0 <= j0 < j1 <= nk[qt]
        for j in range(j0, j1):
            assert (qt, head, j) not in seen
            seen[(qt, head, j)] = slot
        if slot >= 0:
            assert slot not in slots and slot < 2 * S
            slots[slot] = (qt, head, j0, j1)
    assert len(seen) == heads * sum(nk)
    # each cut item's records are exactly the pieces written for it, and they
    # partition its key tiles
    cut = {(qt, head) for qt, head, j0, j1, slot in pieces if slot >= 0}
    assert cut == set(merge)
    for key, recs in merge.items():
        assert len(recs) >= 2
        spans = sorted(slots[r][2:] for r in recs)
        assert all(slots[r][:2] == key for r in recs)
        assert spans[0][0] == 0 and spans[-1][1] == nk[key[0]]
        assert all(a[1] == b[0] for a, b in zip(spans, spans[1:]))
    if T:
        assert len(nk) * heads - nw < S + heads       # the merge grid covers the tail
        assert min(j1 - j0 for *_, j0, j1, _s in pieces[nw:]) >= 1
    # the launch: max_qtiles x heads + S blocks; those that are neither a whole
    # item nor a tail range exit before reading a q-tile descriptor
    N = sum(t * h * w for t, h, w in grids)
    max_qtiles = -(-N // WQ) + len(grids)
    assert len(nk) <= max_qtiles
    n_run = 0
    for b in range(max_qtiles * heads + S):
        in_tail = T > 0 and b >= nw
        if not in_tail and b >= nw:
            continue
        if in_tail:
            assert b - nw >= 0
            n_run += b - nw < S
        else:
            assert b // heads < len(nk)
            n_run += 1
    assert n_run == nw + (S if T else 0)


# ---------------------------------------------------------------- GEMM stream-K tail
def gemm_streamk(M, N, K, CUs=256):
    """gemm.hip plan_gemm (256 x 256 tiles), the piece walk of
    gemm_dl_kernel<..., SK = true> and streamk_reduce_kernel's record lookup.
    Returns (n_whole, sk_wgs, pieces, reduce map)."""
    cdiv = lambda a, b: -(-a // b)
    t256 = cdiv(M, 256) * cdiv(N, 256)
    if not (t256 >= 192 and t256 > CUs and t256 % CUs and K >= 2048 and K % 32 == 0):
        return None
    nks = K // 32
    n_whole = t256 // CUs * CUs
    n_tail = t256 - n_whole
    if CUs % n_tail or nks < 8 * (CUs // n_tail):
        return None
    S = CUs
    T = n_tail * nks
    assert T < 2 ** 31
    pieces = []
    for k in range(S):
        lo, hi = k * T // S, (k + 1) * T // S
        pos = lo
        while pos < hi:
            u, s0 = pos // nks, pos % nks
            s1 = min(nks, s0 + (hi - pos))
            pieces.append((u, s0, s1, k if pos == lo else S + k))
            pos += s1 - s0
    red = {}
    for u in range(n_tail):
        P0 = u * nks
        wg_of = lambda p: ((p + 1) * S - 1) // T
        kA, kB = wg_of(P0), wg_of(P0 + nks - 1)
        red[u] = [k if k * T // S >= P0 else S + k for k in range(kA, kB + 1)]
    return n_whole, S, pieces, red


@pytest.mark.parametrize("M,N,K", [(16384, 1280, 5120), (4096, 6144, 24576), (4096, 6144, 6144),
                                   (4608, 4096, 2048), (16384, 2560, 2048), (20736, 1280, 5120),
                                   (5184, 6144, 24576)])
def test_gemm_streamk_tail_covers_every_k_step_once(M, N, K):
    plan = gemm_streamk(M, N, K)
    if plan is None:
        pytest.skip("no stream-K tail for this shape")
    n_whole, S, pieces, red = plan
    nks = K // 32
    n_tail = -(-M // 256) * -(-N // 256) - n_whole
    seen, slots = set(), {}
    per_wg = {}
    for u, s0, s1, slot in pieces:
        assert 0 <= u < n_tail and 0 <= s0 < s1 <= nks
        for j in range(s0, s1):
            assert (u, j) not in seen
            seen.add((u, j))
        assert slot not in slots and 0 <= slot < S          # inside the S records of the workspace
        slots[slot] = (u, s0, s1)
        per_wg[slot % S] = per_wg.get(slot % S, 0) + 1
    assert len(seen) == n_tail * nks
    assert max(per_wg.values()) == 1 and len(per_wg) == S   # one aligned piece per workgroup
    for u, recs in red.items():                             # the reduce reads exactly the pieces of its tile
        spans = sorted(slots[r][1:] for r in recs)
        assert all(slots[r][0] == u for r in recs)
        assert spans[0][0] == 0 and spans[-1][1] == nks
        assert all(a[1] == b[0] for a, b in zip(spans, spans[1:]))
    assert sorted(r for rs in red.values() for r in rs) == sorted(slots)


def group_tile(pid, tiles_m, tiles_n, GM=4):
    """gemm.hip group_tile: tile (tm, tn) of linear index pid, in groups of GM tile rows."""
    per_group = GM * tiles_n
    gid = pid // per_group
    first = gid * GM
    gsz = min(tiles_m - first, GM)
    in_g = pid - gid * per_group
    return first + in_g % gsz, in_g // gsz


def xcd_pid(npid, b):
    """gemm.hip xcd_pid: the tile index of block b when npid tiles are spread over 8 XCDs."""
    q, r, x, l = npid // 8, npid % 8, b % 8, b // 8
    return x * (q + 1) + l if x < r else r * (q + 1) + (x - r) * q + l


def quadrant_tail(M, N, K, CUs=256, limit=128):
    """gemm.hip tail_quadrant_tiles / plan_gemm: (n_whole, n_tail) when the
    last partial round of a 256 x 256 tiling runs as 128 x 128 quadrants, else None."""
    cdiv = lambda a, b: -(-a // b)
    t256 = cdiv(M, 256) * cdiv(N, 256)
    if t256 < 192 or t256 <= CUs or K % 32:
        return None
    n_tail = t256 % CUs
    if n_tail == 0 or n_tail > limit:
        return None
    nks = K // 32
    if K >= 2048 and CUs % n_tail == 0 and nks >= 8 * (CUs // n_tail):
        return None                                   # the stream-K tail takes it
    return t256 - n_tail, n_tail


@pytest.mark.parametrize("M,N,K", [(16384, 1280, 1280), (34852, 3840, 1280), (20736, 5120, 1280),
                                   (8192, 5120, 1280), (34852, 1280, 1280), (16500, 1280, 1280)])
def test_gemm_quadrant_tail_covers_every_tile_once(M, N, K):
    """The whole-tile launch (blocks 0 .. n_whole-1 through xcd_pid and
    group_tile) and the quadrant launch (block b: quadrant b % 4 of 256-tile
    n_whole + b / 4; quadrants past M or N exit) cover every 128 x 128 tile
    of the output exactly once; no quadrant launch of more than two rounds."""
    plan = quadrant_tail(M, N, K)
    if plan is None:
        pytest.skip("no quadrant tail for this shape")
    n_whole, n_tail = plan
    cdiv = lambda a, b: -(-a // b)
    tm2, tn2 = cdiv(M, 256), cdiv(N, 256)
    cover = {}
    for b in range(n_whole):
        tm, tn = group_tile(xcd_pid(n_whole, b), tm2, tn2)
        assert 0 <= tm < tm2 and 0 <= tn < tn2
        for q in range(4):
            sub = (2 * tm + q // 2, 2 * tn + q % 2)
            if sub[0] * 128 < M and sub[1] * 128 < N:
                cover[sub] = cover.get(sub, 0) + 1
    assert 4 * n_tail <= 512
    for b in range(4 * n_tail):
        tm, tn = group_tile(n_whole + b // 4, tm2, tn2)
        sub = (2 * tm + (b >> 1 & 1), 2 * tn + (b & 1))
        if sub[0] * 128 >= M or sub[1] * 128 >= N:
            continue
        cover[sub] = cover.get(sub, 0) + 1
    want = {(i, j) for i in range(cdiv(M, 128)) for j in range(cdiv(N, 128))}
    assert set(cover) == want
    assert max(cover.values()) == 1
