"""GPU parity of the attention backward pass (vt_attention_backward) against
the float64 oracle of oracle/grad.py, through the C ABI.

Tolerance: relative L2 error <= 1e-2 for each of dq, dk, dv (the bar used for
one block's output).  The kernels round q, k, v, dO, P and dS to fp16 (2^-11
relative) and accumulate in fp32, so the expected error is a few times 2^-11;
the bf16 output adds 2^-9 relative.  The library orders tokens by 2x2
windows; attention is equivariant under any permutation inside an image, so
the oracle runs in the same order with the positions permuted alike."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_f32, dev_bits, host_bits, log, rel_l2, rng, window_to_raster
from oracle import grad as G

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

H, HD = 16, 80


@pytest.fixture(scope="module")
def vt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vision_transformer_encoder_tiled_amd as m
    return m


def run_backward(vt, grids, qkv_bits, dout_bits, f32=True):
    """vt_attention_backward on window-order bf16 inputs; returns dqkv
    [N, 3, H, 80] as float32 (window order)."""
    N = qkv_bits.shape[0]
    cfg = vt.config()
    cu = torch.empty(len(grids) + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, 3), dtype=torch.int32, device="cuda")
    vt.vt_build_metadata(grids, cu, pos)
    max_seq = max(t * h * w for t, h, w in grids)
    ws = vt.workspace(vt.vt_attention_backward_workspace_size(cfg, N, len(grids), max_seq))
    dq = torch.full((N, 3, H, HD), float("nan"), dtype=torch.float32, device="cuda") if f32 else \
        torch.full((N, 3, H, HD), -1, dtype=torch.int16, device="cuda")
    vt.vt_attention_backward(cfg, dev_bits(qkv_bits, torch), cu, pos, len(grids), N, max_seq,
                             dev_bits(dout_bits, torch), dq, vt.VT_FP32 if f32 else vt.VT_BF16, ws)
    torch.cuda.synchronize()
    return dq.cpu().numpy() if f32 else bf16_f32(host_bits(dq))


def window_positions(grids):
    return oracle.positions(grids)[window_to_raster(grids)]


def random_inputs(N, seed, qk_scale=1.0):
    g = rng(seed)
    qkv = g.standard_normal((N, 3, H, HD), dtype=np.float32)
    qkv[:, :2] *= np.float32(qk_scale)
    dout = g.standard_normal((N, H * HD), dtype=np.float32)
    return synth.bf16_bits(qkv), synth.bf16_bits(dout)


def check_parts(got, want, tol, what):
    errs = [rel_l2(got[:, i], want[:, i]) for i in range(3)]
    log(f"  {what}: rel-L2 dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}")
    assert np.all(np.isfinite(got))
    assert max(errs) <= tol


@pytest.mark.parametrize("grids,seed", [
    ([(1, 12, 14)], 41),                         # 168 tokens: 2 full 64-key tiles + 40, 128-tile + 40
    ([(1, 16, 18), (1, 2, 2), (3, 4, 6)], 42),   # several items, a 4-token image, a clip
    ([(1, 2, 2)], 43),                           # one 4-token image: a single ragged tile
    ([(1, 4, 4)] * 62 + [(1, 16, 18), (1, 6, 8)], 48),  # 64 items: the 8-wavefront dK/dV pass
])
@pytest.mark.parametrize("out_dtype", ["fp32", "bf16"])
def test_attention_backward_parity(vt, grids, seed, out_dtype):
    log(f"attention backward {grids} {out_dtype}")
    N = sum(t * h * w for t, h, w in grids)
    qkv, dout = random_inputs(N, seed)
    got = run_backward(vt, grids, qkv, dout, f32=out_dtype == "fp32")
    want = G.attention_qkv_backward(bf16_f32(qkv).astype(np.float64), window_positions(grids),
                                    oracle.cu_seqlens(grids), bf16_f32(dout).astype(np.float64))
    check_parts(got, want, 1e-2, "full")


def test_attention_backward_sharp_scores(vt):
    """q, k ~ N(0, 9): peaked softmax rows (scores of std ~9)."""
    grids = [(1, 10, 12)]
    qkv, dout = random_inputs(120, 44, qk_scale=3.0)
    got = run_backward(vt, grids, qkv, dout)
    want = G.attention_qkv_backward(bf16_f32(qkv).astype(np.float64), window_positions(grids),
                                    oracle.cu_seqlens(grids), bf16_f32(dout).astype(np.float64))
    check_parts(got, want, 1e-2, "sharp")


def test_attention_backward_block0_448(vt):
    """The block-0 QKV activations of the 448x448 image (1024 tokens), whole."""
    from test_gpu_kernels import layer0_qkv_bits
    grids = [(1, 32, 32)]
    perm = window_to_raster(grids)
    qkv = layer0_qkv_bits(grids, [2])[perm].reshape(1024, 3, H, HD)
    dout = synth.bf16_bits(rng(45).standard_normal((1024, H * HD), dtype=np.float32))
    got = run_backward(vt, grids, qkv, dout)
    want = G.attention_qkv_backward(bf16_f32(qkv).astype(np.float64), window_positions(grids),
                                    oracle.cu_seqlens(grids), bf16_f32(dout).astype(np.float64))
    check_parts(got, want, 1e-2, "block0 448")


def test_attention_backward_2016_sampled(vt):
    """One 2016x2016 image (20,736 tokens, the largest configuration): dq on
    sampled rows against the oracle row by row; dv and dk through identities
    that hold at any size -- sum over keys of dv = sum over queries of dO, and
    the keys' dk rotated forward by RoPE sum to zero -- each to 1e-2 of the
    root-sum-square of the summed gradients (the size that independent
    relative errors of 1e-2 would leave)."""
    grids = [(1, 144, 144)]
    N = 20736
    qkv, dout = random_inputs(N, 46)
    got = run_backward(vt, grids, qkv, dout)
    pos = window_positions(grids)
    x = bf16_f32(qkv).astype(np.float64)
    d = bf16_f32(dout).astype(np.float64)
    rows = np.unique(np.r_[0:16, N - 16:N, rng(47).integers(0, N, 160)])
    want_q = G.attention_dq_rows(x, pos, oracle.cu_seqlens(grids), d, rows)
    e = rel_l2(got[rows, 0], want_q)
    log(f"  2016 sampled dq rel-L2 {e:.2e}")
    assert e <= 1e-2
    dv = got[:, 2].astype(np.float64)
    s_err = np.linalg.norm(dv.sum(0) - d.reshape(N, H, HD).sum(0))
    rss = np.sqrt((dv ** 2).sum())
    log(f"  dv sum error {s_err:.3e} (rss {rss:.3e})")
    assert s_err <= 1e-2 * rss
    axis, inv = oracle.rope_tables()
    dk_rot = oracle.apply_rope(got[:, 1].astype(np.float64), pos, axis, inv)
    k_sum = np.linalg.norm(dk_rot.sum(0))
    rss_k = np.sqrt((dk_rot ** 2).sum())
    log(f"  rotated dk sum {k_sum:.3e} (rss {rss_k:.3e})")
    assert k_sum <= 1e-2 * rss_k


# ---------------------------------------------------------------- one block
GRAD_NAMES = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g", "ln2_b", "w_fc1", "b_fc1",
              "w_fc2", "b_fc2")


def block_backward_case(vt, grids, R, dR2, affine, seed=0):
    """vt_block_backward on window-order fp32 R and dL/d(output); returns
    (dR, grads) from the GPU and from the float64 oracle."""
    N = R.shape[0]
    W = synth.make_weights(1, projector=False, affine=affine)
    cfg = vt.config(layers=1)
    dw = {k: dev_bits(v, torch) for k, v in W.items()}
    bw = vt.block_weights(dw, "l0.")
    cu = torch.empty(len(grids) + 1, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, 3), dtype=torch.int32, device="cuda")
    vt.vt_build_metadata(grids, cu, pos)
    max_seq = max(t * h * w for t, h, w in grids)
    ws = vt.workspace(vt.vt_block_backward_workspace_size(cfg, N, len(grids), max_seq))
    shapes = {k[3:]: v.shape for k, v in W.items() if k.startswith("l0.")}
    gd = {n: torch.full(shapes[n], float("nan"), dtype=torch.float32, device="cuda") for n in GRAD_NAMES}
    Rd = torch.from_numpy(R).cuda()
    dRd = torch.from_numpy(dR2.copy()).cuda()
    vt.vt_block_backward(cfg, Rd, bw, cu, pos, len(grids), N, max_seq, dRd, vt.block_grads(gd), ws)
    torch.cuda.synchronize()
    assert np.array_equal(Rd.cpu().numpy(), R)                      # the input is not modified
    got = {n: t.cpu().numpy() for n, t in gd.items()}
    Wf = {k: v.astype(np.float64) for k, v in oracle.weights_f32(W).items()}
    want_dR, want = G.block_backward(R.astype(np.float64), Wf, window_positions(grids),
                                     oracle.cu_seqlens(grids), oracle.Config(),
                                     dR2.astype(np.float64), prefix="l0.")
    return dRd.cpu().numpy(), got, want_dR, want


def check_block(got_dR, got, want_dR, want, what):
    errs = {n: rel_l2(got[n], want[n]) for n in GRAD_NAMES}
    e = rel_l2(got_dR, want_dR)
    log(f"  {what}: dR rel-L2 {e:.2e}; " + " ".join(f"{n} {v:.1e}" for n, v in errs.items()))
    assert np.all(np.isfinite(got_dR)) and all(np.all(np.isfinite(g)) for g in got.values())
    assert e <= 1e-2
    assert max(errs.values()) <= 1e-2


@pytest.mark.parametrize("affine", ["canonical", "random"])
def test_block_backward_224(vt, affine):
    """One block on the 224x224 image's patch embedding, random dL/d(output)."""
    log(f"block backward 224 {affine}")
    wl = synth.WORKLOADS["block_224"]
    W = synth.make_weights(1, projector=False, affine=affine)
    px = synth.make_batch_pixels(wl)
    R0 = oracle.patch_embed(oracle.split_pixels(bf16_f32(px), wl.grids), oracle.weights_f32(W),
                            wl.grids).astype(np.float32)
    perm = window_to_raster(wl.grids)
    R = np.ascontiguousarray(R0[perm])
    dR2 = rng(50).standard_normal(R.shape, dtype=np.float32)
    check_block(*block_backward_case(vt, list(wl.grids), R, dR2, affine), "224")


def test_block_backward_ragged_images(vt):
    """Two images (168 + 4 tokens: the transposed token dimension padded to
    192), random residual stream and dL/d(output)."""
    grids = [(1, 12, 14), (1, 2, 2)]
    N = 172
    R = rng(51).standard_normal((N, 1280), dtype=np.float32)
    dR2 = rng(52).standard_normal((N, 1280), dtype=np.float32)
    check_block(*block_backward_case(vt, grids, R, dR2, "random"), "ragged")


# ---------------------------------------------------------------- the tower
def tower_backward_case(vt, grids, seeds, n_layers, d_tower, affine="random", progress=None):
    """vt_tower_backward (n_layers blocks) on seeded items and dL/d(tower
    output) (raster order); returns (gpu grads, oracle grads), keyed like the
    oracle's."""
    W = synth.make_weights(n_layers, projector=False, affine=affine)
    px = np.concatenate([(synth.make_pixels(h, w, s) if t == 1 else synth.make_clip(t, h, w, s)).reshape(-1)
                         for (t, h, w), s in zip(grids, seeds)])
    cfg = vt.config(layers=n_layers)
    dw = {k: dev_bits(v, torch) for k, v in W.items()}
    tw = vt.TowerWeights(dw, n_layers)
    gd = {k: torch.full(v.shape, float("nan"), dtype=torch.float32, device="cuda") for k, v in W.items()}
    tg = vt.TowerGrads(gd, n_layers)
    ws = vt.workspace(vt.vt_tower_backward_workspace_size(cfg, grids))
    vt.vt_tower_backward(cfg, dev_bits(px, torch), grids, tw, torch.from_numpy(d_tower).cuda(), tg, ws)
    torch.cuda.synchronize()
    got = {k: t.cpu().numpy() for k, t in gd.items()}
    Wf = {k: v.astype(np.float64) for k, v in oracle.weights_f32(W).items()}
    imgs = [x.astype(np.float64) for x in oracle.split_pixels(bf16_f32(px), grids)]
    want = G.tower_backward(imgs, grids, Wf, oracle.Config(), n_layers, d_tower.astype(np.float64),
                            progress=progress)
    return got, want


def check_tower(got, want, what, tol=1e-2):
    errs = {k: rel_l2(got[k], want[k]) for k in want}
    worst = max(errs, key=errs.get)
    log(f"  {what}: patch_w {errs['patch_w']:.1e} patch_b {errs['patch_b']:.1e}; worst {worst} {errs[worst]:.1e}")
    assert all(np.all(np.isfinite(got[k])) for k in want)
    assert errs[worst] <= tol


def test_tower_backward_two_layers(vt):
    """Two blocks over two items (224x224 and a 6x8-patch image), random
    dL/d(tower output): every parameter gradient of both blocks and of the
    patch embed."""
    grids = [(1, 16, 16), (1, 6, 8)]
    N = 256 + 48
    dT = rng(53).standard_normal((N, 1280), dtype=np.float32)
    check_tower(*tower_backward_case(vt, grids, [1, 7], 2, dT), "2 layers")


def test_tower_backward_clip(vt):
    """A 4-frame clip (t = 2, the temporal RoPE pairs rotate) beside a still
    image, two blocks: every gradient against the oracle."""
    grids = [(2, 6, 8), (1, 4, 6)]
    N = 96 + 24
    dT = rng(58).standard_normal((N, 1280), dtype=np.float32)
    check_tower(*tower_backward_case(vt, grids, [8, 9], 2, dT), "clip 2 layers")


def test_attention_backward_many_items(vt):
    """300 small items (4 and 8 tokens), so the schedule spans several
    metadata chunks and many one-tile images."""
    grids = [(1, 2, 2) if i % 3 else (1, 2, 4) for i in range(300)]
    N = sum(t * h * w for t, h, w in grids)
    qkv, dout = random_inputs(N, 59)
    got = run_backward(vt, grids, qkv, dout)
    want = G.attention_qkv_backward(bf16_f32(qkv).astype(np.float64), window_positions(grids),
                                    oracle.cu_seqlens(grids), bf16_f32(dout).astype(np.float64))
    check_parts(got, want, 1e-2, f"{len(grids)} items")


def test_tower_backward_mean_pool_probe(vt):
    """The pages' probe (mean-pool the tower output, then a backward pass) on
    a 4-layer tower of one 224x224 image, with the loss sum over features of
    the pooled feature: dL/d(token) = 1/n for every token and feature.  The
    gradient norm over all parameters is compared with the oracle's."""
    grids = [(1, 16, 16)]
    dT = np.full((256, 1280), 1.0 / 256, np.float32)
    got, want = tower_backward_case(vt, grids, [1], 4, dT, affine="canonical")
    check_tower(got, want, "probe 4 layers")
    g_gpu = np.sqrt(sum(float((got[k].astype(np.float64) ** 2).sum()) for k in want))
    g_ref = np.sqrt(sum(float((want[k] ** 2).sum()) for k in want))
    log(f"  grad_l2 {g_gpu:.6g} (oracle {g_ref:.6g})")
    assert abs(g_gpu - g_ref) <= 1e-2 * g_ref


def test_block_backward_is_reproducible(vt):
    """Two calls on the same inputs give bitwise-equal gradients: every sum
    (split-K, bias and LayerNorm gradients) runs in a fixed order, with no
    atomics."""
    grids = [(1, 12, 14), (1, 2, 2)]
    N = 172
    W = synth.make_weights(1, projector=False, affine="random")
    cfg = vt.config(layers=1)
    bw = vt.block_weights({k: dev_bits(v, torch) for k, v in W.items()}, "l0.")
    cu = torch.empty(3, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, 3), dtype=torch.int32, device="cuda")
    vt.vt_build_metadata(grids, cu, pos)
    ws = vt.workspace(vt.vt_block_backward_workspace_size(cfg, N, 2, 168))
    R = torch.from_numpy(rng(54).standard_normal((N, 1280), dtype=np.float32)).cuda()
    dR0 = torch.from_numpy(rng(55).standard_normal((N, 1280), dtype=np.float32)).cuda()
    runs = []
    for _ in range(2):
        gd = {k[3:]: torch.empty(v.shape, dtype=torch.float32, device="cuda")
              for k, v in W.items() if k.startswith("l0.")}
        dR = dR0.clone()
        vt.vt_block_backward(cfg, R, bw, cu, pos, 2, N, 168, dR, vt.block_grads(gd), ws)
        torch.cuda.synchronize()
        runs.append({"dR": dR.cpu().numpy(), **{k: t.cpu().numpy() for k, t in gd.items()}})
    diff = {k: float(np.max(np.abs(runs[0][k] - runs[1][k]))) for k in runs[0]
            if not np.array_equal(runs[0][k], runs[1][k])}
    log(f"  differing outputs: {diff}")
    assert not diff


def test_block_backward_partial_gradients(vt):
    """Gradients left NULL are not formed; the others are unchanged by it."""
    grids = [(1, 16, 16)]
    N = 256
    W = synth.make_weights(1, projector=False, affine="random")
    cfg = vt.config(layers=1)
    bw = vt.block_weights({k: dev_bits(v, torch) for k, v in W.items()}, "l0.")
    cu = torch.empty(2, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, 3), dtype=torch.int32, device="cuda")
    vt.vt_build_metadata(grids, cu, pos)
    ws = vt.workspace(vt.vt_block_backward_workspace_size(cfg, N, 1, N))
    R = torch.from_numpy(rng(56).standard_normal((N, 1280), dtype=np.float32)).cuda()
    dR0 = torch.from_numpy(rng(57).standard_normal((N, 1280), dtype=np.float32)).cuda()
    full = {k[3:]: torch.empty(v.shape, dtype=torch.float32, device="cuda") for k, v in W.items()
            if k.startswith("l0.")}
    dR_full = dR0.clone()
    vt.vt_block_backward(cfg, R, bw, cu, pos, 1, N, N, dR_full, vt.block_grads(full), ws)
    some = {k: torch.full_like(full[k], 7.0) for k in ("w_o", "b_fc1", "ln1_g")}
    dR_some = dR0.clone()
    vt.vt_block_backward(cfg, R, bw, cu, pos, 1, N, N, dR_some, vt.block_grads(some), ws)
    torch.cuda.synchronize()
    assert torch.equal(dR_full, dR_some)
    for k, t in some.items():
        assert torch.equal(t, full[k]), k


def test_tower_backward_448_full(vt):
    """The configuration bench.py times: the whole 32-layer tower on the
    448x448 image (1,024 tokens) under the mean-pool probe, every one of the
    386 gradients and the gradient norm against the float64 oracle (about a
    minute of host time; progress is logged every 8 blocks)."""
    grids = [(1, 32, 32)]
    dT = np.full((1024, 1280), 1.0 / 1024, np.float32)
    got, want = tower_backward_case(vt, grids, [2], 32, dT, affine="canonical",
                                    progress=lambda i: i % 8 == 0 and log(f"  oracle block {i} done"))
    check_tower(got, want, "448 32 layers")
    g_gpu = np.sqrt(sum(float((got[k].astype(np.float64) ** 2).sum()) for k in want))
    g_ref = np.sqrt(sum(float((want[k] ** 2).sum()) for k in want))
    log(f"  grad_l2 {g_gpu:.6g} (oracle {g_ref:.6g})")
    assert abs(g_gpu - g_ref) <= 1e-2 * g_ref
