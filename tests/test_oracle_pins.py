"""Pins of the CPU oracle against things other than itself.

Each test names what fixes the expected value: a brute-force float64
computation written independently, a library routine (torch CPU float64), a
closed form, an invariant, or a value printed on the pages.  Runs on CPU.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = np.float64


def tiny_cfg(**kw):
    base = dict(hidden=32, heads=2, head_dim=16, mlp=64, layers=2, proj=24,
                rope_sections=(2, 3, 3))
    base.update(kw)
    return oracle.Config(**base)


def rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- bf16 decode
def test_bf16_decode_known_bit_patterns():
    # IEEE-754 binary32 values of the bf16 patterns (high half of the word).
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0000, 0x8000, 0x7F80, 0x0001, 0x3E80], np.uint16)
    want = [1.0, -2.0, 3.140625, 0.0, -0.0, math.inf, 2.0 ** -133, 0.25]
    got = oracle.bf16_to_f32(bits)
    assert [float(x) for x in got] == want
    assert np.signbit(got[4])


def test_bf16_round_nearest_even_in_the_input_generator():
    # 1 + 2^-8 lies half way between bf16 1.0 and 1.0078125: ties go to the even mantissa.
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -1.5], np.float32)
    assert [int(b) for b in synth.bf16_bits(x)] == [0x3F80, 0x3F82, 0x3F81, 0xBFC0]
    v = rng(1).standard_normal(10000).astype(np.float32)
    back = oracle.bf16_to_f32(synth.bf16_bits(v))
    assert np.all(np.abs(back - v) <= np.abs(v) * 2.0 ** -8)


# ---------------------------------------------------------------- metadata
def test_cu_seqlens_and_positions_closed_form():
    grids = [(1, 4, 6), (1, 2, 2), (1, 6, 2)]
    cu = oracle.cu_seqlens(grids)
    assert list(cu) == [0, 24, 28, 40]
    pos = oracle.positions(grids)
    for i, (t, h, w) in enumerate(grids):
        for j in range(h * w):
            assert tuple(pos[cu[i] + j]) == (0, j // w, j % w)


def test_merge_map_is_a_bijection_of_2x2_blocks():
    grids = [(1, 4, 6), (1, 2, 2), (1, 6, 8)]
    mm = oracle.merge_map(grids)
    N = sum(h * w for _, h, w in grids)
    assert mm.shape == (N // 4, 4)
    assert sorted(mm.reshape(-1).tolist()) == list(range(N))
    pos = oracle.positions(grids)
    for m in range(mm.shape[0]):
        p = pos[mm[m]]
        r0, c0 = p[0, 1], p[0, 2]
        assert r0 % 2 == 0 and c0 % 2 == 0
        for k in range(4):  # slot k = 2*dr + dc
            assert tuple(p[k, 1:]) == (r0 + k // 2, c0 + k % 2)


def test_positions_and_merge_map_for_clips():
    # a clip with t = 3 temporal patches next to a still image
    grids = [(3, 2, 4), (1, 2, 2)]
    cu = oracle.cu_seqlens(grids)
    assert list(cu) == [0, 24, 28]
    pos = oracle.positions(grids)
    for j in range(24):
        assert tuple(pos[j]) == (j // 8, (j % 8) // 4, j % 4)
    mm = oracle.merge_map(grids)
    assert mm.shape == (7, 4)
    assert sorted(mm.reshape(-1).tolist()) == list(range(28))
    for m in range(7):
        p = pos[mm[m]]
        assert len(set(p[:, 0].tolist())) == 1  # the merge never crosses temporal patches
        for k in range(4):
            assert tuple(p[k, 1:]) == (p[0, 1] + k // 2, p[0, 2] + k % 2)


# ---------------------------------------------------------------- patchify / embed
def test_patchify_roundtrip_bit_exact():
    img = synth.make_pixels(6, 4, seed=7)
    x = oracle.patchify(img)
    assert x.shape == (24, 1176)
    assert np.array_equal(oracle.unpatchify(x, 6, 4), img)
    # the duplicated frame: tau = 0 and tau = 1 slices are identical
    x6 = x.reshape(24, 3, 2, 14, 14)
    assert np.array_equal(x6[:, :, 0], x6[:, :, 1])


def test_patch_embed_equals_direct_conv3d_loops():
    # Conv3d with kernel = stride = (2, 14, 14) over a 2-frame clip made of the
    # repeated frame, evaluated by explicit float64 loops.
    h, w, co = 2, 3, 4
    img = oracle.bf16_to_f32(synth.make_pixels(h, w, seed=3)).astype(F64)
    W5 = rng(2).standard_normal((co, 3, 2, 14, 14))
    b = rng(3).standard_normal(co)
    clip = np.stack([img, img], axis=1)  # [3, 2, H, W]
    direct = np.zeros((h * w, co))
    for o in range(co):
        for r in range(h):
            for c in range(w):
                acc = b[o]
                for ch in range(3):
                    for tau in range(2):
                        blk = clip[ch, tau, 14 * r:14 * r + 14, 14 * c:14 * c + 14]
                        acc += float(np.sum(W5[o, ch, tau] * blk))
                direct[r * w + c, o] = acc
    got = oracle.linear(oracle.patchify(img), W5.reshape(co, -1), b)
    np.testing.assert_allclose(got, direct, rtol=1e-12, atol=1e-12)
    # special case: a repeated frame makes the Conv3d a Conv2d with W[:,:,0] + W[:,:,1]
    conv2d = torch.nn.functional.conv2d(torch.from_numpy(img)[None],
                                        torch.from_numpy(W5[:, :, 0] + W5[:, :, 1]),
                                        torch.from_numpy(b), stride=14)[0]
    np.testing.assert_allclose(got, conv2d.permute(1, 2, 0).reshape(h * w, co).numpy(),
                               rtol=1e-12, atol=1e-12)


def test_clip_patch_embed_equals_direct_conv3d_loops():
    # Conv3d with kernel = stride = (2, 14, 14) over a 4-frame clip (t = 2),
    # explicit float64 loops; temporal patch tt covers frames 2tt, 2tt+1.
    t, h, w, co = 2, 2, 2, 3
    clip = oracle.bf16_to_f32(synth.make_clip(t, h, w, seed=5)).astype(F64)  # [4, 3, H, W]
    W5 = rng(4).standard_normal((co, 3, 2, 14, 14))
    b = rng(5).standard_normal(co)
    direct = np.zeros((t * h * w, co))
    for o in range(co):
        for tt in range(t):
            for r in range(h):
                for c in range(w):
                    acc = b[o]
                    for ch in range(3):
                        for tau in range(2):
                            blk = clip[2 * tt + tau, ch, 14 * r:14 * r + 14, 14 * c:14 * c + 14]
                            acc += float(np.sum(W5[o, ch, tau] * blk))
                    direct[(tt * h + r) * w + c, o] = acc
    got = oracle.linear(oracle.patchify(clip), W5.reshape(co, -1), b)
    np.testing.assert_allclose(got, direct, rtol=1e-12, atol=1e-12)
    # a 2-frame clip of one repeated frame is the still image
    img = synth.make_pixels(h, w, seed=6)
    assert np.array_equal(oracle.patchify(np.stack([img, img])), oracle.patchify(img))
    # flat split: a still image then a clip
    flat = np.concatenate([img.reshape(-1), synth.make_clip(t, h, w, seed=5).reshape(-1)])
    parts = oracle.split_pixels(flat, [(1, h, w), (t, h, w)])
    assert parts[0].shape == img.shape and parts[1].shape == (4, 3, 14 * h, 14 * w)


# ---------------------------------------------------------------- basic ops
def test_linear_is_out_by_in():
    x = rng(4).standard_normal((3, 5))
    W = rng(5).standard_normal((7, 5))
    b = rng(6).standard_normal(7)
    want = np.array([[sum(W[o, i] * x[n, i] for i in range(5)) + b[o] for o in range(7)]
                     for n in range(3)])
    np.testing.assert_allclose(oracle.linear(x, W, b), want, rtol=1e-13)


def test_layer_norm_against_torch_and_moments():
    x = rng(7).standard_normal((9, 1280)) * 3 + 1.5
    g = rng(8).standard_normal(1280)
    b = rng(9).standard_normal(1280)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (1280,), torch.from_numpy(g),
                                          torch.from_numpy(b), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.layer_norm(x, g, b, 1e-6), want, rtol=1e-10, atol=1e-12)
    y = oracle.layer_norm(x, np.ones(1280), np.zeros(1280), 1e-6)
    np.testing.assert_allclose(y.mean(-1), 0, atol=1e-12)
    np.testing.assert_allclose((y * y).mean(-1), 1.0 / (1.0 + 1e-6 / x.var(-1)), rtol=1e-12)


def test_gelu_forms():
    x = np.linspace(-8, 8, 2001)
    want_t = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    want_e = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(x), want_t, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(oracle.gelu_erf(x), want_e, rtol=1e-12, atol=1e-15)
    assert oracle.gelu_erf(np.array([1.0]))[0] == pytest.approx(0.8413447460685429, abs=1e-15)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    # the two forms differ by at most ~4.7e-4 (tanh-approximation error)
    assert np.max(np.abs(oracle.gelu_tanh(x) - oracle.gelu_erf(x))) < 5e-4


# ---------------------------------------------------------------- RoPE
def test_rope_frequency_ladder_values():
    axis, inv = oracle.rope_tables(80, (8, 16, 16), 10000.0)
    assert list(axis[:8]) == [0] * 8 and list(axis[8:24]) == [1] * 16 and list(axis[24:]) == [2] * 16
    # per-axis ladder: pair k of an axis with n pairs turns at 10000^(-k/n)
    assert inv[0] == 1.0 and inv[8] == 1.0 and inv[24] == 1.0
    assert inv[1] == pytest.approx(10000 ** (-1 / 8), rel=1e-15)
    assert inv[9] == pytest.approx(0.5623413251903491, rel=1e-15)
    assert inv[39] == pytest.approx(10000 ** (-15 / 16), rel=1e-15)
    _, shared = oracle.rope_tables(80, (8, 16, 16), 10000.0, shared_ladder=True)
    assert shared[39] == pytest.approx(10000 ** (-78 / 80), rel=1e-15)


def test_rope_identity_at_origin_and_norm_preserving():
    x = rng(10).standard_normal((5, 16, 80))
    axis, inv = oracle.rope_tables()
    assert np.array_equal(oracle.apply_rope(x, np.zeros((5, 3), np.int32), axis, inv), x)
    pos = rng(11).integers(0, 150, size=(5, 3)).astype(np.int32)
    y = oracle.apply_rope(x, pos, axis, inv)
    # each (j, j+40) pair keeps its length
    np.testing.assert_allclose(y[..., :40] ** 2 + y[..., 40:] ** 2,
                               x[..., :40] ** 2 + x[..., 40:] ** 2, rtol=1e-12)


def test_rope_is_a_complex_rotation():
    # Independent form: z_j = x_j + i x_{j+40} is multiplied by exp(i * pos[axis_j] * f_j).
    x = rng(12).standard_normal((4, 2, 80))
    pos = np.array([[0, 3, 7], [0, 0, 1], [0, 95, 2], [0, 11, 143]], np.int32)
    axis, inv = oracle.rope_tables()
    z = x[..., :40] + 1j * x[..., 40:]
    rot = z * np.exp(1j * pos[:, axis][:, None, :] * inv[None, None, :])
    y = oracle.apply_rope(x, pos, axis, inv)
    np.testing.assert_allclose(y[..., :40], rot.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[..., 40:], rot.imag, rtol=1e-12, atol=1e-12)


def test_rope_scores_depend_only_on_relative_offset():
    axis, inv = oracle.rope_tables()
    q = rng(13).standard_normal((1, 1, 80))
    k = rng(14).standard_normal((1, 1, 80))
    p1, p2 = np.array([[0, 5, 9]], np.int32), np.array([[0, 2, 30]], np.int32)
    base = float(np.sum(oracle.apply_rope(q, p1, axis, inv) * oracle.apply_rope(k, p2, axis, inv)))
    for shift in ([0, 7, 3], [4, 1, 100], [2, 40, 0]):
        s = np.array([shift], np.int32)
        v = float(np.sum(oracle.apply_rope(q, p1 + s, axis, inv) * oracle.apply_rope(k, p2 + s, axis, inv)))
        assert v == pytest.approx(base, rel=1e-10, abs=1e-10)
    # changing the offset does change the score
    v = float(np.sum(oracle.apply_rope(q, p1, axis, inv) * oracle.apply_rope(k, p1, axis, inv)))
    assert abs(v - base) > 1e-3


def test_rope_t_zero_leaves_temporal_pairs_unrotated():
    axis, inv = oracle.rope_tables()
    x = rng(15).standard_normal((3, 2, 80))
    pos = np.array([[0, 4, 5], [0, 17, 1], [0, 0, 60]], np.int32)
    y = oracle.apply_rope(x, pos, axis, inv)
    idx = np.r_[0:8, 40:48]
    assert np.array_equal(y[..., idx], x[..., idx])


# ---------------------------------------------------------------- attention
def brute_force_attention(q, k, v, scale):
    """Explicit [n, n] score matrix per head, float64, one element at a time."""
    n, H, hd = q.shape
    out = np.zeros_like(q)
    for h in range(H):
        S = np.array([[sum(q[i, h, d] * k[j, h, d] for d in range(hd)) * scale
                       for j in range(n)] for i in range(n)])
        for i in range(n):
            m = max(S[i])
            e = [math.exp(s - m) for s in S[i]]
            tot = sum(e)
            for d in range(hd):
                out[i, h, d] = sum(e[j] * v[j, h, d] for j in range(n)) / tot
    return out


def test_attention_matches_brute_force_and_torch_sdpa():
    n, H, hd = 11, 2, 8
    q, k, v = (rng(s).standard_normal((n, H, hd)) for s in (20, 21, 22))
    got = oracle.attention_image(q, k, v, chunk=4)
    np.testing.assert_allclose(got, brute_force_attention(q, k, v, 1 / math.sqrt(hd)),
                               rtol=1e-12, atol=1e-12)
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    sdpa = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0].permute(1, 0, 2)
    np.testing.assert_allclose(got, sdpa.numpy(), rtol=1e-12, atol=1e-12)
    # the fp32 oracle agrees with the float64 brute force to fp32 rounding
    got32 = oracle.attention_image(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32))
    np.testing.assert_allclose(got32, got, rtol=0, atol=2e-6)


def test_online_softmax_equals_plain_softmax():
    # The tiled kernel's algorithm (running max m, running sum l, rescaled
    # accumulator), written here in float64 over tiles of 5 keys, reaches the
    # same result as the oracle's full-row softmax.
    n, hd = 23, 6
    q = rng(30).standard_normal((n, 1, hd)) * 3
    k = rng(31).standard_normal((n, 1, hd)) * 3
    v = rng(32).standard_normal((n, 1, hd))
    scale = 1 / math.sqrt(hd)
    out = np.zeros((n, hd))
    for i in range(n):
        m, l, acc = -math.inf, 0.0, np.zeros(hd)
        for j0 in range(0, n, 5):
            s = [float(q[i, 0] @ k[j, 0]) * scale for j in range(j0, min(n, j0 + 5))]
            m_new = max(m, max(s))
            corr = math.exp(m - m_new)
            p = [math.exp(x - m_new) for x in s]
            l = l * corr + sum(p)
            acc = acc * corr + sum(pj * v[j0 + t, 0] for t, pj in enumerate(p))
            m = m_new
        out[i] = acc / l
    np.testing.assert_allclose(out, oracle.attention_image(q, k, v)[:, 0], rtol=1e-12, atol=1e-13)


def test_attention_invariants():
    n, H, hd = 17, 3, 8
    q, k = rng(40).standard_normal((n, H, hd)), rng(41).standard_normal((n, H, hd))
    p = oracle.softmax_rows(rng(42).standard_normal((5, 9)) * 10)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-14)
    cv = np.broadcast_to(rng(43).standard_normal((1, H, hd)), (n, H, hd)).copy()
    np.testing.assert_allclose(oracle.attention_image(q, k, cv), cv, rtol=1e-13)   # constant V -> V
    v = rng(44).standard_normal((n, H, hd))
    zq = np.zeros_like(q)
    np.testing.assert_allclose(oracle.attention_image(zq, k, v),                  # Q = 0 -> mean of V
                               np.broadcast_to(v.mean(0), v.shape), rtol=1e-12, atol=1e-14)
    one = oracle.attention_image(q[:1], k[:1], v[:1])                              # one key -> its value
    np.testing.assert_allclose(one, v[:1], rtol=1e-14)


def test_varlen_is_each_image_alone():
    grids = [(1, 2, 4), (1, 4, 4), (1, 2, 2)]
    cu = oracle.cu_seqlens(grids)
    N = cu[-1]
    q, k, v = (rng(s).standard_normal((N, 2, 8)) for s in (50, 51, 52))
    packed = oracle.attention_varlen(q, k, v, cu)
    for i in range(len(grids)):
        a, b = cu[i], cu[i + 1]
        np.testing.assert_allclose(packed[a:b], brute_force_attention(q[a:b], k[a:b], v[a:b],
                                                                      1 / math.sqrt(8)),
                                   rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- block
def tiny_weights(cfg, n_layers=1, seed=60, random_affine=True):
    g = rng(seed)
    d, m, p = cfg.hidden, cfg.mlp, cfg.proj
    W = {"patch_w": g.standard_normal((d, 1176)) * 0.02, "patch_b": g.standard_normal(d) * 0.02}
    for i in range(n_layers):
        for name, shape in synth.block_shapes(d, m).items():
            if name.endswith("_g"):
                W[f"l{i}.{name}"] = 1 + 0.1 * g.standard_normal(shape) if random_affine else np.ones(shape)
            elif name.startswith("w_"):
                W[f"l{i}.{name}"] = g.standard_normal(shape) * 0.2
            else:
                W[f"l{i}.{name}"] = g.standard_normal(shape) * 0.1 if random_affine else np.zeros(shape)
    for name, shape in synth.proj_shapes(d, p).items():
        W[name] = g.standard_normal(shape) * (0.2 if name.startswith("p_w") else 0.1)
    return W


def test_block_with_zeroed_output_projections_keeps_the_residual():
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    W["l0.w_o"][:] = 0
    W["l0.w_fc2"][:] = 0
    grids = [(1, 2, 4)]
    R = rng(61).standard_normal((8, cfg.hidden))
    out = oracle.block_forward(R, W, oracle.positions(grids), oracle.cu_seqlens(grids), cfg)
    np.testing.assert_allclose(out, R + W["l0.b_o"] + W["l0.b_fc2"], rtol=1e-14, atol=1e-14)


def test_block_uniform_attention_closed_form():
    # With the Q and K rows of W_qkv (and their biases) zero, every score is 0,
    # attention is the per-image mean of V, and with the MLP output zeroed the
    # block is R + mean(V) W_o^T + b_o.  V = LN1(R) W_v^T + b_v uses the third
    # block of W_qkv rows.  Written with torch float64 modules.
    cfg = tiny_cfg()
    d = cfg.hidden
    W = tiny_weights(cfg)
    W["l0.w_qkv"][:2 * d] = 0
    W["l0.b_qkv"][:2 * d] = 0
    W["l0.w_fc2"][:] = 0
    W["l0.b_fc2"][:] = 0
    grids = [(1, 2, 2), (1, 2, 4)]
    cu = oracle.cu_seqlens(grids)
    R = rng(62).standard_normal((12, d)) * 2
    out = oracle.block_forward(R, W, oracle.positions(grids), cu, cfg)
    T = lambda a: torch.from_numpy(np.asarray(a))
    x = torch.nn.functional.layer_norm(T(R), (d,), T(W["l0.ln1_g"]), T(W["l0.ln1_b"]), eps=cfg.ln_eps)
    V = torch.nn.functional.linear(x, T(W["l0.w_qkv"][2 * d:]), T(W["l0.b_qkv"][2 * d:]))
    A = torch.cat([V[cu[i]:cu[i + 1]].mean(0, keepdim=True).expand(cu[i + 1] - cu[i], d)
                   for i in range(2)])
    want = T(R) + torch.nn.functional.linear(A, T(W["l0.w_o"]), T(W["l0.b_o"]))
    np.testing.assert_allclose(out, want.numpy(), rtol=1e-12, atol=1e-12)


def test_block_token_permutation_equivariance():
    # Shuffling tokens together with their positions shuffles the output.
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    grids = [(1, 4, 4)]
    pos, cu = oracle.positions(grids), oracle.cu_seqlens(grids)
    R = rng(63).standard_normal((16, cfg.hidden))
    perm = rng(64).permutation(16)
    a = oracle.block_forward(R, W, pos, cu, cfg)
    b = oracle.block_forward(R[perm], W, pos[perm], cu, cfg)
    np.testing.assert_allclose(b, a[perm], rtol=1e-12, atol=1e-12)
    # but moving tokens without their positions changes it (RoPE is in the path)
    c = oracle.block_forward(R[perm], W, pos, cu, cfg)
    assert np.max(np.abs(c - a[perm])) > 1e-6


def test_single_token_image_attention_is_its_value():
    # n = 1: softmax weight 1, so the attention output is V exactly (no RoPE on V).
    cfg = tiny_cfg()
    d = cfg.hidden
    W = tiny_weights(cfg)
    W["l0.w_fc2"][:] = 0
    W["l0.b_fc2"][:] = 0
    pos = np.array([[0, 7, 3]], np.int32)
    R = rng(65).standard_normal((1, d))
    out = oracle.block_forward(R, W, pos, np.array([0, 1]), cfg)
    x = oracle.layer_norm(R, W["l0.ln1_g"], W["l0.ln1_b"], cfg.ln_eps)
    v = x @ W["l0.w_qkv"][2 * d:].T + W["l0.b_qkv"][2 * d:]
    np.testing.assert_allclose(out, R + v @ W["l0.w_o"].T + W["l0.b_o"], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- projector
def test_projector_mlp_then_gather_equals_blockwise():
    cfg = tiny_cfg()
    W = tiny_weights(cfg)
    grids = [(1, 2, 4), (1, 4, 2)]
    N = 16
    T = rng(70).standard_normal((N, cfg.hidden))
    got = oracle.projector(T, W, grids, cfg)
    # gather first, then run the first MLP on each of the four slots of a merged token
    mm = oracle.merge_map(grids)
    P = cfg.proj
    want = []
    for m in range(mm.shape[0]):
        parts = []
        for k in range(4):
            t = T[mm[m, k]]
            y = torch.nn.functional.gelu(torch.from_numpy(t @ W["p_w1"].T + W["p_b1"]), approximate="tanh")
            parts.append(y.numpy() @ W["p_w2"].T + W["p_b2"])
        z = np.concatenate(parts)
        assert z.shape == (4 * P,)
        u = torch.nn.functional.gelu(torch.from_numpy(z @ W["p_w3"].T + W["p_b3"]), approximate="tanh")
        want.append(u.numpy() @ W["p_w4"].T + W["p_b4"])
    np.testing.assert_allclose(got, np.array(want), rtol=1e-12, atol=1e-12)


@pytest.mark.slow
def test_output_widths_printed_on_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "pages_shapes.json")))
    wl = synth.WORKLOADS["tower_448"]
    W = synth.make_weights(n_layers=0, projector=True)
    res = oracle.tower_forward(synth.make_batch_pixels(wl), wl.grids, W, n_layers=0)
    assert res["tower"].shape == (1024, g["image_448"]["tower_tokens_width"])
    assert res["merged_raw"].shape == (256, g["image_448"]["merged_tokens_width"])
    assert res["out"].shape == (256, g["image_448"]["projected_tokens_width"])
    pc = g["projector_config"]
    assert W["p_w1"].shape == (pc["hidden_size"], pc["input_size"])
    assert W["p_w3"].shape == (pc["output_size"], pc["merged_hidden_size"])
    # projector: 4 Linear layers, weight + bias each
    assert len(synth.PROJ_TENSORS) == g["tensor_counts"]["projector"]
    # tower: 32 blocks x 16 tensors (q, k, v kept separate) + 3 = 515
    per_block_separate_qkv = len(synth.BLOCK_TENSORS) - 2 + 6
    assert g["tower_layers"] * per_block_separate_qkv + 3 == g["tensor_counts"]["tower"]


# ---------------------------------------------------------------- mean pool
def test_mean_pool_closed_forms():
    grids = [(1, 2, 2), (2, 2, 4), (1, 4, 4)]
    N = sum(t * h * w for t, h, w in grids)
    cu = oracle.cu_seqlens(grids)
    # constant rows per item pool to that constant
    T = np.zeros((N, 8), np.float32)
    for i in range(3):
        T[cu[i]:cu[i + 1]] = i + 0.5
    assert np.array_equal(oracle.mean_pool(T, grids), np.repeat(np.arange(3) + 0.5, 8).reshape(3, 8))
    # an arithmetic ramp pools to its midpoint; shuffling rows inside an item changes nothing
    T = np.arange(N, dtype=np.float64)[:, None] * np.ones((1, 4))
    want = np.array([[(cu[i] + cu[i + 1] - 1) / 2] * 4 for i in range(3)])
    np.testing.assert_allclose(oracle.mean_pool(T, grids), want, rtol=1e-15)
    perm = np.concatenate([cu[i] + rng(i).permutation(cu[i + 1] - cu[i]) for i in range(3)])
    np.testing.assert_allclose(oracle.mean_pool(T[perm], grids), want, rtol=1e-15)


# ---------------------------------------------------------------- the whole tower
def _torch_tower_f64(px_bits, grids, w_bits, cfg, n_layers):
    """An independent float64 implementation of the whole forward pass, from
    the pages' description (MiniMax-M3-Vision README, Architecture table:
    Conv3d patch embed with temporal patch 2, pre-LN blocks with 3D RoPE,
    2x2 merge, the four-Linear projector) and torch library routines:
    conv3d with kernel = stride = (2, 14, 14) for the patch embed,
    layer_norm, scaled_dot_product_attention per item, GELU(tanh).  It
    shares no step with the oracle: bf16 decoding, pixel splitting,
    positions, RoPE angles and the 2x2 gather are written out here."""
    F = torch.nn.functional

    def dec(bits):  # bf16 bits -> float64: the 16 bits are the high half of an fp32 word
        return torch.from_numpy(bits.astype(np.int32) << 16).view(torch.float32).double()

    W = {k: dec(v) for k, v in w_bits.items()}
    pix = dec(px_bits)
    d, H, hd = cfg.hidden, cfg.heads, cfg.head_dim
    half = hd // 2
    kconv = W["patch_w"].reshape(d, 3, 2, 14, 14)
    tokens, pos, off = [], [], 0
    for t, h, w in grids:
        nf = 1 if t == 1 else 2 * t
        n = nf * 3 * 14 * h * 14 * w
        frames = pix[off:off + n].reshape(nf, 3, 14 * h, 14 * w)
        off += n
        if nf == 1:  # a still image fills the temporal patch with its one frame twice
            frames = torch.cat([frames, frames])
        y = F.conv3d(frames.permute(1, 0, 2, 3)[None], kconv, W["patch_b"], stride=(2, 14, 14))
        tokens.append(y[0].permute(1, 2, 3, 0).reshape(-1, d))  # (t, row, col) raster
        tt, rr, cc = torch.meshgrid(torch.arange(t), torch.arange(h), torch.arange(w), indexing="ij")
        pos.append(torch.stack([tt.reshape(-1), rr.reshape(-1), cc.reshape(-1)], 1))
    R = torch.cat(tokens)
    pos = torch.cat(pos).double()
    # rotation angle of pair j: the position on its axis times theta^(-k/n),
    # k = index of the pair within that axis's n pairs
    ang = torch.cat([pos[:, a:a + 1] * cfg.rope_theta ** (-torch.arange(n, dtype=torch.float64) / n)
                     for a, n in enumerate(cfg.rope_sections)], 1)[:, None, :]
    cos, sin = torch.cos(ang), torch.sin(ang)

    def rope(x):
        z = torch.complex(x[..., :half], x[..., half:]) * torch.complex(cos, sin)
        return torch.cat([z.real, z.imag], -1)

    sizes = [t * h * w for t, h, w in grids]
    layers = []
    for l in range(n_layers):
        g = lambda k: W[f"l{l}.{k}"]
        x = F.layer_norm(R, (d,), g("ln1_g"), g("ln1_b"), cfg.ln_eps)
        qkv = F.linear(x, g("w_qkv"), g("b_qkv")).reshape(-1, 3, H, hd)
        q, k, v = rope(qkv[:, 0]), rope(qkv[:, 1]), qkv[:, 2]
        att = torch.cat([F.scaled_dot_product_attention(qi.transpose(0, 1), ki.transpose(0, 1),
                                                        vi.transpose(0, 1)).transpose(0, 1)
                         for qi, ki, vi in zip(q.split(sizes), k.split(sizes), v.split(sizes))])
        R = R + F.linear(att.reshape(-1, d), g("w_o"), g("b_o"))
        y = F.layer_norm(R, (d,), g("ln2_g"), g("ln2_b"), cfg.ln_eps)
        R = R + F.linear(F.gelu(F.linear(y, g("w_fc1"), g("b_fc1")), approximate="tanh"), g("w_fc2"), g("b_fc2"))
        layers.append(R)
    Y = F.linear(F.gelu(F.linear(R, W["p_w1"], W["p_b1"]), approximate="tanh"), W["p_w2"], W["p_b2"])
    raw, Z, base = [], [], 0
    for t, h, w in grids:
        for tt in range(t):
            for r in range(h // 2):
                for c in range(w // 2):
                    ids = [base + tt * h * w + (2 * r + dr) * w + 2 * c + dc for dr in (0, 1) for dc in (0, 1)]
                    raw.append(torch.cat([R[i] for i in ids]))
                    Z.append(torch.cat([Y[i] for i in ids]))
        base += t * h * w
    Z = torch.stack(Z)
    out = F.linear(F.gelu(F.linear(Z, W["p_w3"], W["p_b3"]), approximate="tanh"), W["p_w4"], W["p_b4"])
    return {"tower": R.numpy(), "merged_raw": torch.stack(raw).numpy(), "out": out.numpy(),
            "layers": [x.numpy() for x in layers]}


def test_tower_forward_composition_against_independent_float64():
    """oracle.tower_forward (run in float64) against the independent torch
    float64 tower above, on two still images and a clip with a 3-layer tower
    whose layers all differ: the composition (patch rows of several items
    concatenated in item order, block l reading the l-th weights, blocks in
    order, the projector on the last block's output, the 2x2 gather) agrees
    to rounding.  The same comparison fails for a tower whose first two layers
    are swapped, and for one missing its last layer."""
    cfg = tiny_cfg(layers=3)
    L = 3
    W = {k: synth.bf16_bits(v.astype(np.float32)) for k, v in tiny_weights(cfg, n_layers=L, seed=91).items()}
    grids = [(1, 4, 6), (2, 2, 4), (1, 2, 2)]
    px = np.concatenate([synth.make_pixels(4, 6, 92).reshape(-1), synth.make_clip(2, 2, 4, 93).reshape(-1),
                         synth.make_pixels(2, 2, 94).reshape(-1)])
    want = _torch_tower_f64(px, grids, W, cfg, L)
    got = oracle.tower_forward(px, grids, W, cfg, n_layers=L, keep_layers=True, dtype=np.float64)
    for key in ("tower", "merged_raw", "out"):
        np.testing.assert_allclose(got[key], want[key], rtol=1e-10, atol=1e-12, err_msg=key)
    for l in range(L):
        np.testing.assert_allclose(got["layers"][l], want["layers"][l], rtol=1e-10, atol=1e-12)
    # the fp32 default follows the same composition to fp32 rounding
    f32 = oracle.tower_forward(px, grids, W, cfg, n_layers=L)
    assert np.linalg.norm(f32["out"] - want["out"]) <= 1e-5 * np.linalg.norm(want["out"])
    # planted composition mistakes are caught
    Wsw = dict(W)
    for k in synth.BLOCK_TENSORS:
        Wsw[f"l0.{k}"], Wsw[f"l1.{k}"] = W[f"l1.{k}"], W[f"l0.{k}"]
    bad = oracle.tower_forward(px, grids, Wsw, cfg, n_layers=L, dtype=np.float64)
    assert np.linalg.norm(bad["tower"] - want["tower"]) > 1e-3 * np.linalg.norm(want["tower"])
    short = oracle.tower_forward(px, grids, W, cfg, n_layers=L - 1, dtype=np.float64)
    assert np.linalg.norm(short["out"] - want["out"]) > 1e-3 * np.linalg.norm(want["out"])
