"""Pins of the oracle's backward pass (oracle.grad): every gradient against
central finite differences of the oracle's own forward in float64, and the
whole block against torch autograd in float64 (a library routine)."""
import numpy as np
import pytest

import oracle
from oracle import grad as G

F64 = np.float64
TINY = oracle.Config(hidden=16, heads=2, head_dim=8, mlp=24, rope_sections=(2, 1, 1))


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def fd_dot(f, x, dy, dx_analytic, n_dirs=6, h=1e-6, seed=0):
    """Check <dx, e> == (f(x + h e) - f(x - h e)) . dy / 2h for random directions e."""
    g = rng(seed)
    for _ in range(n_dirs):
        e = g.standard_normal(x.shape)
        num = (np.sum(f(x + h * e) * dy) - np.sum(f(x - h * e) * dy)) / (2 * h)
        ana = np.sum(dx_analytic * e)
        assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (num, ana)


def test_linear_gelu_layernorm_gradients():
    x = rng(1).standard_normal((5, 7))
    w = rng(2).standard_normal((4, 7))
    b = rng(3).standard_normal(4)
    dy = rng(4).standard_normal((5, 4))
    dx, dw, db = G.linear_backward(x, w, dy)
    fd_dot(lambda t: oracle.linear(t, w, b), x, dy, dx)
    fd_dot(lambda t: oracle.linear(x, t, b), w, dy, dw)
    fd_dot(lambda t: oracle.linear(x, w, t), b, dy, db)
    h = rng(5).standard_normal((6, 9)) * 2
    dg = rng(6).standard_normal((6, 9))
    fd_dot(oracle.gelu_tanh, h, dg, G.gelu_tanh_backward(h, dg))
    xl = rng(7).standard_normal((4, 12)) * 3 + 1
    gam = rng(8).standard_normal(12)
    bet = rng(9).standard_normal(12)
    dyl = rng(10).standard_normal((4, 12))
    dxl, dgl, dbl = G.layer_norm_backward(xl, gam, dyl, 1e-6)
    fd_dot(lambda t: oracle.layer_norm(t, gam, bet, 1e-6), xl, dyl, dxl)
    fd_dot(lambda t: oracle.layer_norm(xl, t, bet, 1e-6), gam, dyl, dgl)
    fd_dot(lambda t: oracle.layer_norm(xl, gam, t, 1e-6), bet, dyl, dbl)


def test_rope_gradient_is_the_inverse_rotation():
    pos = np.array([[0, 1, 2], [1, 3, 0], [2, 0, 5]], dtype=np.int32)
    axis, inv = oracle.rope_tables(8, (2, 1, 1))
    x = rng(11).standard_normal((3, 2, 8))
    dy = rng(12).standard_normal((3, 2, 8))
    dx = G.rope_backward(dy, pos, axis, inv)
    fd_dot(lambda t: oracle.apply_rope(t, pos, axis, inv), x, dy, dx)
    # orthogonal: the backward undoes the forward
    np.testing.assert_allclose(G.rope_backward(oracle.apply_rope(x, pos, axis, inv), pos, axis, inv), x,
                               rtol=1e-12, atol=1e-12)


def test_attention_gradients_finite_differences():
    n, H, hd = 7, 2, 8
    q, k, v = (rng(s).standard_normal((n, H, hd)) for s in (13, 14, 15))
    do = rng(16).standard_normal((n, H, hd))
    dq, dk, dv = G.attention_image_backward(q, k, v, do)
    fd_dot(lambda t: oracle.attention_image(t, k, v), q, do, dq)
    fd_dot(lambda t: oracle.attention_image(q, t, v), k, do, dk)
    fd_dot(lambda t: oracle.attention_image(q, k, t), v, do, dv)
    # varlen = each image alone; gradients never cross images
    cu = np.array([0, 3, 7])
    q2, k2, v2, do2 = (rng(s).standard_normal((7, H, hd)) for s in (17, 18, 19, 20))
    dq2, dk2, dv2 = G.attention_varlen_backward(q2, k2, v2, do2, cu)
    a = G.attention_image_backward(q2[3:], k2[3:], v2[3:], do2[3:])
    np.testing.assert_allclose(dk2[3:], a[1], rtol=1e-12, atol=1e-12)
    # constant V: the output does not depend on q or k
    vc = np.broadcast_to(rng(21).standard_normal((1, H, hd)), (n, H, hd)).copy()
    dqc, dkc, _ = G.attention_image_backward(q, k, vc, do)
    assert np.max(np.abs(dqc)) < 1e-12 and np.max(np.abs(dkc)) < 1e-12


def test_block_gradient_finite_differences_and_autograd():
    torch = pytest.importorskip("torch")
    cfg = TINY
    grids = [(1, 2, 2), (1, 2, 4)]
    N, d = 12, cfg.hidden
    pos = oracle.positions(grids)
    cu = oracle.cu_seqlens(grids)
    g = rng(22)
    shapes = {"ln1_g": (d,), "ln1_b": (d,), "w_qkv": (3 * d, d), "b_qkv": (3 * d,), "w_o": (d, d),
              "b_o": (d,), "ln2_g": (d,), "ln2_b": (d,), "w_fc1": (cfg.mlp, d), "b_fc1": (cfg.mlp,),
              "w_fc2": (d, cfg.mlp), "b_fc2": (d,)}
    W = {"l0." + k: g.standard_normal(s) * (0.3 if k.startswith("w") else 0.1) + (1.0 if k.endswith("_g") else 0.0)
         for k, s in shapes.items()}
    R = g.standard_normal((N, d))
    dR2 = g.standard_normal((N, d))
    dR, grads = G.block_backward(R, W, pos, cu, cfg, dR2)
    f = lambda t: oracle.block_forward(t, W, pos, cu, cfg)
    fd_dot(f, R, dR2, dR, h=1e-5)
    for name in ("w_qkv", "ln2_g", "b_fc1"):
        def fw(t, name=name):
            W2 = dict(W)
            W2["l0." + name] = t
            return oracle.block_forward(R, W2, pos, cu, cfg)
        fd_dot(fw, W["l0." + name], dR2, grads[name], h=1e-5)
    # torch autograd in float64 of the same block
    T = {k: torch.tensor(v, requires_grad=True) for k, v in W.items()}
    Rt = torch.tensor(R, requires_grad=True)
    axis, inv = oracle.rope_tables(cfg.head_dim, cfg.rope_sections)
    ang = torch.tensor(pos[:, axis] * inv[None, :])
    cos, sin = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]

    def rope(x):
        x1, x2 = x[..., :4], x[..., 4:]
        return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], -1)

    ln = lambda x, a, b: torch.nn.functional.layer_norm(x, (d,), a, b, 1e-6)
    x = ln(Rt, T["l0.ln1_g"], T["l0.ln1_b"])
    qkv = (x @ T["l0.w_qkv"].T + T["l0.b_qkv"]).reshape(N, 3, 2, 8)
    q, k, v = rope(qkv[:, 0]), rope(qkv[:, 1]), qkv[:, 2]
    outs = []
    for i in range(2):
        a, b = int(cu[i]), int(cu[i + 1])
        outs.append(torch.nn.functional.scaled_dot_product_attention(
            q[a:b].transpose(0, 1), k[a:b].transpose(0, 1), v[a:b].transpose(0, 1)).transpose(0, 1))
    att = torch.cat(outs).reshape(N, d)
    R1 = Rt + att @ T["l0.w_o"].T + T["l0.b_o"]
    hh = ln(R1, T["l0.ln2_g"], T["l0.ln2_b"]) @ T["l0.w_fc1"].T + T["l0.b_fc1"]
    R2 = R1 + torch.nn.functional.gelu(hh, approximate="tanh") @ T["l0.w_fc2"].T + T["l0.b_fc2"]
    R2.backward(torch.tensor(dR2))
    np.testing.assert_allclose(dR, Rt.grad.numpy(), rtol=1e-9, atol=1e-10)
    for k, v in grads.items():
        np.testing.assert_allclose(v, T["l0." + k].grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=k)


def _qkv_attention(qkv, pos, cu, cfg):
    axis, inv = oracle.rope_tables(cfg.head_dim, cfg.rope_sections, cfg.rope_theta, cfg.rope_shared_ladder)
    q = oracle.apply_rope(qkv[:, 0], pos, axis, inv)
    k = oracle.apply_rope(qkv[:, 1], pos, axis, inv)
    return oracle.attention_varlen(q, k, np.ascontiguousarray(qkv[:, 2]), cu).reshape(qkv.shape[0], -1)


def test_attention_qkv_gradient_and_sampled_rows():
    """attention_qkv_backward (RoPE included) against central differences;
    attention_dq_rows equals its q rows; and the two identities the sampled
    GPU checks use: sum over keys of dv = sum over queries of dO (softmax rows
    sum to 1), and sum over keys of the rotated-frame dk = 0 (each row of dS
    sums to 0)."""
    cfg = TINY
    grids = [(1, 2, 4), (1, 2, 2)]
    pos = oracle.positions(grids)
    cu = oracle.cu_seqlens(grids)
    N, H, hd = 12, cfg.heads, cfg.head_dim
    qkv = rng(30).standard_normal((N, 3, H, hd))
    do = rng(31).standard_normal((N, H * hd))
    g = G.attention_qkv_backward(qkv, pos, cu, do, cfg)
    fd_dot(lambda t: _qkv_attention(t, pos, cu, cfg), qkv, do, g)
    rows = np.array([0, 5, 7, 9, 11])
    np.testing.assert_allclose(G.attention_dq_rows(qkv, pos, cu, do, rows, cfg), g[rows, 0],
                               rtol=1e-12, atol=1e-12)
    axis, inv = oracle.rope_tables(hd, cfg.rope_sections, cfg.rope_theta, cfg.rope_shared_ladder)
    dk_rot = oracle.apply_rope(g[:, 1], pos, axis, inv)
    d3 = do.reshape(N, H, hd)
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        np.testing.assert_allclose(g[a:b, 2].sum(0), d3[a:b].sum(0), rtol=1e-12, atol=1e-12)
        assert np.max(np.abs(dk_rot[a:b].sum(0))) < 1e-12
    # a planted sign error in dS breaks the finite-difference pin
    bad = g.copy()
    bad[:, 0] *= -1
    with pytest.raises(AssertionError):
        fd_dot(lambda t: _qkv_attention(t, pos, cu, cfg), qkv, do, bad)


def test_tower_gradient_finite_differences():
    """tower_backward (patch embed + 2 tiny blocks, two items) against central
    differences of the forward oracle along random directions of the patch
    weight, a first-layer weight (its gradient crosses the second block) and
    the last layer's LN gamma."""
    cfg = TINY
    grids = [(1, 2, 2), (1, 2, 4)]
    g0 = rng(40)
    d, mlp, H, hd = cfg.hidden, cfg.mlp, cfg.heads, cfg.head_dim
    W = {"patch_w": g0.standard_normal((d, 1176)) * 0.03, "patch_b": g0.standard_normal(d) * 0.1}
    for i in range(2):
        p = f"l{i}."
        W.update({p + "ln1_g": 1 + 0.1 * g0.standard_normal(d), p + "ln1_b": 0.1 * g0.standard_normal(d),
                  p + "w_qkv": g0.standard_normal((3 * d, d)) * 0.3, p + "b_qkv": 0.1 * g0.standard_normal(3 * d),
                  p + "w_o": g0.standard_normal((d, d)) * 0.3, p + "b_o": 0.1 * g0.standard_normal(d),
                  p + "ln2_g": 1 + 0.1 * g0.standard_normal(d), p + "ln2_b": 0.1 * g0.standard_normal(d),
                  p + "w_fc1": g0.standard_normal((mlp, d)) * 0.3, p + "b_fc1": 0.1 * g0.standard_normal(mlp),
                  p + "w_fc2": g0.standard_normal((d, mlp)) * 0.3, p + "b_fc2": 0.1 * g0.standard_normal(d)})
    images = [g0.random((3, 14 * h, 14 * w)) for _, h, w in grids]
    N = sum(h * w for _, h, w in grids)
    dT = g0.standard_normal((N, d))
    pos, cu = oracle.positions(grids), oracle.cu_seqlens(grids)

    def tower(Wx):
        R = oracle.patch_embed(images, Wx, grids)
        for i in range(2):
            R = oracle.block_forward(R, Wx, pos, cu, cfg, prefix=f"l{i}.")
        return R

    grads = G.tower_backward(images, grids, W, cfg, 2, dT)
    for name in ("patch_w", "patch_b", "l0.w_qkv", "l1.ln2_g"):
        def f(t, name=name):
            Wx = dict(W)
            Wx[name] = t
            return tower(Wx)
        fd_dot(f, W[name], dT, grads[name])
