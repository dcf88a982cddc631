"""Oracle of the backward pass of one tower block (test infrastructure only).

The pages' towers are differentiable (their probe runs a backward pass and
reports a gradient norm, "v2_loaders FINDINGS" s.3); these functions give the
gradients of the forward steps in oracle/vit.py by their textbook formulas,
in plain numpy, in the dtype they are given (float64 in the pin tests, where
they are checked against central finite differences and torch autograd).

Notation: for y = f(x), ``f_backward(..., dy)`` returns dL/dx (and the
parameter gradients) given dL/dy.
"""
from __future__ import annotations

import numpy as np

from . import vit


def linear_backward(x, w, dy):
    """y = x W^T + b:  dx = dy W,  dW = dy^T x,  db = sum over rows of dy."""
    return dy @ w, dy.T @ x, dy.sum(axis=0)


def gelu_tanh_backward(h, dy):
    """d/dh of 0.5 h (1 + tanh(u)), u = sqrt(2/pi) (h + 0.044715 h^3)."""
    c = np.sqrt(2.0 / np.pi)
    u = c * (h + 0.044715 * h ** 3)
    t = np.tanh(u)
    du = c * (1.0 + 3 * 0.044715 * h ** 2)
    return dy * (0.5 * (1.0 + t) + 0.5 * h * (1.0 - t * t) * du)


def layer_norm_backward(x, g, dy, eps):
    """y = (x - mean) / sqrt(var + eps) * g + b over the last axis (biased
    variance).  Returns dx, dg, db."""
    mu = x.mean(axis=-1, keepdims=True)
    xc = x - mu
    var = (xc * xc).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xh = xc * rstd
    dxh = dy * g
    dx = rstd * (dxh - dxh.mean(axis=-1, keepdims=True) - xh * (dxh * xh).mean(axis=-1, keepdims=True))
    return dx, (dy * xh).sum(axis=0), dy.sum(axis=0)


def rope_backward(dy, pos, axis, inv_freq):
    """The rotation of each pair is orthogonal: its gradient is the rotation
    by the opposite angle."""
    return vit.apply_rope(dy, pos, axis, -inv_freq)


def attention_image_backward(q, k, v, dout, scale=None):
    """O = softmax(q k^T scale) v per head, q, k, v, dout: [n, heads, hd].
    With P the softmax and D_i = sum_d dO_id O_id:
    dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  dQ = dS K scale,  dK = dS^T Q scale."""
    n, H, hd = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    qh, kh, vh, dh = (np.ascontiguousarray(a.transpose(1, 0, 2)) for a in (q, k, v, dout))
    p = vit.softmax_rows(np.matmul(qh, kh.transpose(0, 2, 1)) * scale)     # H, n, n
    o = np.matmul(p, vh)
    dv = np.matmul(p.transpose(0, 2, 1), dh)
    dp = np.matmul(dh, vh.transpose(0, 2, 1))
    ds = p * (dp - (dh * o).sum(axis=-1, keepdims=True))
    dq = np.matmul(ds, kh) * scale
    dk = np.matmul(ds.transpose(0, 2, 1), qh) * scale
    return tuple(np.ascontiguousarray(a.transpose(1, 0, 2)) for a in (dq, dk, dv))


def attention_varlen_backward(q, k, v, dout, cu, scale=None):
    """Block-diagonal (per image) attention backward."""
    dq, dk, dv = (np.empty_like(q) for _ in range(3))
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        dq[a:b], dk[a:b], dv[a:b] = attention_image_backward(q[a:b], k[a:b], v[a:b], dout[a:b], scale)
    return dq, dk, dv


def attention_qkv_backward(qkv, pos, cu, dout, cfg: vit.Config = None):
    """Gradient of the attention step of a block with respect to its input,
    the QKV Linear output [N, 3, heads, hd] (before RoPE); dout [N, heads*hd]."""
    cfg = cfg or vit.Config()
    N = qkv.shape[0]
    H, hd = cfg.heads, cfg.head_dim
    axis, inv = vit.rope_tables(hd, cfg.rope_sections, cfg.rope_theta, cfg.rope_shared_ladder)
    q = vit.apply_rope(qkv[:, 0], pos, axis, inv)
    k = vit.apply_rope(qkv[:, 1], pos, axis, inv)
    v = np.ascontiguousarray(qkv[:, 2])
    dq, dk, dv = attention_varlen_backward(q, k, v, dout.reshape(N, H, hd), cu)
    return np.stack([rope_backward(dq, pos, axis, inv), rope_backward(dk, pos, axis, inv), dv], axis=1)


def block_backward(R, W, pos, cu, cfg: vit.Config, dR2, prefix="l0."):
    """Gradients of one pre-LN block (vit.block_forward) given dL/d(output).
    Returns (dL/dR, {parameter name: gradient})."""
    N, d = R.shape
    H, hd = cfg.heads, cfg.head_dim
    g = lambda name: W[prefix + name]
    # forward, keeping the intermediates
    x1 = vit.layer_norm(R, g("ln1_g"), g("ln1_b"), cfg.ln_eps)
    qkv = vit.linear(x1, g("w_qkv"), g("b_qkv")).reshape(N, 3, H, hd)
    axis, inv = vit.rope_tables(hd, cfg.rope_sections, cfg.rope_theta, cfg.rope_shared_ladder)
    q = vit.apply_rope(qkv[:, 0], pos, axis, inv)
    k = vit.apply_rope(qkv[:, 1], pos, axis, inv)
    v = np.ascontiguousarray(qkv[:, 2])
    a = vit.attention_varlen(q, k, v, cu).reshape(N, d)
    R1 = R + vit.linear(a, g("w_o"), g("b_o"))
    x2 = vit.layer_norm(R1, g("ln2_g"), g("ln2_b"), cfg.ln_eps)
    h = vit.linear(x2, g("w_fc1"), g("b_fc1"))
    u = vit.gelu_tanh(h)
    # backward
    grads = {}
    du, grads["w_fc2"], grads["b_fc2"] = linear_backward(u, g("w_fc2"), dR2)
    dh = gelu_tanh_backward(h, du)
    dx2, grads["w_fc1"], grads["b_fc1"] = linear_backward(x2, g("w_fc1"), dh)
    dln2, grads["ln2_g"], grads["ln2_b"] = layer_norm_backward(R1, g("ln2_g"), dx2, cfg.ln_eps)
    dR1 = dR2 + dln2
    da, grads["w_o"], grads["b_o"] = linear_backward(a, g("w_o"), dR1)
    dq, dk, dv = attention_varlen_backward(q, k, v, da.reshape(N, H, hd), cu)
    dqkv = np.stack([rope_backward(dq, pos, axis, inv), rope_backward(dk, pos, axis, inv), dv],
                    axis=1).reshape(N, 3 * d)
    dx1, grads["w_qkv"], grads["b_qkv"] = linear_backward(x1, g("w_qkv"), dqkv)
    dln1, grads["ln1_g"], grads["ln1_b"] = layer_norm_backward(R, g("ln1_g"), dx1, cfg.ln_eps)
    return dR1 + dln1, grads


def attention_dq_rows(qkv, pos, cu, dout, rows, cfg: vit.Config = None):
    """Rows ``rows`` (token indices) of the q part of attention_qkv_backward.
    A query's gradient needs only its own softmax row, so this costs
    O(len(rows) * n) per head and serves sampled checks of long images."""
    cfg = cfg or vit.Config()
    N = qkv.shape[0]
    H, hd = cfg.heads, cfg.head_dim
    axis, inv = vit.rope_tables(hd, cfg.rope_sections, cfg.rope_theta, cfg.rope_shared_ladder)
    rows = np.asarray(rows)
    out = np.empty((len(rows), H, hd), qkv.dtype)
    d = dout.reshape(N, H, hd)
    scale = 1.0 / np.sqrt(hd)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        sel = np.nonzero((rows >= a) & (rows < b))[0]
        if len(sel) == 0:
            continue
        r = rows[sel]
        q = vit.apply_rope(qkv[r, 0], pos[r], axis, inv)                # m, H, hd
        k = vit.apply_rope(qkv[a:b, 1], pos[a:b], axis, inv)           # n, H, hd
        v = qkv[a:b, 2]
        for h in range(H):
            p = vit.softmax_rows(q[:, h] @ k[:, h].T * scale)          # m, n
            o = p @ v[:, h]
            dp = d[r, h] @ v[:, h].T
            ds = p * (dp - (d[r, h] * o).sum(axis=-1, keepdims=True))
            out[sel, h] = ds @ k[:, h] * scale
        out[sel] = rope_backward(out[sel], pos[r], axis, inv)
    return out


def tower_backward(images, grids, W, cfg: vit.Config, n_layers, d_tower, progress=None):
    """Gradients of the tower -- patch embed, then n_layers blocks -- given
    dL/d(tower output) ``d_tower`` [N, d] (raster order).  ``images`` are the
    items as vit.split_pixels returns them, ``W`` float weights.  Returns
    {"patch_w", "patch_b", "l<i>.<name>"} (the bias gradient even where the
    bias is absent).  ``progress(i)``, if given, is called after block i's
    backward."""
    pos = vit.positions(grids)
    cu = vit.cu_seqlens(grids)
    X = np.concatenate([vit.patchify(img) for img in images], axis=0)
    R = vit.linear(X, W["patch_w"], W.get("patch_b"))
    inputs = []
    for i in range(n_layers):
        inputs.append(R)
        R = vit.block_forward(R, W, pos, cu, cfg, prefix=f"l{i}.")
    dR = d_tower
    grads = {}
    for i in reversed(range(n_layers)):
        dR, g = block_backward(inputs[i], W, pos, cu, cfg, dR, prefix=f"l{i}.")
        grads.update({f"l{i}.{k}": v for k, v in g.items()})
        if progress:
            progress(i)
    _, grads["patch_w"], grads["patch_b"] = linear_backward(X, W["patch_w"], dR)
    return grads
