"""Gradients of the forward's operators, in fp64 on the CPU.

Test infrastructure only.  Nothing on the product path imports this.

The trainer calls the inference kernels for its forward and adds its own backward;
forward agreement does not prove the gradients right, so they are checked against an
independent reference (page "Finish RL Training Faster" digest, section
"让训练前向使用推理的数值").  Reading: the backward is evaluated at the forward's
stored values (the bf16-rounded residual, gate/up outputs, activations and hidden
states) and treats every rounding of the forward as the identity (straight-through);
everything here is the exact derivative of the unrounded operator at those values.
Each function writes the derivative out; the pins compare it with finite differences
and with torch's autograd.
"""
from __future__ import annotations

import numpy as np

from .ops import silu


def rmsnorm_backward(r, g, dh, eps: float, dr_in=None):
    """h = r * s * g with s = (mean(r^2) + eps)^(-1/2) per row.

    dL/dr = g*dh*s - r * s^3 * sum_k(g_k dh_k r_k) / H (+ dr_in, the gradient that
    reaches r through the residual stream); dL/dg = sum over rows of dh * r * s.
    r, dh, dr_in: [rows, H]; g: [H].  Returns (dr, dg)."""
    r = np.asarray(r, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    dh = np.asarray(dh, dtype=np.float64)
    H = r.shape[-1]
    s = 1.0 / np.sqrt(np.mean(r * r, axis=-1, keepdims=True) + eps)
    dot = np.sum(g * dh * r, axis=-1, keepdims=True)
    dr = g * dh * s - r * s ** 3 * dot / H
    if dr_in is not None:
        dr = dr + np.asarray(dr_in, dtype=np.float64)
    dg = np.sum(dh * r * s, axis=0)
    return dr, dg


def silu_mul_backward(gate, up, dact):
    """act = silu(gate) * up.  d gate = dact * up * silu'(gate), d up = dact * silu(gate),
    silu'(x) = sig(x) * (1 + x * (1 - sig(x)))."""
    gate = np.asarray(gate, dtype=np.float64)
    up = np.asarray(up, dtype=np.float64)
    dact = np.asarray(dact, dtype=np.float64)
    sig = 1.0 / (1.0 + np.exp(-gate))
    return dact * up * sig * (1.0 + gate * (1.0 - sig)), dact * silu(gate)


def linear_backward(x, w, dy):
    """y = x . w^T.  dx = dy . w, dw = dy^T . x."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    return dy @ w, dy.T @ x


def mlp_backward(h, wgu, wd, dout, inter: int, gu, act):
    """The SiLU-gated MLP out = act . wd^T, act = silu(g) u, [g u] = h . wgu^T.

    gu, act: the forward's stored gate/up outputs and activation (bf16 values).
    Returns (dh, dwgu, dwd)."""
    dact, dwd = linear_backward(act, wd, dout)
    dg, du = silu_mul_backward(gu[:, :inter], gu[:, inter:], dact)
    dgu = np.concatenate([dg, du], axis=1)
    dh, dwgu = linear_backward(h, wgu, dgu)
    return dh, dwgu, dwd


def logprob_backward(hf, emb, ids, gout):
    """lp_i = z[i, ids_i] - logsumexp(z_i), z = hf . E^T; L = sum_i gout_i lp_i.

    dz = gout_i (onehot(ids_i) - softmax(z_i)); dhf = dz . E; dE = dz^T . hf.
    hf [M, H] and emb [V, H] as float64 values.  Returns (dhf, dE, dz)."""
    hf = np.asarray(hf, dtype=np.float64)
    emb = np.asarray(emb, dtype=np.float64)
    gout = np.asarray(gout, dtype=np.float64)
    z = hf @ emb.T
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    dz = -gout[:, None] * p
    dz[np.arange(len(ids)), np.asarray(ids)] += gout
    return dz @ emb, dz.T @ hf, dz


def attention_backward(q, k, v, o, do):
    """Causal GQA attention of one sequence (positions 0..T-1): o = softmax(q k^T / sqrt(d)) v.

    q, o, do: [T, nq, d]; k, v: [T, nkv, d] (the keys and values the forward attended
    to -- for an FP8 cache the dequantised ones; the quantiser's gradient is taken as
    the identity, so dk and dv are also the gradients of the keys and values before
    quantisation).  With P the attention weights, D_i = sum_d do_i o_i (o as stored):
        dv_j = sum_i P_ij do_i,  dP_ij = do_i . v_j,  dS = P * (dP - D),
        dq_i = sum_j dS_ij k_j / sqrt(d),  dk_j = sum_i dS_ij q_i / sqrt(d),
    summed over the query heads that read each kv head.  Returns (dq, dk, dv)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    T, nq, d = q.shape
    nkv = k.shape[1]
    grp = nq // nkv
    mask = np.tril(np.ones((T, T), dtype=bool))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(nq):
        g = h // grp
        s = q[:, h] @ k[:, g].T / np.sqrt(d)
        s = np.where(mask, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        D = np.sum(do[:, h] * o[:, h], axis=1, keepdims=True)
        dP = do[:, h] @ v[:, g].T
        dS = p * (dP - D)
        dv[:, g] += p.T @ do[:, h]
        dq[:, h] = dS @ k[:, g] / np.sqrt(d)
        dk[:, g] += dS.T @ q[:, h] / np.sqrt(d)
    return dq, dk, dv


def rope_backward(dx_rot, positions, theta: float):
    """The rotation's transpose: x_rot = (x1 c - x2 s, x2 c + x1 s) per pair (i, i + d/2),
    so dx1 = dr1 c + dr2 s, dx2 = dr2 c - dr1 s.  dx_rot: [T, heads, d]."""
    from .ops import rope_tables
    dx_rot = np.asarray(dx_rot, dtype=np.float64)
    d = dx_rot.shape[-1]
    c, s = rope_tables(positions, d, theta)
    c, s = c[:, None, :], s[:, None, :]
    r1, r2 = dx_rot[..., : d // 2], dx_rot[..., d // 2:]
    return np.concatenate([r1 * c + r2 * s, r2 * c - r1 * s], axis=-1)


def decoder_layer_backward(cfg, W, li: int, fwd: dict, d_r, d_m):
    """Gradient of one pre-norm decoder layer of one sequence at positions 0..n-1 (the
    layer of ``oracle.model.decoder_layer``, one chunk, empty cache before it):

        r1, h = AddNorm(m_prev, r_in, g_attn);  q, k, v = RoPE(split(h Wqkv^T))
        a = Attn(q, k, v) Wo^T;  r2, h2 = AddNorm(a, r1, g_mlp);  m = MLP(h2)

    ``fwd`` holds the forward's stored values (keys r_mid = r1, h, q, K, V, o, r = r2,
    h2, as ``decoder_layer`` returns them); d_r and d_m are the gradients reaching the
    layer's outputs r2 and m.  The chain runs the layer backwards, each step the exact
    derivative evaluated at the stored values with every rounding (and an FP8 cache's
    quantiser) taken as the identity:
        dh2, dWgu, dWd = MLP backward;      dr2 = d_r + AddNorm backward of h2
        do, dWo = dr2 through a = o Wo^T;   dq, dk, dv = attention backward
        dqkv = [R^T dq, R^T dk, dv];        dh, dWqkv = dqkv through h Wqkv^T
        dr1 = dr2 + AddNorm backward of h   (= d m_prev = d r_in, the add's two inputs)
    Returns a dict of float64 arrays: d_r_in, attn_norm, wqkv, wo, mlp_norm, wgu, wd."""
    from . import ops
    nq, nkv, d, inter = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.intermediate
    p = f"layers.{li}."
    n = fwd["h"].shape[0]
    pos = np.arange(n)
    h2 = np.asarray(fwd["h2"], dtype=np.float64)
    gu = fwd.get("gu")
    if gu is None:
        gu = ops.bf(ops.linear(h2, W(p + "wgu")))
    act = fwd.get("act")
    if act is None:
        act = ops.silu_mul(gu[:, :inter], gu[:, inter:])
    dh2, dwgu, dwd = mlp_backward(h2, W(p + "wgu"), W(p + "wd"), d_m, inter, gu, act)
    dr2, dg2 = rmsnorm_backward(fwd["r"], W(p + "mlp_norm"), dh2, cfg.rms_eps, d_r)
    o = np.asarray(fwd["o"], dtype=np.float64)
    do, dwo = linear_backward(o.reshape(n, nq * d), W(p + "wo"), dr2)
    dq, dk, dv = attention_backward(fwd["q"], fwd["K"], fwd["V"], o, do.reshape(n, nq, d))
    dqkv = np.concatenate([rope_backward(dq, pos, cfg.rope_theta).reshape(n, nq * d),
                           rope_backward(dk, pos, cfg.rope_theta).reshape(n, nkv * d),
                           dv.reshape(n, nkv * d)], axis=1)
    dh, dwqkv = linear_backward(fwd["h"], W(p + "wqkv"), dqkv)
    dr1, dg1 = rmsnorm_backward(fwd["r_mid"], W(p + "attn_norm"), dh, cfg.rms_eps, dr2)
    return dict(d_r_in=dr1, attn_norm=dg1, wqkv=dwqkv, wo=dwo, mlp_norm=dg2, wgu=dwgu, wd=dwd)
