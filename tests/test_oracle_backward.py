"""Pins of the gradient oracle (CPU only): every derivative it writes out is compared
with central finite differences of the forward written in numpy, and with torch's
autograd in fp64 (a library routine, independent of the explicit formulas).  A sign
slip, a missing s^3 term, silu' written as sig(x) alone, or a transposed weight
gradient fails these."""
import numpy as np
import pytest
import torch

from oracle import backward as bw
from oracle.ops import silu


def fd(f, x, eps=1e-6):
    """Central differences of the scalar f at x (float64 array), same shape as x."""
    x = np.array(x, dtype=np.float64)
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f(x)
        x[i] = old - eps
        fm = f(x)
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


def test_rmsnorm_backward_against_finite_differences_and_autograd():
    rng = np.random.default_rng(0)
    rows, H, eps = 3, 8, 1e-6
    r = rng.standard_normal((rows, H))
    g = 1 + 0.1 * rng.standard_normal(H)
    dh = rng.standard_normal((rows, H))
    dr_in = rng.standard_normal((rows, H))
    dr, dg = bw.rmsnorm_backward(r, g, dh, eps, dr_in)

    def h_of(rr, gg):
        return rr / np.sqrt(np.mean(rr * rr, axis=-1, keepdims=True) + eps) * gg
    np.testing.assert_allclose(dr - dr_in, fd(lambda rr: np.sum(h_of(rr, g) * dh), r), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dg, fd(lambda gg: np.sum(h_of(r, gg) * dh), g), rtol=1e-6, atol=1e-8)
    rt = torch.tensor(r, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    (torch.nn.functional.rms_norm(rt, (H,), gt, eps) * torch.tensor(dh)).sum().backward()
    np.testing.assert_allclose(dr - dr_in, rt.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_silu_mul_backward():
    rng = np.random.default_rng(1)
    gate, up, dact = (rng.standard_normal((4, 6)) * 3 for _ in range(3))
    dg, du = bw.silu_mul_backward(gate, up, dact)
    np.testing.assert_allclose(dg, fd(lambda x: np.sum(silu(x) * up * dact), gate), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(du, fd(lambda x: np.sum(silu(gate) * x * dact), up), rtol=1e-6, atol=1e-8)
    # silu'(0) = 1/2; silu' -> 1 for large x, -> 0 for very negative x
    d0, _ = bw.silu_mul_backward(np.array([0.0, 40.0, -40.0]), np.ones(3), np.ones(3))
    np.testing.assert_allclose(d0, [0.5, 1.0, 0.0], atol=1e-12)


def test_linear_and_mlp_backward_against_autograd():
    rng = np.random.default_rng(2)
    M, H, inter = 5, 8, 6
    h = rng.standard_normal((M, H))
    wgu = rng.standard_normal((2 * inter, H)) * 0.3
    wd = rng.standard_normal((H, inter)) * 0.3
    dout = rng.standard_normal((M, H))
    gu = h @ wgu.T
    act = silu(gu[:, :inter]) * gu[:, inter:]
    dh, dwgu, dwd = bw.mlp_backward(h, wgu, wd, dout, inter, gu, act)
    ht = torch.tensor(h, requires_grad=True)
    wgut = torch.tensor(wgu, requires_grad=True)
    wdt = torch.tensor(wd, requires_grad=True)
    g = ht @ wgut.T
    out = (torch.nn.functional.silu(g[:, :inter]) * g[:, inter:]) @ wdt.T
    (out * torch.tensor(dout)).sum().backward()
    for mine, ref in ((dh, ht.grad), (dwgu, wgut.grad), (dwd, wdt.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-12, atol=1e-12)
    # finite differences on one weight entry of each matrix
    def loss(wgu_, wd_):
        gg = h @ wgu_.T
        return np.sum((silu(gg[:, :inter]) * gg[:, inter:]) @ wd_.T * dout)
    e = 1e-6
    for (i, j) in ((0, 0), (7, 3)):
        wp, wm = wgu.copy(), wgu.copy()
        wp[i, j] += e
        wm[i, j] -= e
        assert abs((loss(wp, wd) - loss(wm, wd)) / (2 * e) - dwgu[i, j]) < 1e-6
    wp, wm = wd.copy(), wd.copy()
    wp[2, 4] += e
    wm[2, 4] -= e
    assert abs((loss(wgu, wp) - loss(wgu, wm)) / (2 * e) - dwd[2, 4]) < 1e-6


def test_logprob_backward():
    rng = np.random.default_rng(3)
    M, H, V = 4, 6, 11
    hf = rng.standard_normal((M, H))
    emb = rng.standard_normal((V, H)) * 0.5
    ids = np.array([0, 3, 10, 3])
    gout = rng.standard_normal(M)

    def L(hf_, emb_):
        z = hf_ @ emb_.T
        m = z.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(z - m).sum(axis=1))
        return np.sum(gout * (z[np.arange(M), ids] - lse))
    dhf, dE, dz = bw.logprob_backward(hf, emb, ids, gout)
    np.testing.assert_allclose(dhf, fd(lambda x: L(x, emb), hf), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dE, fd(lambda x: L(hf, x), emb), rtol=1e-6, atol=1e-8)
    # each row of dz sums to zero (softmax gradient) and only the sampled column is positive
    np.testing.assert_allclose(dz.sum(axis=1), 0.0, atol=1e-12)
    # a zero upstream gradient gives zero gradients
    z0 = bw.logprob_backward(hf, emb, ids, np.zeros(M))
    assert not any(np.any(t) for t in z0)


def test_attention_backward_against_autograd_and_finite_differences():
    rng = np.random.default_rng(4)
    T, nq, nkv, d = 7, 4, 2, 8
    q, k, v, do = (rng.standard_normal(s) for s in ((T, nq, d), (T, nkv, d), (T, nkv, d), (T, nq, d)))

    def fwd(q_, k_, v_):
        out = np.empty((T, nq, d))
        for h in range(nq):
            g = h // (nq // nkv)
            s = q_[:, h] @ k_[:, g].T / np.sqrt(d)
            s = np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[:, h] = (p / p.sum(axis=1, keepdims=True)) @ v_[:, g]
        return out
    o = fwd(q, k, v)
    dq, dk, dv = bw.attention_backward(q, k, v, o, do)
    np.testing.assert_allclose(dq, fd(lambda x: np.sum(fwd(x, k, v) * do), q), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dk, fd(lambda x: np.sum(fwd(q, x, v) * do), k), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dv, fd(lambda x: np.sum(fwd(q, k, x) * do), v), rtol=1e-6, atol=1e-8)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ke = kt.repeat_interleave(nq // nkv, dim=1)
    ve = vt.repeat_interleave(nq // nkv, dim=1)
    s = torch.einsum("thd,shd->hts", qt, ke) / np.sqrt(d)
    s = s.masked_fill(~torch.tril(torch.ones(T, T, dtype=torch.bool)), float("-inf"))
    out = torch.einsum("hts,shd->thd", torch.softmax(s, dim=-1), ve)
    (out * torch.tensor(do)).sum().backward()
    for mine, ref in ((dq, qt.grad), (dk, kt.grad), (dv, vt.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_rope_backward_is_the_inverse_rotation():
    from oracle import ops
    rng = np.random.default_rng(5)
    T, H, d = 6, 3, 16
    x = rng.standard_normal((T, H, d))
    pos = np.arange(10, 10 + T)
    dy = rng.standard_normal((T, H, d))
    # <R x, dy> = <x, R^T dy> for the rotation R, computed without rounding
    c, s = ops.rope_tables(pos, d, 1e4)
    c, s = c[:, None, :], s[:, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    rx = np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    np.testing.assert_allclose(np.sum(rx * dy), np.sum(x * bw.rope_backward(dy, pos, 1e4)), rtol=1e-12)
    # the transpose of a rotation is its inverse (up to the fp32 rounding of the table)
    back = bw.rope_backward(rx, pos, 1e4)
    np.testing.assert_allclose(back, x, rtol=1e-6, atol=1e-6)


def test_decoder_layer_backward_against_autograd_and_finite_differences():
    """The layer composition (every piece, the residual paths into both norms, the RoPE
    transpose, the split of dqkv) against torch's autograd of the same layer written
    without roundings, fed with that forward's values; and central differences."""
    from types import SimpleNamespace
    from oracle import ops
    rng = np.random.default_rng(6)
    n, H, nq, nkv, d, inter = 6, 16, 4, 2, 8, 12
    cfg = SimpleNamespace(n_q_heads=nq, n_kv_heads=nkv, head_dim=d, intermediate=inter, rms_eps=1e-6,
                          rope_theta=1e4)
    w = {"attn_norm": 1 + 0.1 * rng.standard_normal(H), "wqkv": rng.standard_normal(((nq + 2 * nkv) * d, H)) * 0.3,
         "wo": rng.standard_normal((H, nq * d)) * 0.3, "mlp_norm": 1 + 0.1 * rng.standard_normal(H),
         "wgu": rng.standard_normal((2 * inter, H)) * 0.3, "wd": rng.standard_normal((H, inter)) * 0.3}
    m_prev, r_in, d_r, d_m = (rng.standard_normal((n, H)) for _ in range(4))
    c, s = (torch.tensor(x) for x in ops.rope_tables(np.arange(n), d, cfg.rope_theta))
    causal = torch.tril(torch.ones(n, n, dtype=torch.bool))

    def layer(mp, ri, g1, wqkv, wo, g2, wgu, wd):
        def norm(x, g):
            return x / torch.sqrt((x * x).mean(dim=-1, keepdim=True) + cfg.rms_eps) * g

        def rot(x):   # [n, heads, d], half-split pairs
            x1, x2 = x[..., : d // 2], x[..., d // 2:]
            return torch.cat([x1 * c[:, None] - x2 * s[:, None], x2 * c[:, None] + x1 * s[:, None]], dim=-1)
        r1 = mp + ri
        h = norm(r1, g1)
        qkv = h @ wqkv.T
        q = rot(qkv[:, : nq * d].reshape(n, nq, d))
        k = rot(qkv[:, nq * d:(nq + nkv) * d].reshape(n, nkv, d))
        v = qkv[:, (nq + nkv) * d:].reshape(n, nkv, d)
        heads = []
        for hq in range(nq):
            g = hq // (nq // nkv)
            sc = (q[:, hq] @ k[:, g].T / np.sqrt(d)).masked_fill(~causal, float("-inf"))
            heads.append(torch.softmax(sc, dim=-1) @ v[:, g])
        o = torch.stack(heads, dim=1)
        r2 = r1 + o.reshape(n, nq * d) @ wo.T
        h2 = norm(r2, g2)
        gu = h2 @ wgu.T
        act = torch.nn.functional.silu(gu[:, :inter]) * gu[:, inter:]
        m = act @ wd.T
        return dict(r_mid=r1, h=h, q=q, K=k, V=v, o=o, r=r2, h2=h2, gu=gu, act=act, m=m)

    names = ["attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd"]
    ins = [torch.tensor(m_prev, requires_grad=True), torch.tensor(r_in, requires_grad=True)] + \
          [torch.tensor(w[k], requires_grad=True) for k in names]
    out = layer(*ins)
    ((out["r"] * torch.tensor(d_r)).sum() + (out["m"] * torch.tensor(d_m)).sum()).backward()
    fwd = {k: v.detach().numpy() for k, v in out.items()}
    res = bw.decoder_layer_backward(cfg, lambda name: w[name.split(".")[-1]], 0, fwd, d_r, d_m)
    np.testing.assert_allclose(res["d_r_in"], ins[0].grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res["d_r_in"], ins[1].grad.numpy(), rtol=1e-10, atol=1e-12)
    for k, t in zip(names, ins[2:]):
        np.testing.assert_allclose(res[k], t.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)

    def loss(i, j, e):
        args = [x.detach().clone() for x in ins]
        args[i][j] += e
        o = layer(*args)
        return float((o["r"] * torch.tensor(d_r)).sum() + (o["m"] * torch.tensor(d_m)).sum())
    e = 1e-6
    for i, j, want in ((1, (2, 3), res["d_r_in"][2, 3]), (3, (5, 7), res["wqkv"][5, 7]),
                       (3, ((nq + nkv) * d + 1, 4), res["wqkv"][(nq + nkv) * d + 1, 4]),
                       (4, (1, 2), res["wo"][1, 2]), (2, (9,), res["attn_norm"][9])):
        assert abs((loss(i, j, e) - loss(i, j, -e)) / (2 * e) - want) < 1e-6 * max(1.0, abs(want))
