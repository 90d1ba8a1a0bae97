"""Backward pieces of the invariant forward against the fp64 gradient oracle, and their
determinism: transpose (exact), add+RMSNorm, SiLU*up, linear / SiLU-gated MLP and the
lm_head logprob (config 3's vocabulary), at the Qwen3-shaped widths.

Tolerances.  A kernel that rounds its own fp32 result to bf16 is held to the bf16
grid (1-2 ulp plus the fp32 cancellation bound).  Composite gradients pass through
bf16 intermediates the oracle does not round (dact, dgu, dz -- 2^-9 relative each) and
fp32 GEMM accumulation: they are held to a relative Frobenius error of 1e-2 and
elementwise to 1.5e-2 of the tensor's largest magnitude (measured: 0.9-2.9e-3 and
up to 4.0e-3)."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import BF, assert_bf16_close, f64, same_bits
from oracle import backward as ob
from oracle import ops
from test_gpu_ops import abi, make_ctx

pytestmark = pytest.mark.gpu

REL_FRO, MAX_FRAC = 1e-2, 1.5e-2


def bwd():
    from bitwise_consistent_rl_amd import backward
    return backward


@pytest.fixture(scope="module")
def ctx():
    h = make_ctx(max_tokens=4096, max_scored=512)
    yield h
    torch.cuda.synchronize()
    abi().bci_destroy(h)


def close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    fro = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300)
    print(f"{what}: relative Frobenius {fro:.2e}, max/max {mx:.2e}", flush=True)
    assert fro <= REL_FRO and mx <= MAX_FRAC, (what, fro, mx)


@pytest.mark.parametrize("R,C,ld", [(1, 8, 8), (37, 64, 64), (300, 2048, 320), (4096, 72, 4096)])
def test_transpose_exact(ctx, R, C, ld):
    x = synth.normal_bf16((R, C), index=R + C).cuda()
    out = torch.full((C, ld), float("nan"), dtype=BF, device="cuda")
    abi().bci_op_transpose_bf16(ctx, x, out, R, C, ld)
    torch.cuda.synchronize()
    want = torch.zeros(C, ld, dtype=BF)
    want[:, :R] = x.cpu().T
    assert same_bits(out, want)


@pytest.mark.parametrize("rows,H", [(1, 256), (77, 2048), (600, 4096)])
def test_add_rmsnorm_backward(ctx, rows, H):
    r = synth.normal_bf16((rows, H), index=60).cuda()
    g = synth.normal_bf16((H,), index=61, scale=0.1).cuda()
    g = (g.float() + 1.0).to(BF)
    dh = synth.normal_bf16((rows, H), index=62).cuda()
    dr_in = synth.normal_bf16((rows, H), index=63).cuda()
    dr, dg, rstd = bwd().add_rmsnorm_backward(ctx, r, g, dh, 1e-6, dr_in)
    torch.cuda.synchronize()
    R, G, DH, DRI = f64(r), f64(g), f64(dh), f64(dr_in)
    ref_dr, ref_dg = ob.rmsnorm_backward(R, G, DH, 1e-6, DRI)
    s = 1.0 / np.sqrt(np.mean(R * R, axis=1, keepdims=True) + 1e-6)
    cancel = 2.0 ** -20 * (np.abs(G * DH) * s + np.abs(R) * s ** 3 * np.sum(np.abs(G * DH * R), axis=1,
                                                                             keepdims=True) / H + np.abs(DRI))
    assert_bf16_close(f64(dr), ref_dr, abs_bound=cancel, max_ulp=1, frac_exact=0.99, what="dr")
    np.testing.assert_allclose(rstd.cpu().numpy(), s[:, 0], rtol=1e-6)
    bound = 1e-5 * np.sum(np.abs(DH * R) * s, axis=0) + 1e-30
    assert np.all(np.abs(dg.cpu().numpy() - ref_dg) <= bound)
    # deterministic, and each row of dr independent of the other rows
    dr2, dg2, _ = bwd().add_rmsnorm_backward(ctx, r, g, dh, 1e-6, dr_in)
    assert same_bits(dr2, dr) and same_bits(dg2, dg)
    if rows > 1:
        sub = slice(rows // 3, rows // 3 + 5)
        dr3, _, _ = bwd().add_rmsnorm_backward(ctx, r[sub].contiguous(), g, dh[sub].contiguous(), 1e-6,
                                               dr_in[sub].contiguous())
        assert same_bits(dr3, dr[sub])


def test_silu_mul_backward(ctx):
    rows, inter = 129, 768
    gu = synth.normal_bf16((rows, 2 * inter), index=64, scale=3.0).cuda()
    dact = synth.normal_bf16((rows, inter), index=65).cuda()
    dgu = torch.empty_like(gu)
    abi().bci_op_silu_mul_backward(ctx, gu, dact, dgu, rows, inter)
    torch.cuda.synchronize()
    G, D = f64(gu), f64(dact)
    rg, ru = ob.silu_mul_backward(G[:, :inter], G[:, inter:], D)
    got = f64(dgu)
    assert_bf16_close(got[:, :inter], rg, abs_bound=2.0 ** -20 * np.abs(D * G[:, inter:]), max_ulp=2,
                      what="d gate")
    assert_bf16_close(got[:, inter:], ru, abs_bound=2.0 ** -20 * np.abs(D * G[:, :inter]), max_ulp=2,
                      what="d up")


@pytest.mark.parametrize("M,H,inter", [(37, 256, 768), (300, 2048, 6144)])
def test_mlp_backward(ctx, M, H, inter):
    h = synth.normal_bf16((M, H), index=66).cuda()
    wgu = synth.normal_bf16((2 * inter, H), index=67, scale=0.02).cuda()
    wd = synth.normal_bf16((H, inter), index=68, scale=0.02).cuda()
    dout = synth.normal_bf16((M, H), index=69).cuda()
    dh, dwgu, dwd, gu, act = bwd().mlp_backward(ctx, h, wgu, wd, dout, inter)
    torch.cuda.synchronize()
    # the forward values the oracle is evaluated at: its own forward of the same inputs
    Hh, Wgu, Wd, Do = f64(h), f64(wgu), f64(wd), f64(dout)
    Gu = ops.bf(ops.linear(Hh, Wgu))
    Act = ops.silu_mul(Gu[:, :inter], Gu[:, inter:])
    rdh, rdwgu, rdwd = ob.mlp_backward(Hh, Wgu, Wd, Do, inter, Gu, Act)
    close(f64(dh), rdh, f"dh M={M}")
    close(dwgu.cpu().numpy(), rdwgu, f"dwgu M={M}")
    close(dwd.cpu().numpy(), rdwd, f"dwd M={M}")
    # deterministic; rows of dh independent of the batch
    dh2, dwgu2, dwd2, _, _ = bwd().mlp_backward(ctx, h, wgu, wd, dout, inter)
    assert same_bits(dh2, dh) and same_bits(dwgu2, dwgu) and same_bits(dwd2, dwd)
    sub = slice(M // 2, M // 2 + 3)
    dh3, _, _, _, _ = bwd().mlp_backward(ctx, h[sub].contiguous(), wgu, wd, dout[sub].contiguous(), inter)
    assert same_bits(dh3, dh[sub])


@pytest.mark.parametrize("M,V", [(7, 4096), (64, 151936)])
def test_logprob_backward(ctx, M, V):
    H = 2048
    hs, w, ids = synth.lmhead_inputs(M, hidden=H, vocab=V)
    gout = np.random.default_rng(M).standard_normal(M).astype(np.float32)
    hf, emb = hs.cuda(), w.cuda()
    gids = torch.from_numpy(ids.astype(np.int32)).cuda()
    gg = torch.from_numpy(gout).cuda()
    dhf, dE = bwd().logprob_backward(ctx, hf, emb, gids, gg)
    torch.cuda.synchronize()
    HF, E = f64(hs), f64(w)
    rdhf, rdE, _ = ob.logprob_backward(HF, E, ids, gout)
    close(f64(dhf), rdhf, f"dhf M={M} V={V}")
    if V <= 4096:
        close(dE.cpu().numpy(), rdE, f"dE M={M} V={V}")
    else:   # the sampled rows and 256 others (a 151936 x 2048 comparison is not needed)
        rows = np.unique(np.concatenate([ids, np.random.default_rng(1).choice(V, 256, replace=False)]))
        close(dE[torch.from_numpy(rows).cuda()].cpu().numpy(), rdE[rows], f"dE rows M={M} V={V}")
    dhf2, dE2 = bwd().logprob_backward(ctx, hf, emb, gids, gg)
    assert same_bits(dhf2, dhf) and same_bits(dE2, dE)


@pytest.mark.parametrize("L,nq,nkv,d,kv", [(37, 4, 2, 64, "bf16"), (300, 16, 8, 128, "bf16"),
                                           (200, 32, 4, 128, "fp8"), (129, 16, 8, 128, "fp8"),
                                           (1100, 8, 2, 128, "bf16"), (1100, 4, 1, 64, "fp8")])
def test_attention_backward(L, nq, nkv, d, kv):
    """The GPU's forward (RoPE + KV write, FP8 round trip for an FP8 cache, attention) then
    the backward over the keys and values it attended to; the oracle rotates, round-trips,
    attends and differentiates the same seeded rows itself.  With the part buffer given:
    at L = 1100 (4400 rows per kv head) the dK/dV rows are cut into two parts, within the
    same tolerance; below 4096 rows the part buffer changes no bit."""
    from test_gpu_ops import _attention_run
    a = abi()
    qkv = synth.normal_bf16((L, (nq + 2 * nkv) * d), index=70)
    o, q, kvs = _attention_run(nq, nkv, d, kv, 2048, [L], qkv, [[(0, 0, L)]])
    K, Vv = kvs[0]
    dout = synth.normal_bf16((L, nq * d), index=71).cuda()
    h = make_ctx(hidden=512, nq=nq, nkv=nkv, d=d, inter=512, vocab=4096, kv=kv, max_tokens=2048)
    try:
        outs = []
        ws = torch.full((2 * 4 * L * nkv * d,), float("nan"), device="cuda")
        for w in (ws, ws, None):
            dq = torch.empty(L, nq * d, dtype=BF, device="cuda")
            dk = torch.empty(L, nkv * d, dtype=BF, device="cuda")
            dv = torch.empty(L, nkv * d, dtype=BF, device="cuda")
            a.bci_op_attention_backward(h, q, K, Vv, o, dout, L, dq, dk, dv, w)
            torch.cuda.synchronize()
            outs.append((dq, dk, dv))
        assert all(same_bits(x, y) for x, y in zip(outs[0], outs[1]))       # deterministic
        split = L * (nq // nkv) >= 4096
        assert same_bits(outs[0][0], outs[2][0])                            # dq never split
        if not split:
            assert all(same_bits(x, y) for x, y in zip(outs[0], outs[2]))
    finally:
        torch.cuda.synchronize()
        a.bci_destroy(h)
    X = f64(qkv)
    pos = np.arange(L)
    qo = ops.rope(X[:, : nq * d].reshape(L, nq, d), pos, 1e6)
    ko = ops.rope(X[:, nq * d:(nq + nkv) * d].reshape(L, nkv, d), pos, 1e6)
    vo = X[:, (nq + nkv) * d:].reshape(L, nkv, d)
    if kv == "fp8":
        ko, vo = ops.kv_roundtrip(ko), ops.kv_roundtrip(vo)
    oo = ops.causal_gqa_attention(qo, ko, vo, pos)
    rdq, rdk, rdv = ob.attention_backward(qo, ko, vo, oo, f64(dout).reshape(L, nq, d))
    for tag, (dq, dk, dv) in (("parts", outs[0]), ("unsplit", outs[2])):
        close(f64(dq).reshape(L, nq, d), rdq, f"dq L={L} {kv} {tag}")
        close(f64(dk).reshape(L, nkv, d), rdk, f"dk L={L} {kv} {tag}")
        close(f64(dv).reshape(L, nkv, d), rdv, f"dv L={L} {kv} {tag}")


def _layer_ctx(L, H, nq, nkv, d, inter, kv, pos0=0):
    from test_gpu_ops import _alloc_cache, _batch_for
    a = abi()
    h = make_ctx(hidden=H, nq=nq, nkv=nkv, d=d, inter=inter, vocab=4096, kv=kv, max_tokens=1024)
    lengths = [L] if np.isscalar(L) else list(L)
    p0 = [pos0] * len(lengths) if np.isscalar(pos0) else list(pos0)
    cu, p0a, bt, nb = _batch_for(lengths, p0)
    cache = _alloc_cache(1, nb, nkv, d, kv)
    a.bci_bind_kv_cache(h, *cache, nb)
    a.bci_set_batch(h, np.zeros(int(cu[-1]), np.int32), cu, p0a, bt, [], [])
    return h, cache


def test_rope_backward():
    """The rotation's transpose at every token's own position (two sequences, the second
    starting at position 100): q and k heads within one bf16 rounding of the exact
    transpose applied with the forward's fp32 table, v heads copied bit for bit."""
    nq, nkv, d = 16, 8, 128
    lengths, p0 = [37, 90], [0, 100]
    h, cache = _layer_ctx(lengths, 2048, nq, nkv, d, 6144, "bf16", p0)
    try:
        T = sum(lengths)
        dq = synth.normal_bf16((T, nq * d), index=80).cuda()
        dk = synth.normal_bf16((T, nkv * d), index=81).cuda()
        dv = synth.normal_bf16((T, nkv * d), index=82).cuda()
        got = f64(bwd().rope_backward(h, dq, dk, dv))
        torch.cuda.synchronize()
    finally:
        abi().bci_destroy(h)
    pos = np.concatenate([np.arange(p, p + L) for p, L in zip(p0, lengths)])
    for lo, hi, x, nh in ((0, nq * d, dq, nq), (nq * d, (nq + nkv) * d, dk, nkv)):
        X = f64(x).reshape(T, nh, d)
        ref = ob.rope_backward(X, pos, 1e6).reshape(T, nh * d)
        c, s = ops.rope_tables(pos, d, 1e6)
        cs = np.concatenate([np.abs(c), np.abs(c)], axis=1)[:, None, :]
        ss = np.concatenate([np.abs(s), np.abs(s)], axis=1)[:, None, :]
        sw = np.concatenate([X[..., d // 2:], X[..., : d // 2]], axis=-1)
        bound = (2.0 ** -22 * (np.abs(X) * cs + np.abs(sw) * ss)).reshape(T, nh * d)
        assert_bf16_close(got[:, lo:hi], ref, abs_bound=bound, max_ulp=1, frac_exact=0.999, what="rope bwd")
    assert np.array_equal(got[:, (nq + nkv) * d:], f64(dv))


@pytest.mark.parametrize("L,H,nq,nkv,d,inter,kv", [(200, 512, 8, 4, 64, 768, "bf16"),
                                                   (300, 2048, 16, 8, 128, 6144, "fp8")])
def test_decoder_layer_backward(L, H, nq, nkv, d, inter, kv):
    """A whole decoder layer: the GPU's forward (op by op, keeping its values) and the
    backward composed from the library's entry points, against the oracle's forward of the
    same seeded inputs and its layer gradient (pinned by autograd and finite differences);
    then the same backward again, bit for bit."""
    from types import SimpleNamespace
    from oracle import model as om
    names = ["attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd"]
    sc = 1.0 / np.sqrt(H)
    w = {"attn_norm": (synth.normal_bf16((H,), index=90, scale=0.1).float() + 1.0).to(BF),
         "wqkv": synth.normal_bf16(((nq + 2 * nkv) * d, H), index=91, scale=sc),
         "wo": synth.normal_bf16((H, nq * d), index=92, scale=1.0 / np.sqrt(nq * d)),
         "mlp_norm": (synth.normal_bf16((H,), index=93, scale=0.1).float() + 1.0).to(BF),
         "wgu": synth.normal_bf16((2 * inter, H), index=94, scale=sc),
         "wd": synth.normal_bf16((H, inter), index=95, scale=1.0 / np.sqrt(inter))}
    r_in = synth.normal_bf16((L, H), index=96)
    m_prev = synth.normal_bf16((L, H), index=97)
    d_r = synth.normal_bf16((L, H), index=98)
    d_m = synth.normal_bf16((L, H), index=99)
    wg = {k: v.cuda() for k, v in w.items()}
    h, cache = _layer_ctx(L, H, nq, nkv, d, inter, kv)
    try:
        dims = dict(nq=nq, nkv=nkv, d=d, inter=inter, eps=1e-6)
        saved = bwd().decoder_layer_forward(h, 0, wg, r_in.cuda(), m_prev.cuda(), **dims)
        g1 = bwd().decoder_layer_backward(h, wg, saved, d_r.cuda(), d_m.cuda(), inter=inter, eps=1e-6)
        g2 = bwd().decoder_layer_backward(h, wg, saved, d_r.cuda(), d_m.cuda(), inter=inter, eps=1e-6)
        torch.cuda.synchronize()
        assert all(same_bits(g1[k], g2[k]) for k in g1)                       # deterministic
        got = {k: (f64(v) if v.dtype == BF else v.cpu().numpy().astype(np.float64)) for k, v in g1.items()}
    finally:
        torch.cuda.synchronize()
        abi().bci_destroy(h)
    cfg = SimpleNamespace(n_q_heads=nq, n_kv_heads=nkv, head_dim=d, intermediate=inter, rms_eps=1e-6,
                          rope_theta=1e6)
    Wf = {k: f64(v) for k, v in w.items()}
    W = lambda name: Wf[name.split(".")[-1]]
    fwd = om.decoder_layer(cfg, W, 0, f64(m_prev), f64(r_in), np.arange(L), np.zeros((0, nkv, d)),
                           np.zeros((0, nkv, d)), kv)
    ref = ob.decoder_layer_backward(cfg, W, 0, fwd, f64(d_r), f64(d_m))
    for k in ["d_r_in"] + names:
        close(got[k], ref[k], f"layer {k} L={L} {kv}")
