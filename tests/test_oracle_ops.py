"""Pins of the oracle's operators against closed forms, brute force, invariants and
library routines (CPU only).  Each test is chosen so that a plausible slip (a
dropped term, a wrong sign or index, a transposed operand) fails it."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ops
from oracle.codecs import bf16_round, e4m3_decode


def bfv(x):
    return bf16_round(np.asarray(x, dtype=np.float64))


# ------------------------------------------------------------------ RMSNorm

def test_rmsnorm_constant_row_closed_form():
    H, c, eps = 64, 0.75, 1e-6
    g = bfv(np.linspace(0.5, 1.5, H))
    r, h = ops.add_rmsnorm(None, np.full((1, H), c), g, eps)
    np.testing.assert_array_equal(r, np.full((1, H), c))
    np.testing.assert_array_equal(h[0], bfv(g * c / math.sqrt(c * c + eps)))


def test_rmsnorm_scale_invariance_and_eps_inside_sqrt():
    rng = np.random.default_rng(0)
    x = bfv(rng.standard_normal((4, 128)))
    g = bfv(1 + 0.02 * rng.standard_normal(128))
    _, h1 = ops.add_rmsnorm(None, x, g, 0.0)
    _, h2 = ops.add_rmsnorm(None, x * 2.0 ** 5, g, 0.0)
    np.testing.assert_array_equal(h1, h2)
    # eps is inside the square root: a row of tiny values is damped, not blown up
    _, h3 = ops.add_rmsnorm(None, np.full((1, 128), 1e-4), np.ones(128), 1e-6)
    assert abs(h3[0, 0] - 1e-4 / math.sqrt(1e-8 + 1e-6)) < 1e-2


def test_add_rmsnorm_rounds_residual_before_variance():
    a = np.array([[1.0, 2.0 ** -9]])
    r = np.array([[2.0 ** -9, 1.0]])
    rr, h = ops.add_rmsnorm(a, r, np.ones(2), 0.0)
    # 1 + 2^-9 rounds to 1 in bf16: the residual is stored rounded
    np.testing.assert_array_equal(rr, [[1.0, 1.0]])
    np.testing.assert_array_equal(h, [[1.0, 1.0]])


def test_rmsnorm_matches_torch_rms_norm():
    rng = np.random.default_rng(1)
    x = bfv(rng.standard_normal((16, 256)))
    g = bfv(1 + 0.02 * rng.standard_normal(256))
    _, h = ops.add_rmsnorm(None, x, g, 1e-6)
    ref = F.rms_norm(torch.from_numpy(x), (256,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_array_equal(h, bfv(ref))


# ------------------------------------------------------------------- linear

def test_linear_vs_triple_loop():
    rng = np.random.default_rng(2)
    x = bfv(rng.standard_normal((3, 5)))
    w = bfv(rng.standard_normal((4, 5)))
    y = ops.linear(x, w)
    for i in range(3):
        for j in range(4):
            s = 0.0
            for k in range(5):
                s += x[i, k] * w[j, k]
            assert abs(y[i, j] - s) < 1e-12


def test_silu_closed_forms_and_mlp_gate_up_order():
    assert ops.silu(0.0) == 0.0
    assert abs(ops.silu(40.0) - 40.0) < 1e-12
    assert abs(ops.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-15
    # zero input -> zero output
    H, I = 8, 4
    rng = np.random.default_rng(3)
    wgu = bfv(rng.standard_normal((2 * I, H)))
    wd = bfv(rng.standard_normal((H, I)))
    np.testing.assert_array_equal(ops.mlp(np.zeros((2, H)), wgu, wd, I), 0.0)
    # gate rows come first: with up == 1 for unit input, act == bf(silu(gate))
    x = np.zeros((1, H)); x[0, 0] = 1.0
    wgu2 = np.zeros((2 * I, H)); wgu2[:I, 0] = [0.5, -1.0, 2.0, 3.0]; wgu2[I:, 0] = 1.0
    wd2 = np.eye(H, I)
    out = ops.mlp(x, wgu2, wd2, I)
    expect = bfv(ops.silu(np.array([0.5, -1.0, 2.0, 3.0])))
    np.testing.assert_array_equal(out[0, :I], expect)


# --------------------------------------------------------------------- RoPE

def test_rope_identity_at_zero_and_half_split_closed_form():
    rng = np.random.default_rng(4)
    d, theta = 16, 1e6
    x = bfv(rng.standard_normal((1, 2, d)))
    np.testing.assert_array_equal(ops.rope(x, [0], theta), x)
    # unit vector at index i rotates into index i + d/2 (NeoX half-split pairing)
    e = np.zeros((1, 1, d)); e[0, 0, 1] = 1.0
    t = 7
    inv1 = theta ** (-2.0 * 1 / d)
    out = ops.rope(e, [t], theta)
    assert out[0, 0, 1] == bfv(np.float32(math.cos(t * inv1)))
    assert out[0, 0, 1 + d // 2] == bfv(np.float32(math.sin(t * inv1)))
    assert np.count_nonzero(out) == 2


def test_rope_relative_position_invariance():
    rng = np.random.default_rng(5)
    d, theta = 32, 10000.0
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    c, s = ops.rope_tables(np.arange(0, 40), d, theta)

    def rot(v, t):  # fp64, no rounding: the mathematical rotation with the fp32 table
        a, b = v[: d // 2], v[d // 2:]
        return np.concatenate([a * c[t] - b * s[t], b * c[t] + a * s[t]])
    dots = [rot(q, t + 5) @ rot(k, t) for t in range(0, 30)]
    assert np.ptp(dots) < 1e-5                   # fp32 table error only
    for t in (0, 3, 17):
        assert abs(np.linalg.norm(rot(q, t)) - np.linalg.norm(q)) < 1e-6


# ---------------------------------------------------------------- FP8 cache

def test_kv_quantise_rule():
    rng = np.random.default_rng(6)
    x = bfv(rng.standard_normal((5, 3, 128)) * 3.0)
    x[0, 0] = 0.0
    codes, sig = ops.kv_quantise(x)
    assert sig.dtype == np.float32 and sig[0, 0] == 1.0
    amax = np.abs(x).max(axis=-1)
    np.testing.assert_array_equal(sig[amax > 0], (amax[amax > 0].astype(np.float32) / np.float32(448)))
    # the element with the largest magnitude maps to +-448 (code 0x7E / 0xFE)
    i = np.unravel_index(np.argmax(np.abs(x[1, 1])), (128,))[0]
    assert codes[1, 1, i] in (0x7E, 0xFE)
    xh = ops.kv_dequantise(codes, sig)
    rel = np.abs(xh - x) / np.maximum(amax[..., None], 1e-30)
    assert rel.max() <= 2.0 ** -4 * 448 / 256 + 2 ** -8   # half e4m3 ulp at top binade + bf16
    # the dequantised value is exactly bf(fp32(code) * sigma)
    prod = e4m3_decode(codes).astype(np.float32) * sig[..., None]
    np.testing.assert_array_equal(xh, bfv(prod.astype(np.float64)))


def test_kv_quantise_matches_torch_scaled_cast():
    rng = np.random.default_rng(7)
    x = bfv(rng.standard_normal((64, 128)))
    codes, sig = ops.kv_quantise(x)
    xt = torch.from_numpy(x.astype(np.float32))
    st = torch.from_numpy(sig)
    ref = (xt / st[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, ref)


# ---------------------------------------------------------------- attention

def test_attention_first_position_returns_v0():
    rng = np.random.default_rng(8)
    q = bfv(rng.standard_normal((1, 4, 16)))
    k = bfv(rng.standard_normal((3, 2, 16)))
    v = bfv(rng.standard_normal((3, 2, 16)))
    o = ops.causal_gqa_attention(q, k, v, [0])
    np.testing.assert_array_equal(o[0, 0], v[0, 0])
    np.testing.assert_array_equal(o[0, 1], v[0, 0])
    np.testing.assert_array_equal(o[0, 2], v[0, 1])       # heads 2,3 use kv head 1
    np.testing.assert_array_equal(o[0, 3], v[0, 1])


def test_attention_equal_keys_give_mean_and_causality():
    rng = np.random.default_rng(9)
    T, d = 6, 8
    q = bfv(rng.standard_normal((T, 2, d)))
    k = np.repeat(bfv(rng.standard_normal((1, 1, d))), T, axis=0)
    v = bfv(rng.standard_normal((T, 1, d)))
    o = ops.causal_gqa_attention(q, k, v, np.arange(T))
    for t in range(T):
        np.testing.assert_allclose(o[t, 0], bfv(v[: t + 1, 0].mean(axis=0)), rtol=0, atol=0)
    # output at t does not depend on keys/values after t
    k2, v2 = k.copy(), v.copy()
    k2[4:] = 7.0
    v2[4:] = -3.0
    o2 = ops.causal_gqa_attention(q, k2, v2, np.arange(T))
    np.testing.assert_array_equal(o[:4], o2[:4])


def test_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(10)
    T, nq, nkv, d = 37, 8, 2, 32
    q = bfv(rng.standard_normal((T, nq, d)))
    k = bfv(rng.standard_normal((T, nkv, d)))
    v = bfv(rng.standard_normal((T, nkv, d)))
    pos = np.arange(T)
    o = ops.causal_gqa_attention(q, k, v, pos)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(nq // nkv, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(nq // nkv, dim=0)
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True).permute(1, 0, 2).numpy()
    # fp64 on both sides: equal up to a rare bf16 rounding-boundary flip (1 ulp)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(o - bfv(ref)) <= ulp)
    assert np.mean(o == bfv(ref)) > 0.999


def test_attention_offset_queries_match_full():
    # queries at positions 10..12 against keys 0..12 equal the tail of the full computation
    rng = np.random.default_rng(11)
    T, d = 13, 16
    q = bfv(rng.standard_normal((T, 2, d)))
    k = bfv(rng.standard_normal((T, 1, d)))
    v = bfv(rng.standard_normal((T, 1, d)))
    full = ops.causal_gqa_attention(q, k, v, np.arange(T))
    tail = ops.causal_gqa_attention(q[10:], k, v, np.arange(10, 13))
    np.testing.assert_array_equal(full[10:], tail)


# ----------------------------------------------------------------- logprobs

def _emb_bits(V, H, scale, seed):
    from oracle.codecs import bf16_encode
    rng = np.random.default_rng(seed)
    return bf16_encode(rng.standard_normal((V, H)) * scale)


def test_logprobs_zero_weight_is_minus_log_v():
    V, H = 1000, 16
    emb = np.zeros((V, H), dtype=np.uint16)
    hf = bfv(np.random.default_rng(12).standard_normal((3, H)))
    lp = ops.logprobs(hf, emb, [0, 5, 999])
    np.testing.assert_array_equal(lp, np.float32(-math.log(V)))


def test_logprobs_normalised_and_match_torch():
    V, H = 3000, 32
    emb = _emb_bits(V, H, 0.3, 13)
    hf = bfv(np.random.default_rng(14).standard_normal((5, H)))
    full = ops.full_logprobs(hf, emb)
    assert np.all(full <= 0)
    np.testing.assert_allclose(np.exp(full).sum(axis=1), 1.0, atol=1e-9)
    ids = np.array([0, 17, 2999, 1500, 7])
    lp = ops.logprobs(hf, emb, ids, vocab_block=700)        # block split must not matter
    from oracle.codecs import bf16_decode
    ref = torch.log_softmax(torch.from_numpy(hf) @ torch.from_numpy(bf16_decode(emb)).T, dim=1)
    ref = ref[torch.arange(5), torch.from_numpy(ids)].numpy().astype(np.float32)
    np.testing.assert_array_equal(lp, ref)


# ---------------------------------------------------------------------- MoE

def test_topk_ties_brute_force_and_special_cases():
    rng = np.random.default_rng(15)
    z = rng.integers(-8, 9, size=(50, 64)).astype(np.float64) / 4
    ids = ops.topk_ties(z, 6)
    for t in range(50):
        np.testing.assert_array_equal(ids[t], np.lexsort((np.arange(64), -z[t]))[:6])
    np.testing.assert_array_equal(ops.topk_ties(np.zeros((1, 64)), 6)[0], [0, 1, 2, 3, 4, 5])
    # 7-way tie straddling rank 6: the 3 lowest indices of the tie fill slots 3..5
    row = np.full(64, -1.0); row[[40, 50, 60]] = 2.0; row[[3, 9, 11, 20, 33, 41, 62]] = 1.0
    np.testing.assert_array_equal(ops.topk_ties(row[None], 6)[0], [40, 50, 60, 3, 9, 11])
    # without ties, permuting columns permutes the ids
    zz = rng.permutation(64).astype(np.float64)[None]
    perm = rng.permutation(64)
    a = ops.topk_ties(zz, 6)[0]
    b = ops.topk_ties(zz[:, perm], 6)[0]
    np.testing.assert_array_equal(perm[b], a)


def test_topk_weights_softmax():
    z = np.array([[2.0, 1.0, 0.0, -1.0]])
    ids = np.array([[0, 1, 2]])
    w = ops.topk_weights(z, ids)
    e = np.exp([2.0, 1.0, 0.0])
    np.testing.assert_allclose(w[0], e / e.sum(), rtol=1e-15)
    np.testing.assert_allclose(w.sum(), 1.0, atol=1e-15)


def test_moe_layer_brute_force_per_token():
    from oracle.codecs import bf16_encode
    rng = np.random.default_rng(16)
    T, H, I, E, k = 5, 16, 8, 6, 2
    h = bfv(rng.standard_normal((T, H)))
    wgu = bf16_encode(rng.standard_normal((E, 2 * I, H)) * 0.3)
    wd = bf16_encode(rng.standard_normal((E, H, I)) * 0.3)
    swgu = bf16_encode(rng.standard_normal((2 * I, H)) * 0.3)
    swd = bf16_encode(rng.standard_normal((H, I)) * 0.3)
    z = rng.integers(-4, 5, size=(T, E)) / 4.0
    ids = ops.topk_ties(z, k)
    w = ops.topk_weights(z, ids)
    out = ops.moe_layer(h, ids, w, wgu, wd, swgu, swd, I)
    from oracle.codecs import bf16_decode as d
    for t in range(T):
        acc = ops.mlp(h[t:t + 1], d(swgu), d(swd), I)[0]
        for s in range(k):
            e = ids[t, s]
            acc = acc + w[t, s] * ops.mlp(h[t:t + 1], d(wgu[e]), d(wd[e]), I)[0]
        np.testing.assert_array_equal(out[t], bfv(acc))
    # identical routed experts: the gated sum equals one expert (weights sum to 1)
    wgu_same = np.repeat(wgu[:1], E, axis=0)
    wd_same = np.repeat(wd[:1], E, axis=0)
    out2 = ops.moe_layer(h, ids, w, wgu_same, wd_same, swgu, swd, I)
    y = ops.mlp(h, d(wgu[0]), d(wd[0]), I) + ops.mlp(h, d(swgu), d(swd), I)
    np.testing.assert_allclose(out2, bfv(y), rtol=2 ** -7, atol=1e-12)


# ------------------------------------------------------------- acceptance

def test_acceptance_stats_closed_forms():
    a = np.array([-1.0, -2.0, -3.0], np.float32)
    s = ops.acceptance_stats(a, a.copy())
    assert s == dict(max=0.0, mean=0.0, std=0.0, k3=0.0)
    d = math.log(2.0)
    s = ops.acceptance_stats(np.array([d]), np.array([0.0]))
    assert abs(s["k3"] - (1.0 - math.log(2.0))) < 1e-15
    # small delta: k3 ~ delta^2 / 2, computed without cancellation
    s = ops.acceptance_stats(np.array([1e-6]), np.array([0.0]))
    assert abs(s["k3"] / 0.5e-12 - 1.0) < 1e-5
    s = ops.acceptance_stats(np.array([0.1, -0.1]), np.zeros(2))
    assert s["max"] == 0.1 and abs(s["mean"] - 0.1) < 1e-17 and abs(s["std"] - 0.1) < 1e-17
