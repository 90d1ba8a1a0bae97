"""GPU parity (HIP op vs the fp64 oracle) and batch-invariance (HIP vs itself) of each
libbci operator, called through the C ABI."""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import BF, assert_bf16_close, cuda, f64, same_bits
from oracle import codecs, ops

pytestmark = pytest.mark.gpu


def abi():
    from bitwise_consistent_rl_amd import _abi
    return _abi


def make_ctx(n_layers=1, hidden=2048, nq=16, nkv=8, d=128, inter=6144, vocab=151936, kv="bf16",
             max_tokens=4096, max_seqs=64, max_scored=8192, max_position=2048, seg=2048, split=0):
    a = abi()
    c = a.ModelConfig()
    for k, v in dict(n_layers=n_layers, hidden=hidden, n_q_heads=nq, n_kv_heads=nkv, head_dim=d,
                     intermediate=inter, vocab=vocab, rms_eps=1e-6, rope_theta=1e6,
                     kv_dtype=a.BCI_KV_FP8_E4M3 if kv == "fp8" else a.BCI_KV_BF16,
                     kv_block_tokens=64, attn_segment_keys=seg, max_tokens_per_call=max_tokens,
                     max_seqs_per_call=max_seqs, max_scored_per_call=max_scored,
                     max_position=max_position, mode=a.BCI_MODE_INVARIANT,
                     attn_split_mode=split).items():
        setattr(c, k, v)
    return a.bci_create(c, 0)


@pytest.fixture(scope="module")
def ctx():
    h = make_ctx()
    yield h
    torch.cuda.synchronize()
    abi().bci_destroy(h)


def gemm(ctx, a, w, epi, out_cols=None, dtype=BF):
    M, K = a.shape
    N = w.shape[0]
    C = torch.empty(M, out_cols or N, dtype=dtype, device="cuda")
    abi().bci_op_gemm_bf16(ctx, a, w, C, M, N, K, epi)
    torch.cuda.synchronize()
    return C


# ------------------------------------------------------------------- GEMM

@pytest.mark.parametrize("M,N,K", [(1, 128, 64), (37, 256, 128), (24, 256, 2048), (64, 512, 6144),
                                   (300, 512, 256), (513, 384, 2048), (256, 128, 6144),
                                   (1000, 4096, 2048), (3, 1024, 2048), (4, 2032, 1024)])
def test_gemm_bf16_parity(ctx, M, N, K):
    a, w = synth.gemm_inputs(M, N, K, index=M + N + K)
    C = gemm(ctx, cuda(a), cuda(w), abi().BCI_EPI_BF16)
    A, W = f64(a), f64(w)
    ref = ops.bf(ops.linear(A, W))
    mag = np.abs(A) @ np.abs(W).T
    assert_bf16_close(f64(C), ref, abs_bound=K * 2.0 ** -24 * mag, max_ulp=1, frac_exact=0.999,
                      what=f"gemm {M}x{N}x{K}")


def _ksplit(ctx, a, w, epi, k_split):
    M, K = a.shape
    N = w.shape[0]
    C = torch.empty(M, N, dtype=torch.float32 if epi == abi().BCI_EPI_F32 else BF, device="cuda")
    ws = torch.empty((K + k_split - 1) // k_split * M * N, dtype=torch.float32, device="cuda")
    abi().bci_op_gemm_bf16_ksplit(ctx, a, w, C, M, N, K, k_split, epi, ws)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("M,N,K,k_split", [(37, 300, 2368, 256), (300, 512, 4096, 1024), (5, 128, 64, 64)])
def test_gemm_ksplit(ctx, M, N, K, k_split):
    """Contraction in fixed slices (the last one shorter when K % k_split != 0): within
    the fp32 bound of the oracle's product, equal bit for bit to the fp32 sum, in slice
    order, of the single-slice GEMMs, rows independent of M, and repeatable."""
    a, w = synth.gemm_inputs(M, N, K, index=M + N + K + k_split)
    ga, gw = cuda(a), cuda(w)
    c32 = _ksplit(ctx, ga, gw, abi().BCI_EPI_F32, k_split)
    cbf = _ksplit(ctx, ga, gw, abi().BCI_EPI_BF16, k_split)
    A, W = f64(a), f64(w)
    ref = ops.linear(A, W)
    mag = np.abs(A) @ np.abs(W).T
    got = c32.cpu().numpy()
    assert np.all(np.abs(got - ref) <= K * 2.0 ** -24 * mag + 1e-30)
    assert_bf16_close(f64(cbf), ops.bf(ref), abs_bound=K * 2.0 ** -24 * mag, max_ulp=1, frac_exact=0.999,
                      what=f"ksplit {M}x{N}x{K}/{k_split}")
    # the slices' own GEMMs (contiguous copies of the column slices), summed in order in fp32
    acc = None
    for k0 in range(0, K, k_split):
        k1 = min(K, k0 + k_split)
        part = gemm(ctx, ga[:, k0:k1].contiguous(), gw[:, k0:k1].contiguous(), abi().BCI_EPI_F32,
                    dtype=torch.float32).cpu().numpy()
        acc = part if acc is None else (acc + part).astype(np.float32)
    assert np.array_equal(got.view(np.int32), acc.view(np.int32))
    assert same_bits(cbf, torch.from_numpy(acc).to(BF))
    sub = slice(M // 3, M // 3 + min(3, M))
    assert same_bits(_ksplit(ctx, ga[sub].contiguous(), gw, abi().BCI_EPI_F32, k_split), c32[sub])
    assert same_bits(_ksplit(ctx, ga, gw, abi().BCI_EPI_F32, k_split), c32)


def test_gemm_ksplit_rejects_bad_arguments(ctx):
    a, w = synth.gemm_inputs(4, 64, 128, index=3)
    ga, gw = cuda(a), cuda(w)
    C = torch.empty(4, 64, dtype=BF, device="cuda")
    ws = torch.empty(4 * 64 * 2, dtype=torch.float32, device="cuda")
    for k_split, epi in ((96, abi().BCI_EPI_BF16), (0, abi().BCI_EPI_BF16), (64, abi().BCI_EPI_SILU_MUL)):
        with pytest.raises(abi().BciError):
            abi().bci_op_gemm_bf16_ksplit(ctx, ga, gw, C, 4, 64, 128, k_split, epi, ws)


def test_gemm_f32_epilogue_parity(ctx):
    M, N, K = 129, 256, 2048
    a, w = synth.gemm_inputs(M, N, K, index=11)
    C = gemm(ctx, cuda(a), cuda(w), abi().BCI_EPI_F32, dtype=torch.float32).cpu().numpy()
    A, W = f64(a), f64(w)
    ref = ops.linear(A, W)
    mag = np.abs(A) @ np.abs(W).T
    assert np.all(np.abs(C - ref) <= K * 2.0 ** -24 * mag + 1e-30)


def test_gemm_silu_mul_epilogue_parity(ctx):
    M, I, K = 77, 384, 256
    a, w = synth.gemm_inputs(M, 2 * I, K, index=12, w_scale=0.1)
    C = gemm(ctx, cuda(a), cuda(w), abi().BCI_EPI_SILU_MUL, out_cols=I)
    A, W = f64(a), f64(w)
    gu = ops.bf(ops.linear(A, W))
    ref = ops.silu_mul(gu[:, :I], gu[:, I:])
    mag = (np.abs(A) @ np.abs(W).T)
    bound = K * 2.0 ** -24 * (mag[:, :I] + mag[:, I:]) * 4
    assert_bf16_close(f64(C), ref, abs_bound=bound, max_ulp=2, frac_exact=0.99, what="silu")


def test_gemm_silu_equals_unfused(ctx):
    """The fused SiLU*up epilogue equals a bf16 GEMM followed by silu(g)*u on the same bits."""
    M, I, K = 300, 256, 512
    a, w = synth.gemm_inputs(M, 2 * I, K, index=13, w_scale=0.1)
    ga, gw = cuda(a), cuda(w)
    fused = gemm(ctx, ga, gw, abi().BCI_EPI_SILU_MUL, out_cols=I)
    gu = f64(gemm(ctx, ga, gw, abi().BCI_EPI_BF16))
    ref = ops.silu_mul(gu[:, :I], gu[:, I:])
    # only the fp32-vs-fp64 silu evaluation differs: at most one bf16 ulp
    assert_bf16_close(f64(fused), ref, max_ulp=1, frac_exact=0.99, what="fused vs unfused")


@pytest.mark.parametrize("epi", ["bf16", "silu"])
def test_gemm_rows_invariant_to_M_and_order(ctx, epi):
    a_ = abi()
    K, N = 2048, 512
    a, w = synth.gemm_inputs(4096, N, K, index=14)
    ga, gw = cuda(a), cuda(w)
    e = a_.BCI_EPI_BF16 if epi == "bf16" else a_.BCI_EPI_SILU_MUL
    cols = N if epi == "bf16" else N // 2
    full = gemm(ctx, ga, gw, e, out_cols=cols)
    for M in (1, 2, 7, 24, 64, 255, 256, 257, 1000, 4095):
        part = gemm(ctx, ga[:M].contiguous(), gw, e, out_cols=cols)
        assert same_bits(part, full[:M]), M
    perm = torch.from_numpy(np.array(synth.shuffled(list(range(4096))))).cuda()
    shuf = gemm(ctx, ga[perm].contiguous(), gw, e, out_cols=cols)
    assert same_bits(shuf, full[perm])
    # a row surrounded by different neighbours
    other = cuda(synth.normal_bf16((300, K), index=15))
    mix = torch.cat([other[:150], ga[17:18], other[150:]]).contiguous()
    out = gemm(ctx, mix, gw, e, out_cols=cols)
    assert same_bits(out[150:151], full[17:18])


@pytest.mark.parametrize("N,K,epi", [(12288, 2048, "silu"), (4096, 2048, "bf16"), (2048, 6144, "bf16")])
def test_gemm_mid_m_schedule_choice_bitwise(ctx, N, K, epi):
    """Between 129 and 512 rows each launch takes the skinny or the tiled schedule by a
    latency model of its shape (at these widths the choice flips with M: gate_up goes to
    tiles above 128 rows, QKV above ~400, down stays skinny to 512); every row must equal
    the same row of a 1024-row call, which runs on tiles."""
    a_ = abi()
    a, w = synth.gemm_inputs(1024, N, K, index=N + K)
    ga, gw = cuda(a), cuda(w)
    e = a_.BCI_EPI_BF16 if epi == "bf16" else a_.BCI_EPI_SILU_MUL
    cols = N if epi == "bf16" else N // 2
    full = gemm(ctx, ga, gw, e, out_cols=cols)
    for M in (100, 129, 160, 256, 384, 511, 512, 600):
        part = gemm(ctx, ga[1024 - M:].contiguous(), gw, e, out_cols=cols)
        assert same_bits(part, full[1024 - M:]), (N, K, M)


def test_gemm_rejects_bad_shapes(ctx):
    a_ = abi()
    x = torch.empty(4, 64, dtype=BF, device="cuda")
    with pytest.raises(a_.BciError):
        a_.bci_op_gemm_bf16(ctx, x, x, x, 4, 128, 48, a_.BCI_EPI_BF16)   # K % 64
    with pytest.raises(a_.BciError):
        a_.bci_op_gemm_bf16(ctx, x, x, x, 4, 384, 64, a_.BCI_EPI_SILU_MUL)   # I % 128
    with pytest.raises(a_.BciError):
        a_.bci_op_gemm_bf16(ctx, x, x, x, 4, 128, 64, 7)   # unknown epilogue
    y = torch.empty(4 * 64 + 8, dtype=BF, device="cuda")
    with pytest.raises(a_.BciError):   # A 2 bytes past a 16-byte boundary
        a_.bci_op_gemm_bf16(ctx, y[1:], x, x, 4, 4, 64, a_.BCI_EPI_BF16)
    with pytest.raises(a_.BciError):   # W likewise
        a_.bci_op_gemm_bf16(ctx, x, y[1:], x, 4, 4, 64, a_.BCI_EPI_BF16)


def test_gemm_ragged_n_parity_and_invariance(ctx):
    """N not a multiple of the 128-column tile: the tail columns are masked."""
    M, N, K = 300, 200, 256
    a, w = synth.gemm_inputs(M, N, K, index=16)
    ga, gw = cuda(a), cuda(w)
    C = gemm(ctx, ga, gw, abi().BCI_EPI_BF16)
    A, W = f64(a), f64(w)
    mag = np.abs(A) @ np.abs(W).T
    assert_bf16_close(f64(C), ops.bf(ops.linear(A, W)), abs_bound=K * 2.0 ** -24 * mag,
                      max_ulp=1, frac_exact=0.999, what="ragged N")
    assert same_bits(gemm(ctx, ga[5:6].contiguous(), gw, abi().BCI_EPI_BF16), C[5:6])


# ----------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("rows,cols,with_add", [(37, 2048, True), (5, 256, False), (64, 4096, True)])
def test_add_rmsnorm_parity(ctx, rows, cols, with_add):
    a_ = abi()
    x = synth.normal_bf16((rows, cols), index=20)
    r = synth.normal_bf16((rows, cols), index=21)
    g = synth.to_bf16(1 + 0.02 * np.random.default_rng(0).standard_normal(cols).astype(np.float32))
    gr, gh = cuda(r.clone()), torch.empty(rows, cols, dtype=BF, device="cuda")
    a_.bci_op_add_rmsnorm(ctx, cuda(x) if with_add else None, gr, gh, cuda(g), rows, cols, 1e-6)
    torch.cuda.synchronize()
    rr, hh = ops.add_rmsnorm(f64(x) if with_add else None, f64(r), f64(g), 1e-6)
    assert_bf16_close(f64(gr), rr, max_ulp=1, frac_exact=0.999, what="residual")
    assert_bf16_close(f64(gh), hh, max_ulp=1, frac_exact=0.99, what="norm")


def test_add_rmsnorm_row_invariance(ctx):
    a_ = abi()
    cols = 2048
    x = cuda(synth.normal_bf16((512, cols), index=22))
    r0 = cuda(synth.normal_bf16((512, cols), index=23))
    g = cuda(synth.to_bf16(np.ones(cols, np.float32)))

    def run(idx):
        r = r0[idx].contiguous()
        h = torch.empty_like(r)
        a_.bci_op_add_rmsnorm(ctx, x[idx].contiguous(), r, h, g, len(idx), cols, 1e-6)
        torch.cuda.synchronize()
        return r, h
    rf, hf = run(torch.arange(512, device="cuda"))
    r1, h1 = run(torch.tensor([300], device="cuda"))
    assert same_bits(h1, hf[300:301]) and same_bits(r1, rf[300:301])


# ----------------------------------------------------------------- lm_head

@pytest.fixture(scope="module")
def lm_inputs():
    hs, w, ids = synth.lmhead_inputs(8192)
    return hs, w, ids, cuda(hs), cuda(w), torch.from_numpy(ids).cuda()


def lmhead(ctx, hs, w, ids, V=None):
    M, H = hs.shape
    V = V or w.shape[0]
    lp = torch.empty(M, dtype=torch.float32, device="cuda")
    abi().bci_op_lmhead_logprob(ctx, hs, w, ids, M, H, V, lp)
    torch.cuda.synchronize()
    return lp


@pytest.mark.parametrize("M", [1, 7, 64])
def test_lmhead_logprob_parity_full_vocab(ctx, lm_inputs, M):
    hs, w, ids, ghs, gw, gids = lm_inputs
    lp = lmhead(ctx, ghs[:M].contiguous(), gw, gids[:M].contiguous()).cpu().numpy()
    ref = ops.logprobs(f64(hs[:M]), synth.bf16_bits(w), ids[:M])
    assert np.all(lp <= 0)
    assert np.max(np.abs(lp - ref)) <= 1e-3, np.max(np.abs(lp - ref))


def test_lmhead_rows_invariant_across_M(ctx, lm_inputs):
    hs, w, ids, ghs, gw, gids = lm_inputs
    full = lmhead(ctx, ghs, gw, gids)
    for M in (1, 7, 64, 512, 4096):
        part = lmhead(ctx, ghs[:M].contiguous(), gw, gids[:M].contiguous())
        assert same_bits(part, full[:M]), M
    perm = torch.from_numpy(np.array(synth.shuffled(list(range(8192)), index=3))).cuda()
    shuf = lmhead(ctx, ghs[perm].contiguous(), gw, gids[perm].contiguous())
    assert same_bits(shuf, full[perm])


def test_lmhead_ragged_vocab_and_normalisation(ctx):
    """V = 4000 (last 256-column chunk partial): one hidden state scored against every
    id gives the full distribution; sum exp(lp) = 1 and each lp matches the oracle."""
    H, V = 256, 4000
    hs = synth.normal_bf16((1, H), index=30)
    w = synth.normal_bf16((V, H), index=31, scale=0.1)
    ghs = cuda(hs).expand(V, H).contiguous()
    ids = torch.arange(V, dtype=torch.int32, device="cuda")
    lp = lmhead(ctx, ghs, cuda(w), ids, V).cpu().numpy().astype(np.float64)
    assert abs(np.exp(lp).sum() - 1.0) < 1e-4
    ref = ops.full_logprobs(f64(hs), synth.bf16_bits(w))[0]
    assert np.max(np.abs(lp - ref)) < 1e-4


def test_lmhead_zero_weight_is_minus_log_v(ctx):
    H, V = 2048, 151936
    w = torch.zeros(V, H, dtype=BF, device="cuda")
    hs = cuda(synth.normal_bf16((3, H), index=32))
    ids = torch.tensor([0, 5, V - 1], dtype=torch.int32, device="cuda")
    lp = lmhead(ctx, hs, w, ids).cpu().numpy()
    assert np.all(np.abs(lp.astype(np.float64) + math.log(V)) < 2e-6)
    bad = torch.tensor([-1, V, 3], dtype=torch.int32, device="cuda")
    lp2 = lmhead(ctx, hs, w, bad).cpu().numpy()
    assert np.isnan(lp2[0]) and np.isnan(lp2[1]) and not np.isnan(lp2[2])


# ------------------------------------------------- RoPE, KV write, attention

def _batch_for(lengths, pos0=None, blocks_per_seq=None):
    """Whole sequences (or given start positions) with consecutive block ids."""
    pos0 = pos0 or [0] * len(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    maxb = max((p + L + 63) // 64 for p, L in zip(pos0, lengths))
    bt, nxt = [], 0
    for p, L in zip(pos0, lengths):
        nb = (p + L + 63) // 64
        bt.append(list(range(nxt, nxt + nb)) + [0] * (maxb - nb))
        nxt += nb
    return cu, np.array(pos0, np.int32), np.array(bt, np.int32), nxt


def _alloc_cache(n_layers, n_blocks, nkv, d, kv):
    shape = (n_layers, n_blocks, nkv, 64, d)
    if kv == "fp8":
        k = torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda")   # NaN codes: unwritten
        v = torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda")
        ks = torch.full(shape[:-1], float("nan"), device="cuda")
        vs = torch.full(shape[:-1], float("nan"), device="cuda")
        return k, v, ks, vs
    k = torch.full(shape, float("nan"), dtype=BF, device="cuda")
    v = torch.full(shape, float("nan"), dtype=BF, device="cuda")
    return k, v, None, None


HEADS = [(4, 2, 64), (16, 8, 128), (32, 4, 128)]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("nq,nkv,d", HEADS)
def test_rope_kv_write_and_gather(nq, nkv, d, kv):
    a_ = abi()
    lengths = [5, 70, 130, 1, 200]
    cu, pos0, bt, nb = _batch_for(lengths)
    T = int(cu[-1])
    width = (nq + 2 * nkv) * d
    qkv = synth.normal_bf16((T, width), index=40)
    ctxs, out = {}, {}
    for mode in ("bf16", kv):
        h = make_ctx(hidden=512, nq=nq, nkv=nkv, d=d, inter=512, vocab=4096, kv=mode)
        cache = _alloc_cache(1, nb, nkv, d, mode)
        a_.bci_bind_kv_cache(h, *cache, nb)
        a_.bci_set_batch(h, np.zeros(T, np.int32), cu, pos0, bt, [], [])
        q = torch.empty(T, nq * d, dtype=BF, device="cuda")
        a_.bci_op_rope_kv_write(h, cuda(qkv), q, 0)
        ks, vs = [], []
        for i, L in enumerate(lengths):
            ko = torch.empty(L, nkv, d, dtype=BF, device="cuda")
            vo = torch.empty(L, nkv, d, dtype=BF, device="cuda")
            a_.bci_op_kv_gather_dequant(h, i, L, 0, ko, vo)
            ks.append(ko)
            vs.append(vo)
        torch.cuda.synchronize()
        out[mode] = (q, torch.cat(ks), torch.cat(vs), cache)
        ctxs[mode] = h
    q, kb, vb, _ = out["bf16"]
    pos = np.concatenate([np.arange(L) for L in lengths])
    X = f64(qkv)
    qr = ops.rope(X[:, : nq * d].reshape(T, nq, d), pos, 1e6)
    kr = ops.rope(X[:, nq * d:(nq + nkv) * d].reshape(T, nkv, d), pos, 1e6)
    # x1*c - x2*s can cancel: the fp32 rounding of the two products (2^-24 relative
    # each) then dominates a tiny result, so allow it on top of 1 ulp.
    def cancel(x):
        a = np.abs(x[..., : d // 2]) + np.abs(x[..., d // 2:])
        return 2.0 ** -22 * np.concatenate([a, a], axis=-1)
    Xq = X[:, : nq * d].reshape(T, nq, d)
    Xk = X[:, nq * d:(nq + nkv) * d].reshape(T, nkv, d)
    assert_bf16_close(f64(q).reshape(T, nq, d), qr, abs_bound=cancel(Xq), max_ulp=1,
                      frac_exact=0.999, what="q rope")
    assert_bf16_close(f64(kb), kr, abs_bound=cancel(Xk), max_ulp=1, frac_exact=0.999, what="k rope")
    np.testing.assert_array_equal(f64(vb), X[:, (nq + nkv) * d:].reshape(T, nkv, d))
    if kv == "fp8":
        _, kf, vf, (kc, vc, ksc, vsc) = out["fp8"]
        # same bf16 inputs -> bit-identical codes, scales and dequantised values
        for src, got_deq, codes_t, sc_t in ((f64(kb), kf, kc, ksc), (f64(vb), vf, vc, vsc)):
            codes, sig = ops.kv_quantise(src)
            np.testing.assert_array_equal(f64(got_deq), ops.kv_dequantise(codes, sig))
            for i, L in enumerate(lengths):
                rows = np.arange(L)
                blk = bt[i][rows // 64]
                off = rows % 64
                got_c = codes_t[0].cpu().numpy()[blk, :, off, :]
                got_s = sc_t[0].cpu().numpy()[blk, :, off]
                np.testing.assert_array_equal(got_c, codes[cu[i]:cu[i + 1]])
                np.testing.assert_array_equal(got_s, sig[cu[i]:cu[i + 1]])
    for h in ctxs.values():
        a_.bci_destroy(h)


def _attention_run(nq, nkv, d, kv, seg, lengths, qkv, calls, split=0):
    """Runs RoPE+KV write then attention for a sequence of calls, each a list of
    (seq, start, n) chunks; returns o for every (seq, position) and the rotated q."""
    a_ = abi()
    h = make_ctx(hidden=512, nq=nq, nkv=nkv, d=d, inter=512, vocab=4096, kv=kv, seg=seg,
                 split=split)
    n_blocks = sum((L + 63) // 64 for L in lengths)
    cache = _alloc_cache(1, n_blocks, nkv, d, kv)
    a_.bci_bind_kv_cache(h, *cache, n_blocks)
    blocks, nxt = [], 0
    for L in lengths:
        nb = (L + 63) // 64
        blocks.append(list(range(nxt, nxt + nb)))
        nxt += nb
    offs = np.concatenate([[0], np.cumsum(lengths)])
    gq = cuda(qkv)
    o_all = torch.empty(int(offs[-1]), nq * d, dtype=BF, device="cuda")
    q_all = torch.empty(int(offs[-1]), nq * d, dtype=BF, device="cuda")
    for call in calls:
        rows = np.concatenate([np.arange(offs[s] + p, offs[s] + p + n) for s, p, n in call])
        rows_t = torch.from_numpy(rows).cuda()
        cu = np.concatenate([[0], np.cumsum([n for _, _, n in call])]).astype(np.int32)
        maxb = max(len(blocks[s]) for s, _, _ in call)
        bt = np.array([blocks[s] + [0] * (maxb - len(blocks[s])) for s, _, _ in call], np.int32)
        T = len(rows)
        a_.bci_set_batch(h, np.zeros(T, np.int32), cu, np.array([p for _, p, _ in call], np.int32),
                         bt, [], [])
        q = torch.empty(T, nq * d, dtype=BF, device="cuda")
        o = torch.empty(T, nq * d, dtype=BF, device="cuda")
        a_.bci_op_rope_kv_write(h, gq[rows_t].contiguous(), q, 0)
        a_.bci_op_attention(h, q, 0, o)
        o_all[rows_t] = o
        q_all[rows_t] = q
    # gather the final cache for the oracle
    kvs = []
    a_.bci_set_batch(h, np.zeros(len(lengths), np.int32), np.arange(len(lengths) + 1, dtype=np.int32),
                     np.array([L - 1 for L in lengths], np.int32),
                     np.array([b + [0] * (max(map(len, blocks)) - len(b)) for b in blocks], np.int32),
                     [], [])
    for i, L in enumerate(lengths):
        ko = torch.empty(L, nkv, d, dtype=BF, device="cuda")
        vo = torch.empty(L, nkv, d, dtype=BF, device="cuda")
        a_.bci_op_kv_gather_dequant(h, i, L, 0, ko, vo)
        kvs.append((ko, vo))
    torch.cuda.synchronize()
    a_.bci_destroy(h)
    return o_all, q_all, kvs


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("nq,nkv,d,seg", [(4, 2, 64, 2048), (16, 8, 128, 2048), (32, 4, 128, 128),
                                          (16, 8, 128, 64)])
def test_attention_parity(nq, nkv, d, seg, kv):
    lengths = [3, 64, 65, 200, 331]
    T = sum(lengths)
    qkv = synth.normal_bf16((T, (nq + 2 * nkv) * d), index=41)
    calls = [[(i, 0, L) for i, L in enumerate(lengths)]]
    o, q, kvs = _attention_run(nq, nkv, d, kv, seg, lengths, qkv, calls)
    offs = np.concatenate([[0], np.cumsum(lengths)])
    X = f64(qkv)
    for i, L in enumerate(lengths):
        # the oracle's own rotation (and FP8 round trip) of the same qkv rows
        Xi = X[offs[i]:offs[i + 1]]
        pos = np.arange(L)
        qi = ops.rope(Xi[:, : nq * d].reshape(L, nq, d), pos, 1e6)
        K = ops.rope(Xi[:, nq * d:(nq + nkv) * d].reshape(L, nkv, d), pos, 1e6)
        V = Xi[:, (nq + nkv) * d:].reshape(L, nkv, d)
        if kv == "fp8":
            K, V = ops.kv_roundtrip(K), ops.kv_roundtrip(V)
        ref = ops.causal_gqa_attention(qi, K, V, pos)
        got = f64(o[offs[i]:offs[i + 1]]).reshape(L, nq, d)
        err = np.abs(got - ref)
        scale = np.max(np.abs(V))
        assert err.max() <= 1.5e-2 * scale, (i, err.max())
        assert err.mean() <= 1.5e-3 * scale, (i, err.mean())


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("nq,nkv,d", [(4, 2, 64), (16, 8, 128)])
def test_attention_one_segment_schedule_bitwise(nq, nkv, d, kv):
    """A call whose positions all lie in the first segment runs the one-segment schedule
    (one LDS buffer, no segment state); the same rows in a call that also holds a sequence
    past the first segment run the general schedule.  Both give the same bits (the
    oracle comparison of the one-segment schedule is test_attention_parity's seg = 2048
    cases, whose calls all lie in the first segment)."""
    seg = 1024
    lengths = [150, 67, 1, 300, 1100]
    T = sum(lengths)
    qkv = synth.normal_bf16((T, (nq + 2 * nkv) * d), index=43)
    short = [(i, 0, L) for i, L in enumerate(lengths[:4])]
    o_one, _, _ = _attention_run(nq, nkv, d, kv, seg, lengths, qkv, [short, [(4, 0, 1100)]], split=1)
    o_gen, _, _ = _attention_run(nq, nkv, d, kv, seg, lengths, qkv, [short + [(4, 0, 1100)]], split=1)
    n_short = sum(lengths[:4])
    assert same_bits(o_one[:n_short], o_gen[:n_short])
    assert same_bits(o_one[n_short:], o_gen[n_short:])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("nq,nkv,d,seg", [(4, 2, 64, 128), (16, 8, 128, 2048), (32, 4, 128, 128)])
def test_attention_prefill_decode_chunked_bitwise(nq, nkv, d, seg, kv):
    """The same rows through whole prefill, token-by-token decode, chunked prefill and
    mixed batches give identical bits."""
    lengths = [150, 67, 1, 300]
    T = sum(lengths)
    qkv = synth.normal_bf16((T, (nq + 2 * nkv) * d), index=42)
    full = [[(i, 0, L) for i, L in enumerate(lengths)]]
    o_ref, _, _ = _attention_run(nq, nkv, d, kv, seg, lengths, qkv, full, split=1)
    # decode: one token per sequence per call, all sequences in each call; the KV
    # segments run in one workgroup each (split) or in sequence (never split)
    dec = []
    for t in range(max(lengths)):
        dec.append([(i, t, 1) for i, L in enumerate(lengths) if t < L])
    for split in (1, 2, 0):
        o_dec, _, _ = _attention_run(nq, nkv, d, kv, seg, lengths, qkv, dec, split=split)
        assert same_bits(o_dec, o_ref), split
    # chunked prefill with chunk 17 for seq 0 and 3, alone per call, others whole
    ch = [[(1, 0, 67)], [(2, 0, 1)]]
    for i in (0, 3):
        for s in range(0, lengths[i], 17):
            ch.append([(i, s, min(17, lengths[i] - s))])
    o_ch, _, _ = _attention_run(nq, nkv, d, kv, seg, lengths, qkv, ch)
    assert same_bits(o_ch, o_ref)
    # prompt prefill of 40 then decode, in a mixed batch with a chunked sequence
    mix = [[(0, 0, 40), (3, 0, 100)]]
    t0, t3 = 40, 100
    while t0 < 150 or t3 < 300:
        call = []
        if t0 < 150:
            call.append((0, t0, 1))
            t0 += 1
        if t3 < 300:
            n = min(33, 300 - t3)
            call.append((3, t3, n))
            t3 += n
        mix.append(call)
    mix += [[(1, 0, 67), (2, 0, 1)]]
    o_mix, _, _ = _attention_run(nq, nkv, d, kv, seg, lengths, qkv, mix)
    assert same_bits(o_mix, o_ref)
