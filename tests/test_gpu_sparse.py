"""Sparse attention over a Top-K selected key set on the FP8 KV path (32 q / 4 kv heads
of 128, e4m3 cache; indexer with 64 heads of 128).

Parity: the oracle builds its own rotated, FP8-round-tripped K/V and index keys from
the same seeded inputs, scores every key, selects the Top-K by (score desc, position
asc) and attends over the selected set.  With the integer index inputs of synth every
score is exact in any summation order, so scores and selections must match the oracle
bit for bit; attention outputs match within the bf16 tolerance of the dense operator.

Invariance: scores, selections and outputs of a token are bitwise the same in whole
prefill, chunked prefill (ragged chunks) and decode, in any batch, under both score
schedules; with every key selected the output equals the dense operator's bits on a
context with 256-key segments."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import BF, f64, same_bits
from oracle import ops, sparse
from test_gpu_ops import abi, make_ctx

pytestmark = pytest.mark.gpu

NQ, NKV, D = 32, 4, 128
HI, DI = 64, 128
WIDTH = (NQ + 2 * NKV) * D
THETA = 1e6


class SparseCtx:
    """A context holding the listed sequences; sequence i's inputs are rows
    [off_i, off_i + L_i) of the shared input buffers (off_i = i * 131)."""

    def __init__(self, lengths, max_tokens=4096, seg=256, inputs=None):
        a = abi()
        self.lengths = lengths
        self.max_position = max(lengths) + 64
        self.h = make_ctx(hidden=512, nq=NQ, nkv=NKV, d=D, inter=512, vocab=4096, kv="fp8",
                          max_tokens=max_tokens, max_seqs=64, max_scored=64,
                          max_position=self.max_position, seg=seg)
        self.blocks, nxt = [], 0
        for L in lengths:
            nb = (L + 63) // 64
            self.blocks.append(list(range(nxt, nxt + nb)))
            nxt += nb
        self.nb = nxt
        shape = (1, nxt, NKV, 64, D)
        self.k = torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda")
        self.v = torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda")
        self.ks = torch.full(shape[:-1], float("nan"), device="cuda")
        self.vs = torch.full(shape[:-1], float("nan"), device="cuda")
        self.ic = torch.full((nxt, 64, DI), 0x7F, dtype=torch.uint8, device="cuda")
        self.isc = torch.full((nxt, 64), float("nan"), device="cuda")
        a.bci_bind_kv_cache(self.h, self.k, self.v, self.ks, self.vs, nxt)
        self.maxb = max(len(b) for b in self.blocks)
        self.stride = (self.max_position + 3) // 4 * 4
        self.inp = inputs

    def rows(self, seq, start, n):
        return slice(seq * 131 + start, seq * 131 + start + n)

    def call(self, chunks, topk, schedule=0, attend=True):
        """chunks: list of (seq, start, n).  Writes K/V and index keys of those tokens,
        then (attend) scores, selects and attends.  Returns (scores, sel, o) on the GPU."""
        a = abi()
        qkv, qidx, w, kidx = self.inp
        T = sum(n for _, _, n in chunks)
        cu = np.concatenate([[0], np.cumsum([n for _, _, n in chunks])]).astype(np.int32)
        bt = np.array([self.blocks[s] + [0] * (self.maxb - len(self.blocks[s])) for s, _, _ in chunks],
                      np.int32)
        a.bci_set_batch(self.h, np.zeros(T, np.int32), cu,
                        np.array([p for _, p, _ in chunks], np.int32), bt, [], [])
        sl = [self.rows(s, p, n) for s, p, n in chunks]
        x = torch.cat([qkv[r] for r in sl]).contiguous()
        q = torch.empty(T, NQ * D, dtype=BF, device="cuda")
        a.bci_op_rope_kv_write(self.h, x, q, 0)
        a.bci_op_index_key_write(self.h, torch.cat([kidx[r] for r in sl]).contiguous(), DI, self.ic,
                                 self.isc, self.nb)
        if not attend:
            return None
        qi = torch.cat([qidx[r] for r in sl]).contiguous()
        wi = torch.cat([w[r] for r in sl]).contiguous()
        scores = torch.full((T, self.stride), float("nan"), device="cuda")
        a.bci_op_index_scores(self.h, qi, wi, HI, DI, self.ic, self.isc, self.nb, scores, self.stride,
                              schedule)
        sel = torch.empty(T, topk, dtype=torch.int32, device="cuda")
        a.bci_op_sparse_topk(self.h, scores, self.stride, topk, sel)
        o = torch.empty(T, NQ * D, dtype=BF, device="cuda")
        a.bci_op_sparse_attention(self.h, q, 0, sel, topk, o)
        torch.cuda.synchronize()
        return scores, sel, o

    def dense(self, chunks):
        """The dense operator on the same cache (K/V already written)."""
        a = abi()
        qkv = self.inp[0]
        T = sum(n for _, _, n in chunks)
        cu = np.concatenate([[0], np.cumsum([n for _, _, n in chunks])]).astype(np.int32)
        bt = np.array([self.blocks[s] + [0] * (self.maxb - len(self.blocks[s])) for s, _, _ in chunks],
                      np.int32)
        a.bci_set_batch(self.h, np.zeros(T, np.int32), cu,
                        np.array([p for _, p, _ in chunks], np.int32), bt, [], [])
        x = torch.cat([qkv[self.rows(s, p, n)] for s, p, n in chunks]).contiguous()
        q = torch.empty(T, NQ * D, dtype=BF, device="cuda")
        a.bci_op_rope_kv_write(self.h, x, q, 0)     # rewrites the same K/V codes
        o = torch.empty(T, NQ * D, dtype=BF, device="cuda")
        a.bci_op_attention(self.h, q, 0, o)
        torch.cuda.synchronize()
        return o

    def fill(self, seq, upto, chunk=4096):
        for s in range(0, upto, chunk):
            self.call([(seq, s, min(chunk, upto - s))], 64, attend=False)

    def close(self):
        torch.cuda.synchronize()
        abi().bci_destroy(self.h)


def make_inputs(n_rows, n_query_rows=None, exact=True, seed_index=70):
    """qkv [n_rows, WIDTH] N(0,1); index inputs for n_query_rows rows (all rows by default)."""
    qkv = synth.normal_bf16((n_rows, WIDTH), index=seed_index).cuda()
    nq = n_rows if n_query_rows is None else n_query_rows
    qi, w, ki = synth.sparse_index_inputs(nq, n_rows, HI, DI, exact=exact, index=seed_index + 1)
    return qkv, qi.cuda(), torch.from_numpy(w).cuda(), ki.cuda()


# ---------------------------------------------------------------- oracle side

class OracleSeq:
    """The oracle's K/V and index keys of one sequence, from the seeded inputs."""

    def __init__(self, ctx, seq, upto):
        qkv, qidx, w, kidx = ctx.inp
        r = ctx.rows(seq, 0, upto)
        self.qkv = qkv[r]
        kv = f64(qkv[r][:, NQ * D:]).reshape(upto, 2 * NKV, D)
        self.k = ops.kv_roundtrip(ops.rope(kv[:, :NKV], np.arange(upto), THETA))
        self.v = ops.kv_roundtrip(kv[:, NKV:])
        self.ki = ops.kv_roundtrip(f64(kidx[r]))
        self.qidx, self.w = qidx[r], w[r]

    def token(self, p, topk):
        q = ops.rope(f64(self.qkv[p, : NQ * D]).reshape(1, NQ, D), [p], THETA)[0]
        return sparse.sparse_token(q, f64(self.qidx[p]), self.w[p].cpu().numpy().astype(np.float64),
                                   self.k, self.v, self.ki, p, topk)


def check_token(ctx, oseq, p, topk, scores_row, sel_row, o_row, exact=True):
    sc, sl, o = oseq.token(p, topk)
    got_sc = scores_row[: p + 1].cpu().numpy().astype(np.float64)
    got_sel = sel_row.cpu().numpy()
    if exact:
        np.testing.assert_array_equal(got_sc, sc.astype(np.float32).astype(np.float64))
        want = np.full(topk, -1, np.int64)
        want[: len(sl)] = sl
        np.testing.assert_array_equal(got_sel, want)
    got = f64(o_row).reshape(NQ, D)
    scale = np.max(np.abs(oseq.v))
    assert np.max(np.abs(got - o)) <= 1.5e-2 * scale, p
    assert np.mean(np.abs(got - o)) <= 1.5e-3 * scale, p


# ---------------------------------------------------------------------- tests

LENGTHS = [300, 1100, 2600]


@pytest.fixture(scope="module")
def small():
    ctx = SparseCtx(LENGTHS, inputs=make_inputs(2 * 131 + 2600 + 64))
    # whole prefill of the three sequences in one call
    res = ctx.call([(i, 0, L) for i, L in enumerate(LENGTHS)], 512)
    yield ctx, res
    ctx.close()


def test_prefill_parity_scores_selection_and_output(small):
    ctx, (scores, sel, o) = small
    cu = np.concatenate([[0], np.cumsum(LENGTHS)])
    for i, L in enumerate(LENGTHS):
        oseq = OracleSeq(ctx, i, L)
        for p in sorted({0, 1, 63, 64, 511, 512, L // 2, L - 1} & set(range(L))):
            t = cu[i] + p
            check_token(ctx, oseq, p, 512, scores[t], sel[t], o[t])


def test_chunked_prefill_and_decode_bitwise(small):
    ctx, (scores, sel, o) = small
    L, seq = LENGTHS[2], 2
    t0 = sum(LENGTHS[:2])
    c2 = SparseCtx([L], inputs=ctx.inp)
    try:
        c2.inp = (ctx.inp[0][seq * 131:], ctx.inp[1][seq * 131:], ctx.inp[2][seq * 131:],
                  ctx.inp[3][seq * 131:])
        outs = []
        for s in range(0, L - 3, 700):                 # ragged chunks: 700, 700, 700, 497
            n = min(700, L - 3 - s)
            outs.append(c2.call([(0, s, n)], 512))
        for p in range(L - 3, L):                      # then decode, one token per call
            outs.append(c2.call([(0, p, 1)], 512))
        sc2 = torch.cat([x[0] for x in outs])
        sel2 = torch.cat([x[1] for x in outs])
        o2 = torch.cat([x[2] for x in outs])
        for t in range(L):
            assert same_bits(sc2[t, : t + 1], scores[t0 + t, : t + 1]), t
        assert same_bits(sel2, sel[t0:t0 + L])
        assert same_bits(o2, o[t0:t0 + L])
    finally:
        c2.close()


def test_decode_batch_composition_and_schedules(small):
    ctx, (scores, sel, o) = small
    cu = np.concatenate([[0], np.cumsum(LENGTHS)])
    last = [(i, L - 1, 1) for i, L in enumerate(LENGTHS)]
    # B = 1, B = 3 in two orders, under both score schedules
    ref = {i: (scores[cu[i] + L - 1], sel[cu[i] + L - 1], o[cu[i] + L - 1]) for i, L in enumerate(LENGTHS)}
    for order in ([2], [0, 1, 2], [2, 0, 1]):
        for sched in (1, 2):
            sc, sl, oo = ctx.call([last[i] for i in order], 512, schedule=sched)
            for j, i in enumerate(order):
                p = LENGTHS[i] - 1
                assert same_bits(sc[j, : p + 1], ref[i][0][: p + 1]), (order, sched, i)
                assert same_bits(sl[j], ref[i][1]), (order, sched, i)
                assert same_bits(oo[j], ref[i][2]), (order, sched, i)


def test_every_key_selected_equals_dense_operator(small):
    """Tokens with pos + 1 <= K select every key; the sparse output then has the dense
    kernel's bits (256-key segments) -- the same operator in a different layout."""
    ctx, (scores, sel, o) = small
    chunks = [(0, 0, 300), (1, 0, 512)]
    od = ctx.dense(chunks)
    assert same_bits(od[:300], o[:300])
    assert same_bits(od[300:812], o[300:812])


def test_small_topk_and_padding_edges():
    ctx = SparseCtx([200], inputs=make_inputs(200, seed_index=80))
    try:
        sc, sl, oo = ctx.call([(0, 0, 200)], 64)
        oseq = OracleSeq(ctx, 0, 200)
        for p in (0, 5, 63, 64, 65, 199):
            check_token(ctx, oseq, p, 64, sc[p], sl[p], oo[p])
        s = sl.cpu().numpy()
        assert s[0, 0] == 0 and np.all(s[0, 1:] == -1)           # first token: one key
        assert np.all(s[63] == np.arange(64))                     # exactly K candidates
        assert np.all(np.diff(s[199]) > 0)                        # ascending positions
    finally:
        ctx.close()


def test_random_index_inputs_within_tolerance():
    """Continuous index inputs: scores within an fp32 accumulation bound of the fp64
    oracle; the selected sets agree except for keys whose oracle score lies within
    that bound of the K-th best."""
    L, K = 1500, 256
    ctx = SparseCtx([L], inputs=make_inputs(L, exact=False, seed_index=90))
    try:
        sc, sl, oo = ctx.call([(0, 0, L)], K)
        oseq = OracleSeq(ctx, 0, L)
        for p in (300, 900, L - 1):
            osc, osl, oo_ref = oseq.token(p, K)
            qi = f64(oseq.qidx[p])
            wv = oseq.w[p].cpu().numpy().astype(np.float64)
            bound = 1e-5 * (np.abs(oseq.ki[: p + 1]) @ np.abs(qi).T) @ np.abs(wv) + 1e-30
            got = sc[p, : p + 1].cpu().numpy().astype(np.float64)
            assert np.all(np.abs(got - osc) <= bound), p
            gsel = sl[p].cpu().numpy()
            kth = np.sort(osc)[::-1][K - 1]
            diff = np.setxor1d(gsel, osl)
            assert np.all(np.abs(osc[diff] - kth) <= 2 * bound[diff]), (p, diff)
            if diff.size == 0:
                got_o = f64(oo[p]).reshape(NQ, D)
                assert np.max(np.abs(got_o - oo_ref)) <= 1.5e-2 * np.max(np.abs(oseq.v))
    finally:
        ctx.close()


def test_argument_errors():
    a = abi()
    ctx = SparseCtx([128], inputs=make_inputs(128, seed_index=95))
    try:
        ctx.call([(0, 0, 128)], 64)
        q = torch.zeros(128, NQ * D, dtype=BF, device="cuda")
        o = torch.empty_like(q)
        sel = torch.zeros(128, 100, dtype=torch.int32, device="cuda")
        with pytest.raises(a.BciError):
            a.bci_op_sparse_attention(ctx.h, q, 0, sel, 100, o)          # not a multiple of 64
        sc = torch.zeros(128, 64, device="cuda")
        with pytest.raises(a.BciError):
            a.bci_op_sparse_topk(ctx.h, sc, 64, 64, sel)                # stride < pos + 1
        with pytest.raises(a.BciError):
            a.bci_op_index_scores(ctx.h, q, sc, 48, DI, ctx.ic, ctx.isc, ctx.nb, sc, 128)  # 48 heads
        with pytest.raises(a.BciError):
            a.bci_op_index_key_write(ctx.h, q, DI, ctx.ic, ctx.isc, ctx.nb - 1)  # index cache too small
    finally:
        ctx.close()
    # a bf16 KV cache: the sparse operator is for the FP8 path
    h = make_ctx(hidden=512, nq=NQ, nkv=NKV, d=D, inter=512, vocab=4096, kv="bf16", max_position=256)
    try:
        k = torch.zeros(1, 4, NKV, 64, D, dtype=BF, device="cuda")
        a.bci_bind_kv_cache(h, k, k.clone(), None, None, 4)
        a.bci_set_batch(h, np.zeros(1, np.int32), [0, 1], [0], np.zeros((1, 4), np.int32), [], [])
        q = torch.zeros(1, NQ * D, dtype=BF, device="cuda")
        with pytest.raises(a.BciError):
            a.bci_op_sparse_attention(h, q, 0, torch.zeros(1, 64, dtype=torch.int32, device="cuda"), 64,
                                      torch.empty_like(q))
    finally:
        torch.cuda.synchronize()
        a.bci_destroy(h)


# ---------------------------------------------- full size, sampled against the oracle

def test_full_size_decode_batch_sampled():
    """Decode at B = 64 over contexts of 8K..57K (K = 2048): two sampled sequences
    against the oracle; sequence 0's bits equal between B = 1 and B = 64."""
    C = 57344
    rng = np.random.default_rng(7)
    lengths = [C, 8192] + [int(x) for x in rng.integers(8192, C + 1, size=62)]
    n_rows = 63 * 131 + C + 64
    qkv = synth.normal_bf16((n_rows, WIDTH), index=100).cuda()
    _, _, ki = synth.sparse_index_inputs(0, n_rows, HI, DI, exact=True, index=101)
    # index queries only for the decode rows (one per sequence)
    qrows = [s * 131 + L - 1 for s, L in enumerate(lengths)]
    qi_s, w_s, _ = synth.sparse_index_inputs(len(qrows), 0, HI, DI, exact=True, index=102)
    qi_full = torch.zeros(n_rows, HI, DI, dtype=BF)
    w_full = torch.zeros(n_rows, HI)
    qi_full[qrows] = qi_s
    w_full[qrows] = torch.from_numpy(w_s)
    ctx = SparseCtx(lengths, max_tokens=8192, inputs=(qkv, qi_full.cuda(), w_full.cuda(), ki.cuda()))
    try:
        for s, L in enumerate(lengths):
            ctx.fill(s, L - 1, chunk=8192)
        sc1, sl1, o1 = ctx.call([(0, C - 1, 1)], 2048)
        order = list(range(63, -1, -1))
        sc64, sl64, o64 = ctx.call([(s, lengths[s] - 1, 1) for s in order], 2048)
        j0 = order.index(0)
        assert same_bits(sc64[j0], sc1[0]) and same_bits(sl64[j0], sl1[0]) and same_bits(o64[j0], o1[0])
        for s in (0, 1):
            j = order.index(s)
            oseq = OracleSeq(ctx, s, lengths[s])
            check_token(ctx, oseq, lengths[s] - 1, 2048, sc64[j], sl64[j], o64[j])
    finally:
        ctx.close()


# ------------------------------------------------ Top-K alone, on chosen score rows

def _topk_rows():
    """Score rows that exercise each path of the selection: equal keys, a crowded
    first-digit bin (> 4096 keys), ties across the cut, signed zeros and negatives,
    n just above K, spread values, and a row past 65536 positions."""
    rng = np.random.default_rng(11)
    rows = []
    rows.append(np.full(9000, 1.5, np.float32))                                   # all equal
    r = np.full(12000, 1.0, np.float32)                                            # crowded bin
    r[rng.choice(12000, 300, replace=False)] = 2.0
    rows.append(r)
    rows.append((rng.integers(0, 40, 5000) * 0.25).astype(np.float32))             # coarse ties
    r = rng.standard_normal(7000).astype(np.float32)
    r[rng.choice(7000, 500, replace=False)] = 0.0
    r[rng.choice(7000, 500, replace=False)] = -0.0
    rows.append(r)                                                                 # signs, zeros
    rows.append(-np.abs(rng.standard_normal(2049)).astype(np.float32))             # n = K + 1
    rows.append((rng.standard_normal(60000) * 1e3).astype(np.float32))             # spread
    r = np.full(30000, 3.0, np.float32)                                            # ties at the cut
    r[:1000] = 5.0
    rows.append(r)
    rows.append(rng.standard_normal(70001).astype(np.float32))                     # > 65536
    return rows


def test_topk_rows_match_oracle():
    a = abi()
    rows = _topk_rows()
    K = 2048
    n_max = max(len(r) for r in rows)
    ctx = SparseCtx([n_max] * len(rows), max_tokens=64, inputs=None)
    try:
        stride = ctx.stride
        sc = np.zeros((len(rows), stride), np.float32)
        for i, r in enumerate(rows):
            sc[i, : len(r)] = r
        chunks = [(i, len(r) - 1, 1) for i, r in enumerate(rows)]
        bt = np.array([ctx.blocks[s] + [0] * (ctx.maxb - len(ctx.blocks[s])) for s, _, _ in chunks],
                      np.int32)
        a.bci_set_batch(ctx.h, np.zeros(len(rows), np.int32), np.arange(len(rows) + 1, dtype=np.int32),
                        np.array([p for _, p, _ in chunks], np.int32), bt, [], [])
        g_sc = torch.from_numpy(sc).cuda()
        sel = torch.empty(len(rows), K, dtype=torch.int32, device="cuda")
        a.bci_op_sparse_topk(ctx.h, g_sc, stride, K, sel)
        torch.cuda.synchronize()
        got = sel.cpu().numpy()
        for i, r in enumerate(rows):
            want = sparse.topk_select(r.astype(np.float64), K)
            np.testing.assert_array_equal(got[i], want, err_msg=f"row {i} (n = {len(r)})")
    finally:
        ctx.close()
