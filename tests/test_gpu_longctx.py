"""Long-context FP8-KV attention (32 q / 4 kv heads of 128, e4m3 cache with
per-token-per-head scales, contexts 8K / 32K / 57K, batch 1..64 of mixed lengths).

Prefill, chunked prefill (chunk 2048) and decode all read the cache through the same
gather + dequantise rule and run the same attention kernel; the output of a query is
bitwise identical across the three phases and across batch sizes, and matches the
oracle's attention over its own rotated, FP8-round-tripped keys and values of the
same seeded qkv rows."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import BF, f64, same_bits
from oracle import ops
from test_gpu_ops import abi, make_ctx

pytestmark = pytest.mark.gpu

NQ, NKV, D, SEG = 32, 4, 128, 1024
CONTEXTS = [8192, 32768, 57344]
WIDTH = (NQ + 2 * NKV) * D


class LongCtx:
    """One context holding up to 64 sequences; sequence i's K/V come from rows
    [i*131, i*131 + L_i) of one random qkv buffer."""

    def __init__(self, lengths, max_tokens=8192, split=0):
        a = abi()
        self.lengths = lengths
        self.h = make_ctx(hidden=512, nq=NQ, nkv=NKV, d=D, inter=512, vocab=4096, kv="fp8",
                          max_tokens=max_tokens, max_seqs=64, max_scored=64,
                          max_position=max(lengths) + 64, seg=SEG, split=split)
        self.blocks, nxt = [], 0
        for L in lengths:
            nb = (L + 63) // 64
            self.blocks.append(list(range(nxt, nxt + nb)))
            nxt += nb
        shape = (1, nxt, NKV, 64, D)
        self.k = torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda")
        self.v = torch.full(shape, 0x7F, dtype=torch.uint8, device="cuda")
        self.ks = torch.full(shape[:-1], float("nan"), device="cuda")
        self.vs = torch.full(shape[:-1], float("nan"), device="cuda")
        a.bci_bind_kv_cache(self.h, self.k, self.v, self.ks, self.vs, nxt)
        self.maxb = max(len(b) for b in self.blocks)

    def call(self, qkv_rows, chunks, attend=True):
        """chunks: list of (seq, start, n); qkv_rows: [sum n, WIDTH] bf16 on the GPU."""
        a = abi()
        T = qkv_rows.shape[0]
        cu = np.concatenate([[0], np.cumsum([n for _, _, n in chunks])]).astype(np.int32)
        bt = np.array([self.blocks[s] + [0] * (self.maxb - len(self.blocks[s])) for s, _, _ in chunks],
                      np.int32)
        a.bci_set_batch(self.h, np.zeros(T, np.int32), cu,
                        np.array([p for _, p, _ in chunks], np.int32), bt, [], [])
        q = torch.empty(T, NQ * D, dtype=BF, device="cuda")
        a.bci_op_rope_kv_write(self.h, qkv_rows, q, 0)
        if not attend:
            return None
        o = torch.empty(T, NQ * D, dtype=BF, device="cuda")
        a.bci_op_attention(self.h, q, 0, o)
        torch.cuda.synchronize()
        return q, o

    def gather(self, seq, n):
        a = abi()
        L = self.lengths[seq]
        a.bci_set_batch(self.h, np.zeros(1, np.int32), [0, 1], [L - 1],
                        np.array([self.blocks[seq] + [0] * (self.maxb - len(self.blocks[seq]))], np.int32),
                        [], [])
        ko = torch.empty(n, NKV, D, dtype=BF, device="cuda")
        vo = torch.empty(n, NKV, D, dtype=BF, device="cuda")
        a.bci_op_kv_gather_dequant(self.h, 0, n, 0, ko, vo)
        torch.cuda.synchronize()
        return ko, vo

    def close(self):
        torch.cuda.synchronize()
        abi().bci_destroy(self.h)


@pytest.fixture(scope="module")
def qkv():
    n = max(CONTEXTS) + 64 * 131
    return synth.normal_bf16((n, WIDTH), index=60).cuda()


def _fill(ctx, qkv, seq, upto, chunk=8192):
    """Write K/V of positions 0 .. upto-1 of a sequence (no attention)."""
    base = seq * 131
    for s in range(0, upto, chunk):
        n = min(chunk, upto - s)
        ctx.call(qkv[base + s: base + s + n].contiguous(), [(seq, s, n)], attend=False)


def _decode(ctx, qkv, seqs):
    """One decode step: the last token of each listed sequence, in one call."""
    rows = torch.cat([qkv[s * 131 + ctx.lengths[s] - 1: s * 131 + ctx.lengths[s]] for s in seqs])
    q, o = ctx.call(rows.contiguous(), [(s, ctx.lengths[s] - 1, 1) for s in seqs])
    return q, o


@pytest.mark.parametrize("C", CONTEXTS)
def test_decode_invariant_across_batch_and_matches_oracle(qkv, C):
    rng = np.random.default_rng(C)
    lengths = [C] + [int(x) for x in rng.integers(C // 2, C + 1, size=63)]
    ctx = LongCtx(lengths)
    try:
        for s in range(64):
            _fill(ctx, qkv, s, lengths[s] - 1)
        q1, o1 = _decode(ctx, qkv, [0])                      # B = 1
        _, o4 = _decode(ctx, qkv, [7, 0, 3, 9])               # B = 4, sequence 0 second
        _, o64 = _decode(ctx, qkv, list(range(63, -1, -1)))   # B = 64, sequence 0 last
        assert same_bits(o4[1:2], o1) and same_bits(o64[63:64], o1)
        # the same B = 64 step with the segments run in sequence inside each workgroup
        ctx_seq = LongCtx(lengths, split=1)
        try:
            for s in (0,):
                _fill(ctx_seq, qkv, s, lengths[s] - 1)
            _, o1s = _decode(ctx_seq, qkv, [0])
            assert same_bits(o1s, o1)
        finally:
            ctx_seq.close()
        # parity: the oracle rotates and FP8-round-trips the same qkv rows itself
        kv = f64(qkv[0:C, NQ * D:]).reshape(C, 2 * NKV, D)
        K = ops.kv_roundtrip(ops.rope(kv[:, :NKV], np.arange(C), 1e6))
        V = ops.kv_roundtrip(kv[:, NKV:])
        qo = ops.rope(f64(qkv[C - 1: C, : NQ * D]).reshape(1, NQ, D), [C - 1], 1e6)
        ref = ops.causal_gqa_attention(qo, K, V, [C - 1])
        got = f64(o1).reshape(1, NQ, D)
        scale = np.max(np.abs(V))
        assert np.max(np.abs(got - ref)) <= 1.5e-2 * scale
        assert np.mean(np.abs(got - ref)) <= 1.5e-3 * scale
    finally:
        ctx.close()


@pytest.mark.parametrize("C", [8192, 57344])
def test_prefill_chunked_and_decode_bitwise(qkv, C):
    """Whole prefill (8K only), chunked prefill with chunk 2048, and decode of the last
    positions give the same bits for the same queries."""
    ctx = LongCtx([C], max_tokens=8192)
    try:
        outs = []
        for s in range(0, C, 2048):
            _, o = ctx.call(qkv[s: s + 2048].contiguous(), [(0, s, 2048)])
            outs.append(o)
        o_chunk = torch.cat(outs)
        if C <= 8192:
            ctx2 = LongCtx([C], max_tokens=8192)
            try:
                _, o_full = ctx2.call(qkv[:C].contiguous(), [(0, 0, C)])
                assert same_bits(o_full, o_chunk)
            finally:
                ctx2.close()
        # decode positions C-3 .. C-1 one by one on a fresh cache holding 0 .. C-4
        ctx3 = LongCtx([C], max_tokens=8192)
        try:
            _fill(ctx3, qkv, 0, C - 3)
            for t in range(C - 3, C):
                _, o = ctx3.call(qkv[t: t + 1].contiguous(), [(0, t, 1)])
                assert same_bits(o, o_chunk[t: t + 1]), t
        finally:
            ctx3.close()
    finally:
        ctx.close()
