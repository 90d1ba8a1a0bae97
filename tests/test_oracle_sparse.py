"""Pins of the sparse-attention oracle (CPU only): Top-K against brute force over
all subsets, index scores against closed forms, attention over a selected set
against the dense attention oracle (itself pinned in test_oracle_ops) and against
closed forms.  A dropped relu, a wrong tie direction, a flipped weight sign or a
transposed head/key operand fails at least one of these."""
import itertools

import numpy as np
import pytest

import synth
from oracle import ops, sparse
from oracle.codecs import bf16_decode, bf16_round


def bfv(x):
    return bf16_round(np.asarray(x, dtype=np.float64))


# -------------------------------------------------------------------- Top-K

def _ranks_above(a, b, s):
    """a ranks above b: higher score, or equal score and earlier position."""
    return s[a] > s[b] or (s[a] == s[b] and a < b)


@pytest.mark.parametrize("seed", range(12))
def test_topk_equals_the_unique_dominating_subset(seed):
    """The selected set is the one subset S of size k whose every member ranks above
    every non-member; brute force over all subsets finds exactly one."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 10))
    k = int(rng.integers(1, n))
    s = rng.integers(-2, 3, size=n).astype(np.float64)   # few values: many ties
    valid = [S for S in itertools.combinations(range(n), k)
             if all(_ranks_above(a, b, s) for a in S for b in range(n) if b not in S)]
    assert len(valid) == 1
    np.testing.assert_array_equal(sparse.topk_select(s, k), np.array(valid[0]))


def test_topk_special_cases():
    n, k = 50, 8
    # all equal: the tie rule takes the earliest positions
    np.testing.assert_array_equal(sparse.topk_select(np.zeros(n), k), np.arange(k))
    # strictly increasing with position: the most recent k (a sliding window)
    np.testing.assert_array_equal(sparse.topk_select(np.arange(n, dtype=float), k),
                                  np.arange(n - k, n))
    # strictly decreasing: the first k
    np.testing.assert_array_equal(sparse.topk_select(-np.arange(n, dtype=float), k), np.arange(k))
    # no more candidates than k: all of them, in order
    np.testing.assert_array_equal(sparse.topk_select(np.array([3.0, 1.0, 2.0]), 8), [0, 1, 2])
    # output ascending even when the best keys come late
    s = np.zeros(n)
    s[[40, 3, 17]] = [5.0, 4.0, 9.0]
    np.testing.assert_array_equal(sparse.topk_select(s, 3), [3, 17, 40])
    # a tie straddling the cut: of the three 1.0s at 5, 9, 30 only the two earliest enter
    s = np.zeros(n)
    s[[2, 44]] = 2.0
    s[[5, 9, 30]] = 1.0
    np.testing.assert_array_equal(sparse.topk_select(s, 4), [2, 5, 9, 44])


# ------------------------------------------------------------- index scores

def test_index_scores_closed_forms():
    rng = np.random.default_rng(3)
    dI, n = 16, 40
    k = rng.integers(-5, 6, size=(n, dI)).astype(np.float64)
    j = 7
    e = np.zeros(dI)
    e[j] = 1.0
    pos = n - 1
    # one head, weight 1, query e_j: relu of column j
    np.testing.assert_array_equal(sparse.index_scores(e[None], [1.0], k, pos), np.maximum(k[:, j], 0))
    # heads e_j and -e_j with weights (1, 1): relu(x) + relu(-x) = |x|
    np.testing.assert_array_equal(sparse.index_scores(np.stack([e, -e]), [1.0, 1.0], k, pos),
                                  np.abs(k[:, j]))
    # weights (1, -1): relu(x) - relu(-x) = x
    np.testing.assert_array_equal(sparse.index_scores(np.stack([e, -e]), [1.0, -1.0], k, pos),
                                  k[:, j])
    # causal: only keys 0..pos
    assert sparse.index_scores(e[None], [1.0], k, 5).shape == (6,)
    # linear in the weights, head by head
    q = rng.integers(-2, 3, size=(3, dI)).astype(np.float64)
    w1, w2 = np.array([1.0, -2.0, 0.5]), np.array([0.25, 1.0, -1.0])
    np.testing.assert_array_equal(sparse.index_scores(q, w1 + w2, k, pos),
                                  sparse.index_scores(q, w1, k, pos) + sparse.index_scores(q, w2, k, pos))
    # a head whose dots are all negative contributes nothing
    neg = -np.ones((1, dI))                                # dots with positive keys < 0
    kpos = np.abs(k) + 1.0
    np.testing.assert_array_equal(sparse.index_scores(np.concatenate([neg, e[None]]), [100.0, 1.0],
                                                      kpos, pos), kpos[:, j])


def test_exact_index_inputs_roundtrip_the_fp8_cache_unchanged():
    """The integer index keys of synth (|x| <= 7 with a 7 in every row) have scale
    7/448 = 2^-6 and survive the FP8 cache round trip exactly, so scores computed
    from them are exact integers (times powers of two) in any summation order."""
    _, w, k = synth.sparse_index_inputs(2, 300)
    kk = bf16_decode(synth.bf16_bits(k))
    codes, sig = ops.kv_quantise(kk)
    assert np.all(sig == np.float32(2.0 ** -6))
    np.testing.assert_array_equal(ops.kv_dequantise(codes, sig), kk)


# ------------------------------------------------------- attention over a set

def _qkv(n, nq=8, nkv=2, d=32, seed=0):
    rng = np.random.default_rng(seed)
    return (bfv(rng.standard_normal((nq, d))), bfv(rng.standard_normal((n, nkv, d))),
            bfv(rng.standard_normal((n, nkv, d))))


def test_sparse_attention_over_all_keys_is_dense_causal_attention():
    q, k, v = _qkv(37)
    pos = 36
    got = sparse.sparse_attention(q, k, v, np.arange(pos + 1))
    ref = ops.causal_gqa_attention(q[None], k, v, [pos])[0]
    np.testing.assert_allclose(got, ref, rtol=0, atol=0)


def test_sparse_attention_window_is_dense_attention_on_the_window():
    q, k, v = _qkv(60, seed=1)
    sel = np.arange(45, 60)
    got = sparse.sparse_attention(q, k, v, sel)
    ref = ops.causal_gqa_attention(q[None], k[sel], v[sel], [59], k_pos=sel)[0]
    np.testing.assert_array_equal(got, ref)


def test_sparse_attention_single_key_and_order_and_head_mapping():
    q, k, v = _qkv(20, nq=8, nkv=2, seed=2)
    # one selected key: softmax weight 1, output is that value row (already bf16)
    o = sparse.sparse_attention(q, k, v, [11])
    np.testing.assert_array_equal(o[:4], np.broadcast_to(v[11, 0], (4, 32)))
    np.testing.assert_array_equal(o[4:], np.broadcast_to(v[11, 1], (4, 32)))
    # a set, not a sequence: the list order does not change the result
    sel = np.array([2, 7, 13, 19])
    np.testing.assert_array_equal(sparse.sparse_attention(q, k, v, sel),
                                  sparse.sparse_attention(q, k, v, sel[::-1]))
    # keys outside the set do not matter
    k2, v2 = k.copy(), v.copy()
    k2[[0, 1, 3]] = 100.0
    v2[[0, 1, 3]] = -100.0
    np.testing.assert_array_equal(sparse.sparse_attention(q, k2, v2, sel),
                                  sparse.sparse_attention(q, k, v, sel))


def test_sparse_token_reduces_to_dense_when_k_covers_the_context():
    q, k, v = _qkv(30, seed=4)
    rng = np.random.default_rng(5)
    qi = rng.integers(-2, 3, size=(4, 16)).astype(np.float64)
    ki = rng.integers(-7, 8, size=(30, 16)).astype(np.float64)
    sc, sel, o = sparse.sparse_token(q, qi, np.ones(4), k, v, ki, 29, topk=64)
    np.testing.assert_array_equal(sel, np.arange(30))
    np.testing.assert_array_equal(o, ops.causal_gqa_attention(q[None], k, v, [29])[0])
    # with a small K the selection is the K best, and the output attends only to them
    sc, sel, o = sparse.sparse_token(q, qi, np.ones(4), k, v, ki, 29, topk=6)
    assert len(sel) == 6 and np.all(np.diff(sel) > 0)
    worst_in = sc[sel].min()
    out = np.setdiff1d(np.arange(30), sel)
    assert np.all(sc[out] <= worst_in)
    assert np.all([(sc[b] < worst_in) or (b > sel[sc[sel] == worst_in].max()) for b in out])
