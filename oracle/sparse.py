"""Sparse attention over a Top-K selected key set, in fp64 on the CPU.

Test infrastructure only.  Nothing on the product path imports this.

The DeepSeek-V4-Flash recipe makes three demands of its sparse attention
(page "Finish RL Training Faster" digest, section "让训练前向使用推理的数值"
and its figure caption; news page "A vLLM bitre azonosította...", section
"A tréning közvetlenül a vLLM inferenciás kerneljeit használja"):
  * the Top-K that picks the attended keys breaks ties by a fixed rule;
  * the selected set is laid out in a fixed position order, so the same set
    is always summed in the same order;
  * the FP8 KV cache is gathered and dequantised to BF16 in every phase
    (prefill, decode, the trainer's private cache copy) before the one
    sparse attention operator.

Readings where the pages are silent (each listed with the others of the
build):
  * Index score.  The pages name no scoring function.  The reading is the
    indexer of DeepSeek's sparse attention: per query token t, index heads h
    with an index query q_I[t, h] and a weight w[t, h], and one index key
    k_I[s] per key position s:
        score(t, s) = sum_h w[t, h] * relu(q_I[t, h] . k_I[s]),   s <= pos(t).
    The index keys are kept in the FP8 cache format of K and V (e4m3 codes,
    one fp32 scale per token) and read back through the same dequantiser.
  * Tie rule.  Keys rank by (score descending, position ascending): among
    equal scores the earlier position wins.  A query with pos(t) + 1 <= K
    candidates selects all of them.
  * Position order.  The selected positions are listed ascending.
  * Attention.  Ordinary softmax attention of the query over the selected
    keys (same scale 1/sqrt(d) and GQA head mapping as the dense operator);
    the result does not depend on the order of the list, which only fixes
    the summation order of the product path.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_round

bf = bf16_round


def index_scores(q_idx, w, k_idx, pos: int):
    """Index scores of one query token against keys 0..pos.

    q_idx: [HI, dI] index query heads, w: [HI] head weights, k_idx: [>= pos+1, dI]
    index keys (already dequantised), all float64.  Returns float64 [pos + 1]:
    score[s] = sum_h w[h] * max(q_idx[h] . k_idx[s], 0).
    """
    q_idx = np.asarray(q_idx, dtype=np.float64)
    k = np.asarray(k_idx, dtype=np.float64)[: pos + 1]
    dots = k @ q_idx.T                       # [pos + 1, HI]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float64)


def topk_select(scores, k: int):
    """Positions of the k best keys under (score descending, position ascending),
    returned in ascending position order.  All positions when len(scores) <= k.
    Returns int64 [min(k, n)]."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -s))   # last key primary: -score, then position
    return np.sort(order[:k]).astype(np.int64)


def sparse_attention(q, k, v, sel):
    """Attention of one query token over the keys at positions ``sel``.

    q: [nq, d]; k, v: [n, nkv, d] (dequantised, bf16 grid); sel: positions.
    Query head h reads kv head floor(h * nkv / nq).  Weights softmax(q . k_j /
    sqrt(d)) over j in sel; o = bf(sum_j p_j v_j).  Returns [nq, d] on the bf16 grid.
    """
    q = np.asarray(q, dtype=np.float64)
    sel = np.asarray(sel, dtype=np.int64)
    ks = np.asarray(k, dtype=np.float64)[sel]        # [n_sel, nkv, d]
    vs = np.asarray(v, dtype=np.float64)[sel]
    nq, d = q.shape
    nkv = ks.shape[1]
    grp = nq // nkv
    out = np.empty((nq, d), dtype=np.float64)
    for h in range(nq):
        g = h // grp
        z = ks[:, g, :] @ q[h] / np.sqrt(d)
        p = np.exp(z - z.max())
        p /= p.sum()
        out[h] = p @ vs[:, g, :]
    return bf(out)


def sparse_token(q, q_idx, w, k, v, k_idx, pos: int, topk: int):
    """The whole path for one query token at position ``pos``: index scores over
    keys 0..pos, Top-K selection, attention over the selected keys.
    k, v: [>= pos+1, nkv, d] and k_idx [>= pos+1, dI] dequantised.
    Returns (scores float64 [pos+1], sel int64 ascending, o [nq, d])."""
    sc = index_scores(q_idx, w, k_idx, pos)
    sel = topk_select(sc, topk)
    return sc, sel, sparse_attention(q, k, v, sel)
