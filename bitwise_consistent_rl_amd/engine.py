"""Host-side drivers of the logprob-recompute path on one GPU.

Three ways to obtain the logprob of every valid response token, all through
libbci's HIP kernels (torch provides device memory and the stream only):

* ``recompute``     -- the training-side recompute: sequences packed into
                       varlen calls of whole-sequence prefill.  ``op_by_op``
                       drives the forward one bci_op_* call at a time, the way
                       a trainer's forward calls the inference kernels (page
                       "Finish RL Training Faster" digest, section
                       "让训练前向使用推理的数值"); otherwise one
                       bci_forward_logprobs per call.
* ``rollout``       -- the inference side: continuous batching that mixes
                       (chunked) prompt prefill and token-by-token decode of
                       the given response tokens under a batch cap; the
                       logprob of each response token is taken when it is
                       "sampled".
* ``acceptance``    -- the comparison of two logprob sets: byte equality plus
                       max/mean/std of the difference and the k3 KL estimate
                       (same page, section "零差异需要一个精确的比较对象").

Each logprob row depends only on its own sequence, so every split, packing
and cap gives the same bits; the tests check exactly that.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import _abi as abi

KV_BLOCK = 64


def weight_order(n_layers: int) -> List[str]:
    names = ["embed"]
    for l in range(n_layers):
        p = f"layers.{l}."
        names += [p + "attn_norm", p + "wqkv", p + "wo", p + "mlp_norm", p + "wgu", p + "wd"]
    names.append("final_norm")
    return names


@dataclasses.dataclass
class KVCache:
    k: torch.Tensor
    v: torch.Tensor
    k_scale: Optional[torch.Tensor]
    v_scale: Optional[torch.Tensor]
    n_blocks: int


class BlockAllocator:
    def __init__(self, n_blocks: int):
        self.free = list(range(n_blocks - 1, -1, -1))

    def alloc(self, n: int) -> List[int]:
        if n > len(self.free):
            raise RuntimeError(f"KV cache exhausted: need {n} blocks, {len(self.free)} free")
        return [self.free.pop() for _ in range(n)]

    def release(self, blocks: Sequence[int]) -> None:
        self.free.extend(reversed(list(blocks)))


class Model:
    """Device weights + one libbci context (fixed numeric contract)."""

    def __init__(self, cfg, weights: Dict[str, torch.Tensor], *, kv_dtype: str = "bf16",
                 max_tokens: int = 16384, max_seqs: int = 256, max_scored: int = 16384,
                 max_position: int = 4096, seg_keys: int = 2048, device: int = 0,
                 weight_version: int = 1, mode: str = "invariant"):
        self.cfg = cfg
        self.device = torch.device("cuda", device)
        self.kv_dtype = kv_dtype
        self.max_tokens, self.max_seqs, self.max_scored = max_tokens, max_seqs, max_scored
        self.max_position = max_position
        self.w = {k: v.to(self.device).contiguous() for k, v in weights.items()}
        mc = abi.ModelConfig()
        mc.n_layers, mc.hidden, mc.n_q_heads, mc.n_kv_heads = (cfg.n_layers, cfg.hidden,
                                                               cfg.n_q_heads, cfg.n_kv_heads)
        mc.head_dim, mc.intermediate, mc.vocab = cfg.head_dim, cfg.intermediate, cfg.vocab
        mc.rms_eps, mc.rope_theta = cfg.rms_eps, cfg.rope_theta
        mc.kv_dtype = abi.BCI_KV_FP8_E4M3 if kv_dtype == "fp8" else abi.BCI_KV_BF16
        mc.kv_block_tokens = KV_BLOCK
        mc.attn_segment_keys = seg_keys
        mc.max_tokens_per_call, mc.max_seqs_per_call = max_tokens, max_seqs
        mc.max_scored_per_call, mc.max_position = max_scored, max_position
        mc.mode = abi.BCI_MODE_FAST if mode == "fast" else abi.BCI_MODE_INVARIANT
        self.mode = mode
        self.ctx = abi.bci_create(mc, device)
        abi.bci_bind_weights(self.ctx, [self.w[n] for n in weight_order(cfg.n_layers)],
                             weight_version)
        self.bound_cache: Optional[KVCache] = None

    # ------------------------------------------------------------- weights
    def update_weights(self, weights: Dict[str, torch.Tensor], version: int) -> None:
        """In-place update (e.g. after an optimiser step): new values are copied into
        the bound buffers, whose addresses do not change, so captured graphs stay valid
        and their next replay reads the new weights."""
        for k, v in weights.items():
            self.w[k].copy_(v.to(self.device))
        abi.bci_bind_weights(self.ctx, [self.w[n] for n in weight_order(self.cfg.n_layers)],
                             version)

    def reload_weights(self, weights: Dict[str, torch.Tensor], version: int) -> None:
        """Reload into fresh buffers: the binding moves, so captured graphs are dropped
        and the next graphed call captures again."""
        self.w = {k: v.to(self.device).contiguous().clone() for k, v in weights.items()}
        abi.bci_bind_weights(self.ctx, [self.w[n] for n in weight_order(self.cfg.n_layers)],
                             version)

    def close(self):
        if self.ctx:
            torch.cuda.synchronize(self.device)
            abi.bci_destroy(self.ctx)
            self.ctx = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---------------------------------------------------------------- cache
    def new_cache(self, n_blocks: int) -> KVCache:
        c = self.cfg
        shape = (c.n_layers, n_blocks, c.n_kv_heads, KV_BLOCK, c.head_dim)
        if self.kv_dtype == "fp8":
            k = torch.empty(shape, dtype=torch.uint8, device=self.device)
            v = torch.empty(shape, dtype=torch.uint8, device=self.device)
            ks = torch.empty(shape[:-1], dtype=torch.float32, device=self.device)
            vs = torch.empty(shape[:-1], dtype=torch.float32, device=self.device)
        else:
            k = torch.empty(shape, dtype=torch.bfloat16, device=self.device)
            v = torch.empty(shape, dtype=torch.bfloat16, device=self.device)
            ks = vs = None
        return KVCache(k, v, ks, vs, n_blocks)

    def bind_cache(self, cache: KVCache):
        if self.bound_cache is not cache:
            abi.bci_bind_kv_cache(self.ctx, cache.k, cache.v, cache.k_scale, cache.v_scale,
                                  cache.n_blocks)
            self.bound_cache = cache


# ------------------------------------------------------------ one call

@dataclasses.dataclass
class CallPlan:
    tokens: np.ndarray
    cu_q: np.ndarray
    pos0: np.ndarray
    block_table: np.ndarray
    score_rows: np.ndarray
    score_ids: np.ndarray
    # (sequence index, first response index written) for each scored row, in order
    owners: List[tuple]


def run_call(model: Model, plan: CallPlan, op_by_op: bool = False, stream=None,
             graph: bool = False) -> torch.Tensor:
    """Run one varlen forward call; returns fp32 logprobs [n_scored] on the GPU.
    ``graph``: replay (or capture) the forward as a HIP graph for this batch shape."""
    ctx = model.ctx
    abi.bci_set_batch(ctx, plan.tokens, plan.cu_q, plan.pos0, plan.block_table, plan.score_rows,
                      plan.score_ids, stream)
    lp = torch.empty(len(plan.score_rows), dtype=torch.float32, device=model.device)
    if graph:
        abi.bci_forward_logprobs_graph(ctx, lp if len(plan.score_rows) else None, stream)
    elif not op_by_op:
        abi.bci_forward_logprobs(ctx, lp if len(plan.score_rows) else None, stream)
    else:
        _forward_op_by_op(model, plan, lp, stream)
    return lp


def _forward_op_by_op(model: Model, plan: CallPlan, lp: torch.Tensor, stream=None):
    """The forward as a trainer would write it: one inference kernel per op."""
    c, w, ctx, dev = model.cfg, model.w, model.ctx, model.device
    T, H, d = len(plan.tokens), c.hidden, c.head_dim
    bf = dict(dtype=torch.bfloat16, device=dev)
    r = torch.empty(T, H, **bf)
    h = torch.empty(T, H, **bf)
    qkv = torch.empty(T, c.qkv_rows, **bf)
    q = torch.empty(T, c.n_q_heads * d, **bf)
    o = torch.empty(T, c.n_q_heads * d, **bf)
    x = torch.empty(T, H, **bf)
    act = torch.empty(T, c.intermediate, **bf)
    abi.bci_op_embed(ctx, w["embed"], r, stream)
    for l in range(c.n_layers):
        p = f"layers.{l}."
        abi.bci_op_add_rmsnorm(ctx, x if l else None, r, h, w[p + "attn_norm"], T, H, c.rms_eps, stream)
        abi.bci_op_gemm_bf16(ctx, h, w[p + "wqkv"], qkv, T, c.qkv_rows, H, abi.BCI_EPI_BF16, stream)
        abi.bci_op_rope_kv_write(ctx, qkv, q, l, stream)
        abi.bci_op_attention(ctx, q, l, o, stream)
        abi.bci_op_gemm_bf16(ctx, o, w[p + "wo"], x, T, H, c.n_q_heads * d, abi.BCI_EPI_BF16, stream)
        abi.bci_op_add_rmsnorm(ctx, x, r, h, w[p + "mlp_norm"], T, H, c.rms_eps, stream)
        abi.bci_op_gemm_bf16(ctx, h, w[p + "wgu"], act, T, 2 * c.intermediate, H,
                             abi.BCI_EPI_SILU_MUL, stream)
        abi.bci_op_gemm_bf16(ctx, act, w[p + "wd"], x, T, H, c.intermediate, abi.BCI_EPI_BF16, stream)
    abi.bci_op_add_rmsnorm(ctx, x, r, h, w["final_norm"], T, H, c.rms_eps, stream)
    R = len(plan.score_rows)
    if R:
        hf = torch.empty(R, H, **bf)
        abi.bci_op_gather_scored(ctx, h, H, hf, stream)
        ids = torch.from_numpy(plan.score_ids.astype(np.int32)).to(dev)
        abi.bci_op_lmhead_logprob(ctx, hf, w["embed"], ids, R, H, c.vocab, lp, stream)


# ------------------------------------------------------------ recompute

def plan_recompute(seqs, order: Sequence[int], max_tokens: int, max_seqs: int, max_scored: int,
                   n_blocks: int) -> List[tuple]:
    """Greedy packing of whole sequences (positions 0 .. L-2) into calls, in ``order``.
    Returns [(CallPlan, [seq indices])]."""
    calls, cur = [], []
    tok = sc = blk = 0

    def flush():
        nonlocal cur, tok, sc, blk
        if cur:
            calls.append(_prefill_plan(seqs, cur))
        cur, tok, sc, blk = [], 0, 0, 0

    for i in order:
        s = seqs[i]
        T = s.length - 1
        nb = (T + KV_BLOCK - 1) // KV_BLOCK
        if T > max_tokens or s.n_scored > max_scored or nb > n_blocks:
            raise ValueError(f"sequence {i} (length {s.length}) does not fit one call")
        if cur and (tok + T > max_tokens or len(cur) + 1 > max_seqs or sc + s.n_scored > max_scored
                    or blk + nb > n_blocks):
            flush()
        cur.append(i)
        tok += T
        sc += s.n_scored
        blk += nb
    flush()
    return calls


def _prefill_plan(seqs, idx: List[int]) -> tuple:
    toks, cu, btab, srow, sid, owners = [], [0], [], [], [], []
    nxt = 0
    maxb = max((seqs[i].length - 1 + KV_BLOCK - 1) // KV_BLOCK for i in idx)
    for i in idx:
        s = seqs[i]
        T = s.length - 1
        base = cu[-1]
        toks.append(s.tokens[:T])
        cu.append(base + T)
        nb = (T + KV_BLOCK - 1) // KV_BLOCK
        btab.append(list(range(nxt, nxt + nb)) + [0] * (maxb - nb))
        nxt += nb
        for t in range(s.prompt_len - 1, T):
            srow.append(base + t)
            sid.append(int(s.tokens[t + 1]))
        owners.append((i, 0))
    plan = CallPlan(np.concatenate(toks).astype(np.int32), np.array(cu, np.int32),
                    np.zeros(len(idx), np.int32), np.array(btab, np.int32),
                    np.array(srow, np.int32), np.array(sid, np.int32), owners)
    return plan, idx


def recompute(model: Model, seqs, cache: KVCache, order: Optional[Sequence[int]] = None,
              op_by_op: bool = False, stream=None) -> List[np.ndarray]:
    """Training-side recompute of every valid response token's logprob."""
    model.bind_cache(cache)
    order = list(range(len(seqs))) if order is None else list(order)
    out: List[Optional[np.ndarray]] = [None] * len(seqs)
    calls = plan_recompute(seqs, order, model.max_tokens, model.max_seqs, model.max_scored,
                           cache.n_blocks)
    pending = []
    for plan, idx in calls:
        lp = run_call(model, plan, op_by_op, stream)
        pending.append((lp, idx))
    for lp, idx in pending:
        h = lp.cpu().numpy()
        o = 0
        for i in idx:
            n = seqs[i].n_scored
            out[i] = h[o:o + n].copy()
            o += n
    return out


# ------------------------------------------------------------ rollout

def rollout(model: Model, seqs, cache: KVCache, cap: int, prefill_chunk: Optional[int] = None,
            order: Optional[Sequence[int]] = None, cap_schedule=None, stream=None,
            graph: bool = False) -> List[np.ndarray]:
    """Continuous batching: each step runs, for every active sequence, either its next
    prompt chunk or one decode token (the given response token), in one varlen call.
    ``cap_schedule`` (callable step -> cap) varies the batch cap per step.  ``graph``:
    steps that are pure decode (one token per sequence) replay captured HIP graphs, with
    the block table padded to the context's full width so its shape stays fixed."""
    model.bind_cache(cache)
    alloc = BlockAllocator(cache.n_blocks)
    order = list(range(len(seqs))) if order is None else list(order)
    queue = list(order)
    state = {}  # seq -> [next position, blocks]
    out = {i: [] for i in order}
    active: List[int] = []
    step = 0
    while queue or active:
        c = cap_schedule(step) if cap_schedule else cap
        while queue and len(active) < c:
            i = queue.pop(0)
            state[i] = [0, []]
            active.append(i)
        toks, cu, pos0, srow, sid, owners, rows = [], [0], [], [], [], [], []
        budget = model.max_tokens
        sel = []
        for i in active[:c]:
            s = seqs[i]
            p, blocks = state[i]
            T = s.length - 1
            if p < s.prompt_len:
                n = s.prompt_len - p if prefill_chunk is None else min(prefill_chunk, s.prompt_len - p)
            else:
                n = 1
            n = min(n, T - p, budget - cu[-1])
            if n <= 0:
                continue
            need = (p + n + KV_BLOCK - 1) // KV_BLOCK
            if need > len(blocks):
                blocks.extend(alloc.alloc(need - len(blocks)))
            base = cu[-1]
            toks.append(s.tokens[p:p + n])
            cu.append(base + n)
            pos0.append(p)
            rows.append(list(blocks))
            for t in range(p, p + n):
                if s.prompt_len - 1 <= t <= T - 1:
                    srow.append(base + t - p)
                    sid.append(int(s.tokens[t + 1]))
                    owners.append(i)
            sel.append((i, n))
        decode_only = all(n == 1 for _, n in sel) and all(
            state[i][0] >= seqs[i].prompt_len for i, _ in sel)
        use_graph = graph and decode_only
        maxb = (-(-model.max_position // KV_BLOCK) if use_graph
                else max(len(r) for r in rows))
        btab = np.array([r + [0] * (maxb - len(r)) for r in rows], np.int32)
        plan = CallPlan(np.concatenate(toks).astype(np.int32), np.array(cu, np.int32),
                        np.array(pos0, np.int32), btab, np.array(srow, np.int32),
                        np.array(sid, np.int32), [])
        lp = run_call(model, plan, False, stream, graph=use_graph).cpu().numpy()
        for j, i in enumerate(owners):
            out[i].append(lp[j])
        for i, n in sel:
            state[i][0] += n
            if state[i][0] >= seqs[i].length - 1:
                alloc.release(state[i][1])
                active.remove(i)
        step += 1
    return [np.array(out[i], dtype=np.float32) for i in range(len(seqs))]


# ------------------------------------------------------------ acceptance

def acceptance(lp_recompute: Sequence[np.ndarray], lp_rollout: Sequence[np.ndarray],
               version_recompute: int = 0, version_rollout: int = 0) -> dict:
    """Per valid response token: delta = recompute - rollout (fp64).  Returns byte
    equality, max|delta|, mean|delta|, std(delta) and k3 = mean(expm1(delta) - delta).
    Refuses to compare logprobs taken under different weight versions."""
    if version_recompute != version_rollout:
        raise ValueError("logprobs come from different weight versions; not comparable")
    a = np.concatenate([np.asarray(x, np.float32) for x in lp_recompute]) if lp_recompute else np.zeros(0, np.float32)
    b = np.concatenate([np.asarray(x, np.float32) for x in lp_rollout]) if lp_rollout else np.zeros(0, np.float32)
    if a.shape != b.shape:
        raise ValueError(f"token counts differ: {a.shape} vs {b.shape}")
    d = a.astype(np.float64) - b.astype(np.float64)
    n = d.size
    return dict(
        tokens=int(n),
        bitwise_equal=bool(a.tobytes() == b.tobytes()),
        max=float(np.max(np.abs(d))) if n else 0.0,
        mean=float(np.mean(np.abs(d))) if n else 0.0,
        std=float(np.std(d)) if n else 0.0,
        k3=float(np.mean(np.expm1(d) - d)) if n else 0.0,
    )
