"""HIP-graph-captured decode: the captured forward against the eager one, in-place
weight update, reload and restore (page "Finish RL Training Faster" digest, section
"让训练前向使用推理的数值": stable workspace addresses and in-place weight copies so that
decode graphs stay valid; the first step after an update must see the new weights).

Every replay is checked against an eager forward of the same batch, with eager work
and synchronisations between replays."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def eng():
    from bitwise_consistent_rl_amd import engine
    return engine


def abi():
    from bitwise_consistent_rl_amd import _abi
    return _abi


def bits(x):
    return np.asarray(x.cpu().numpy() if torch.is_tensor(x) else x, np.float32).tobytes()


def _decode_plans(model, seqs, blocks, steps):
    """Plans for `steps` decode steps of all sequences from their prompt end on, with
    the block table padded to the context's full width (fixed graph shape)."""
    e = eng()
    width = -(-model.max_position // e.KV_BLOCK)
    plans = []
    for t in range(steps):
        pos = [s.prompt_len + t for s in seqs]
        toks = np.array([s.tokens[p] for s, p in zip(seqs, pos)], np.int32)
        ids = np.array([s.tokens[p + 1] for s, p in zip(seqs, pos)], np.int32)
        btab = np.array([b + [0] * (width - len(b)) for b in blocks], np.int32)
        plans.append(e.CallPlan(toks, np.arange(len(seqs) + 1, dtype=np.int32),
                                np.array(pos, np.int32), btab,
                                np.arange(len(seqs), dtype=np.int32), ids, []))
    return plans


def _prefill(model, seqs, blocks):
    e = eng()
    width = max(len(b) for b in blocks)
    plan = e.CallPlan(np.concatenate([s.tokens[:s.prompt_len] for s in seqs]).astype(np.int32),
                      np.concatenate([[0], np.cumsum([s.prompt_len for s in seqs])]).astype(np.int32),
                      np.zeros(len(seqs), np.int32),
                      np.array([b + [0] * (width - len(b)) for b in blocks], np.int32),
                      np.zeros(0, np.int32), np.zeros(0, np.int32), [])
    e.run_call(model, plan)


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.TINY
    weights = synth.make_weights(cfg, gain_noise=True)
    seqs = [s for s in synth.tiny_sequences(cfg, n=12, min_len=100, max_len=300)
            if s.length - s.prompt_len > 12][:5]
    model = eng().Model(cfg, weights, max_tokens=2048, max_seqs=16, max_scored=2048,
                        max_position=512, seg_keys=64)
    cache = model.new_cache(64)
    cache.k.fill_(float("nan"))
    cache.v.fill_(float("nan"))
    model.bind_cache(cache)
    blocks = [list(range(6 * i, 6 * i + 6)) for i in range(len(seqs))]
    yield cfg, weights, seqs, model, cache, blocks
    model.close()


def _eager_and_graph(model, plan):
    e = eng()
    lp_e = e.run_call(model, plan)
    torch.cuda.synchronize()
    lp_g = e.run_call(model, plan, graph=True)
    torch.cuda.synchronize()
    return lp_e, lp_g


def test_graph_replays_equal_eager(tiny):
    cfg, weights, seqs, model, cache, blocks = tiny
    abi().bci_graph_reset(model.ctx)
    _prefill(model, seqs, blocks)
    plans = _decode_plans(model, seqs, blocks, 10)
    for t, plan in enumerate(plans):
        # the eager run writes this step's K/V; the replay rewrites the same values
        lp_e, lp_g = _eager_and_graph(model, plan)
        assert bits(lp_e) == bits(lp_g), t
        # eager work of another shape between replays
        if t % 3 == 1:
            eng().run_call(model, plans[0])
            torch.cuda.synchronize()
    assert abi().bci_graph_count(model.ctx) == 1   # one shape, captured once


def test_graph_in_place_update_reload_restore(tiny):
    cfg, weights, seqs, model, cache, blocks = tiny
    e = eng()
    abi().bci_graph_reset(model.ctx)
    _prefill(model, seqs, blocks)
    plan = _decode_plans(model, seqs, blocks, 1)[0]
    base_e, base_g = _eager_and_graph(model, plan)
    assert bits(base_e) == bits(base_g)
    n_graphs = abi().bci_graph_count(model.ctx)
    # in-place update: other values, same buffers -> the next replay must see them
    other = synth.make_weights(cfg, gain_noise=True, seed=4321)
    model.update_weights(other, version=2)
    assert abi().bci_graph_count(model.ctx) == n_graphs      # no recapture needed
    new_g = e.run_call(model, plan, graph=True)
    torch.cuda.synchronize()
    new_e = e.run_call(model, plan)
    torch.cuda.synchronize()
    assert bits(new_g) == bits(new_e)
    assert bits(new_g) != bits(base_g)                       # the update was seen
    # restore the original values in place: bits return exactly
    model.update_weights(weights, version=1)
    back_g = e.run_call(model, plan, graph=True)
    torch.cuda.synchronize()
    assert bits(back_g) == bits(base_g)
    # reload into fresh buffers: graphs are dropped and captured again
    model.reload_weights(weights, version=1)
    re_g = e.run_call(model, plan, graph=True)
    torch.cuda.synchronize()
    assert bits(re_g) == bits(base_g)
    assert abi().bci_graph_count(model.ctx) == 1


def test_graphed_rollout_equals_recompute(tiny):
    cfg, weights, seqs, model, cache, blocks = tiny
    e = eng()
    train_cache = model.new_cache(64)
    rec = e.recompute(model, seqs, train_cache)
    roll_cache = model.new_cache(64)
    for cap in (2, 5):
        abi().bci_graph_reset(model.ctx)
        roll = e.rollout(model, seqs, roll_cache, cap=cap, graph=True)
        assert all(bits(a) == bits(b) for a, b in zip(roll, rec)), cap
        assert abi().bci_graph_count(model.ctx) >= 1


def test_graphed_rollout_parity_with_oracle(tiny):
    """The graph-replayed decode against the fp64 oracle (not only against the eager
    path): every logprob of the captured rollout within the end-to-end tolerance."""
    from oracle import model as om
    cfg, weights, seqs, model, cache, blocks = tiny
    abi().bci_graph_reset(model.ctx)
    roll = eng().rollout(model, seqs, model.new_cache(64), cap=3, graph=True)
    assert abi().bci_graph_count(model.ctx) >= 1
    W = om.Weights({k: synth.bf16_bits(v) for k, v in weights.items()})
    worst = 0.0
    for s, got in zip(seqs, roll):
        ref = om.sequence_logprobs(cfg, W, s.tokens, s.prompt_len)
        assert got.shape == ref.shape and np.all(got <= 0)
        worst = max(worst, float(np.max(np.abs(got.astype(np.float64) - ref))))
    print(f"graphed rollout: max |dlogprob| vs oracle = {worst:.3e}", flush=True)
    assert worst <= 2e-2


def test_qwen3_shaped_decode_graph_equals_eager():
    """Full-size decode step (Qwen3-shaped, 28 layers) at B = 4: captured == eager."""
    cfg = synth.QWEN3_1P7B
    weights = synth.make_weights(cfg)
    seqs = synth.rl_sequences(cfg, n_prompts=1, n_responses=4)
    model = eng().Model(cfg, weights, max_tokens=2048, max_seqs=8, max_scored=2048,
                        max_position=1024, seg_keys=64)
    try:
        cache = model.new_cache(4 * 16)
        model.bind_cache(cache)
        blocks = [list(range(16 * i, 16 * i + 16)) for i in range(4)]
        _prefill(model, seqs, blocks)
        for t, plan in enumerate(_decode_plans(model, seqs, blocks, 3)):
            lp_e, lp_g = _eager_and_graph(model, plan)
            assert bits(lp_e) == bits(lp_g), t
        assert abi().bci_graph_count(model.ctx) == 1
    finally:
        model.close()


def test_graph_refuses_fast_mode():
    cfg = synth.TINY
    model = eng().Model(cfg, synth.make_weights(cfg), max_tokens=256, max_seqs=4,
                        max_scored=256, max_position=256, seg_keys=64, mode="fast")
    try:
        cache = model.new_cache(8)
        model.bind_cache(cache)
        s = synth.tiny_sequences(cfg, n=1)[0]
        plan = eng().CallPlan(np.array(s.tokens[:3], np.int32), np.array([0, 3], np.int32),
                              np.zeros(1, np.int32), np.array([[0, 1, 2, 3]], np.int32),
                              np.array([2], np.int32), np.array([s.tokens[3]], np.int32), [])
        with pytest.raises(abi().BciError):
            eng().run_call(model, plan, graph=True)
    finally:
        model.close()
