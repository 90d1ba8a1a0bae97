"""MoE layer with invariant routing on the GPU: router top-K with lowest-index ties
(exact against the oracle), the grouped expert GEMMs and the FP32 slot-order combine
(parity with the oracle), and per-token invariance across the token count."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import BF, cuda, f64, same_bits
from oracle import ops

pytestmark = pytest.mark.gpu

CFG = synth.MOE


def abi():
    from bitwise_consistent_rl_amd import _abi
    return _abi


@pytest.fixture(scope="module")
def moe():
    a = abi()
    c = a.ModelConfig()
    for k, v in dict(n_layers=1, hidden=CFG.hidden, n_q_heads=32, n_kv_heads=8, head_dim=128,
                     intermediate=CFG.expert_intermediate, vocab=128, rms_eps=1e-6, rope_theta=1e6,
                     kv_dtype=0, kv_block_tokens=64, attn_segment_keys=2048,
                     max_tokens_per_call=8192, max_seqs_per_call=8, max_scored_per_call=8,
                     max_position=64, mode=0, n_experts=CFG.n_experts, top_k=CFG.top_k,
                     expert_intermediate=CFG.expert_intermediate, n_shared_experts=1).items():
        setattr(c, k, v)
    ctx = a.bci_create(c, 0)
    w = synth.moe_weights(CFG)
    g = {k: cuda(v) for k, v in w.items()}
    h_all = synth.normal_bf16((8192, CFG.hidden), index=50)
    yield ctx, w, g, h_all, cuda(h_all)
    torch.cuda.synchronize()
    a.bci_destroy(ctx)


def topk(ctx, logits_np):
    T = logits_np.shape[0]
    z = torch.from_numpy(np.ascontiguousarray(logits_np, np.float32)).cuda()
    ids = torch.empty(T, CFG.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, CFG.top_k, dtype=torch.float32, device="cuda")
    abi().bci_op_moe_topk(ctx, z, T, ids, w)
    torch.cuda.synchronize()
    return ids, w


def forward(ctx, g, h, ids, w):
    T = h.shape[0]
    out = torch.empty(T, CFG.hidden, dtype=BF, device="cuda")
    abi().bci_op_moe_forward(ctx, h, ids, w, T, g["wgu"], g["wd"], g["swgu"], g["swd"], out)
    torch.cuda.synchronize()
    return out


def test_topk_ties_exact(moe):
    ctx = moe[0]
    z = synth.router_logits_quantised(1024)
    ids, w = topk(ctx, z)
    ref = ops.topk_ties(z, CFG.top_k)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref)
    np.testing.assert_array_equal(ids[0].cpu().numpy(), np.arange(6))      # all-equal row
    wref = ops.topk_weights(z, ref)
    np.testing.assert_allclose(w.cpu().numpy(), wref, rtol=2e-6, atol=1e-7)
    # heavy ties: every row is one of only 5 distinct values
    z2 = (np.random.default_rng(3).integers(-2, 3, size=(512, 64)) / 64).astype(np.float32)
    ids2, _ = topk(ctx, z2)
    np.testing.assert_array_equal(ids2.cpu().numpy(), ops.topk_ties(z2, CFG.top_k))


def _router_logits(ctx, g, h_gpu):
    """fp32 router logits h . Wr^T from the invariant GEMM, quantised to 1/64 steps on
    the host so that ties are frequent."""
    T = h_gpu.shape[0]
    z = torch.empty(T, CFG.n_experts, dtype=torch.float32, device="cuda")
    abi().bci_op_gemm_bf16(ctx, h_gpu, g["wr"], z, T, CFG.n_experts, CFG.hidden, abi().BCI_EPI_F32)
    torch.cuda.synchronize()
    zq = np.rint(z.cpu().numpy().astype(np.float64) * 64) / 64
    return zq.astype(np.float32)


def _moe_check(got, ref, what):
    """Element-wise: |got - ref| <= 4 ulp of the coarser value + 2^-7 of the row's RMS.
    The second term covers outputs near zero, where the combine of seven bf16 expert
    rows cancels; a dropped or mis-weighted slot, or a row taken from another token,
    moves elements by about w_s * |y_s| >= 0.1 of the row's RMS, far above it.  Also
    the relative RMS error of the whole block and the fraction within one ulp."""
    from gpu_util import bf16_ulp
    d = np.abs(got - ref)
    ulp = bf16_ulp(np.maximum(np.abs(got), np.abs(ref)))
    rms_row = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    tol = 4 * ulp + 2.0 ** -7 * rms_row
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    within1 = float(np.mean(d <= ulp))
    worst_ulp = float(np.max(d / ulp))
    worst_rms = float(np.max(d / rms_row))
    print(f"moe parity {what}: relative RMS {rel:.2e}, within 1 ulp {within1:.5f}, "
          f"max {worst_ulp:.1f} ulp, max {worst_rms:.2e} of the row RMS", flush=True)
    bad = d > tol
    assert not bad.any(), (what, int(bad.sum()), np.argwhere(bad)[:5].tolist())
    assert rel <= 5e-3 and within1 >= 0.99, (what, rel, within1)


def _oracle_moe(w, h64, z):
    """The oracle's own routing (top-K with lowest-index ties, softmax over the selected
    logits) and MoE layer on the seeded inputs; nothing here comes from the GPU."""
    bits = {k: synth.bf16_bits(v) for k, v in w.items()}
    ids = ops.topk_ties(z, CFG.top_k)
    wts = ops.topk_weights(z, ids)
    return ids, ops.moe_layer(h64, ids, wts, bits["wgu"], bits["wd"], bits["swgu"], bits["swd"],
                              CFG.expert_intermediate)


# T = 1 .. 512 run the per-group skinny expert schedule (at most 128 rows per expert),
# 2048 the tiled grouped schedule
@pytest.mark.parametrize("T", [1, 7, 64, 512, 2048])
def test_moe_forward_parity(moe, T):
    ctx, w, g, h_all, gh = moe
    z = synth.router_logits_quantised(T, seed=11)
    ids, wt = topk(ctx, z)
    ref_ids, ref = _oracle_moe(w, f64(h_all[:T]), z)
    np.testing.assert_array_equal(ids.cpu().numpy(), ref_ids)
    out = forward(ctx, g, gh[:T].contiguous(), ids, wt)
    _moe_check(f64(out), ref, f"T={T}")


def test_moe_forward_parity_sampled_8192(moe):
    """All 8192 tokens through the GPU layer (tiled grouped schedule); 48 seeded rows
    against the oracle, which runs on those rows alone (each row is independent)."""
    ctx, w, g, h_all, gh = moe
    T = 8192
    z = synth.router_logits_quantised(T, seed=11)
    ids, wt = topk(ctx, z)
    out = forward(ctx, g, gh, ids, wt)
    rows = np.sort(np.random.default_rng(23).choice(T, size=48, replace=False))
    ref_ids, ref = _oracle_moe(w, f64(h_all[torch.from_numpy(rows)]), z[rows])
    np.testing.assert_array_equal(ids.cpu().numpy()[rows], ref_ids)
    _moe_check(f64(out)[rows], ref, "T=8192 sampled")


def test_moe_rows_invariant_across_T(moe):
    ctx, w, g, h_all, gh = moe
    z = _router_logits(ctx, g, gh)
    ids, wt = topk(ctx, z)
    full = forward(ctx, g, gh, ids, wt)
    for T in (1, 7, 64, 512, 2048):
        idsT, wT = topk(ctx, z[:T])
        assert same_bits(idsT, ids[:T]) and same_bits(wT, wt[:T])
        part = forward(ctx, g, gh[:T].contiguous(), idsT, wT)
        assert same_bits(part, full[:T]), T
    perm = np.array(synth.shuffled(list(range(8192)), index=5))[:3000]
    pt = torch.from_numpy(perm).cuda()
    idsP, wP = topk(ctx, z[perm])
    shuf = forward(ctx, g, gh[pt].contiguous(), idsP, wP)
    assert same_bits(shuf, full[pt])


def test_moe_invalid_expert_id_gives_nan_row(moe):
    ctx, w, g, h_all, gh = moe
    ids = torch.tensor([[0, 1, 2, 3, 4, 5], [0, 1, 2, 3, 4, 99]], dtype=torch.int32, device="cuda")
    wt = torch.full((2, 6), 1 / 6, dtype=torch.float32, device="cuda")
    out = forward(ctx, g, gh[:2].contiguous(), ids, wt).float().cpu()
    assert torch.isfinite(out[0]).all() and torch.isnan(out[1]).all()
