"""The allocation-free lm_head entry point (bci_lmhead_logprob_noalloc) against the
context entry point it is a variant of (bci_op_lmhead_logprob): identical bits, on two
calls in a row whose second has fewer rows (the fixed device array keeps the first
call's partials; nothing may leak into the second)."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

H, V = 2048, 151936


def test_noalloc_lmhead_equals_context_entry_point():
    from bitwise_consistent_rl_amd import _abi as a
    c = a.ModelConfig()
    for k, v in dict(n_layers=1, hidden=H, n_q_heads=16, n_kv_heads=8, head_dim=128, intermediate=6144,
                     vocab=V, rms_eps=1e-6, rope_theta=1e6, kv_dtype=0, kv_block_tokens=64,
                     attn_segment_keys=0, max_tokens_per_call=512, max_seqs_per_call=8,
                     max_scored_per_call=512, max_position=256, mode=0).items():
        setattr(c, k, v)
    ctx = a.bci_create(c, 0)
    try:
        hs, w, ids = synth.lmhead_inputs(512, hidden=H, vocab=V)
        hs, w = hs.cuda(), w.cuda()
        ids = torch.from_numpy(ids.copy()).cuda()
        ids[5] = -1                                   # an invalid id: NaN on both paths
        for M in (512, 37, 1):
            ref = torch.full((M,), 7.0, dtype=torch.float32, device="cuda")
            got = torch.full((M,), 3.0, dtype=torch.float32, device="cuda")
            a.bci_op_lmhead_logprob(ctx, hs[:M], w, ids[:M], M, H, V, ref)
            torch.cuda.synchronize()
            a.bci_lmhead_logprob_noalloc(hs[:M], w, ids[:M], M, H, V, got)
            torch.cuda.synchronize()
            print(f"M={M}: first logprobs {got[:3].tolist()}", flush=True)
            assert torch.equal(ref.view(torch.int32), got.view(torch.int32)), M
            finite = torch.isfinite(got)
            assert bool(finite.sum() == M - (1 if M > 5 else 0))
            assert bool((got[finite] <= 0).all())
        with pytest.raises(a.BciError):
            a.bci_lmhead_logprob_noalloc(hs, w, ids, 513, H, V, got)
    finally:
        a.bci_destroy(ctx)
