"""Host-side checks of the C ABI that need no GPU: the library loads, exports every
function include/bci.h declares, and rejects bad configurations before touching HIP."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bci.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bci_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from bitwise_consistent_rl_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        pytest.fail("libbci.so is not built (run __graft_entry__.build())")
    return _abi.load()


def test_header_declares_the_boundary():
    fns = declared_functions()
    for must in ("bci_create", "bci_forward_logprobs", "bci_op_gemm_bf16", "bci_op_attention",
                 "bci_op_lmhead_logprob", "bci_op_add_rmsnorm", "bci_op_kv_gather_dequant"):
        assert must in fns


def test_library_exports_every_declared_symbol(lib):
    from bitwise_consistent_rl_amd import _abi
    fns = declared_functions()
    missing = [f for f in fns if not hasattr(lib, f)]
    assert not missing, missing
    assert sorted(_abi.EXPORTS) == fns      # the binding covers the whole header


def _cfg(**kw):
    from bitwise_consistent_rl_amd import _abi
    c = _abi.ModelConfig()
    base = dict(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=768,
                vocab=4096, rms_eps=1e-6, rope_theta=1e6, kv_dtype=0, kv_block_tokens=64,
                attn_segment_keys=0, max_tokens_per_call=128, max_seqs_per_call=8,
                max_scored_per_call=128, max_position=256, mode=0)
    base.update(kw)
    for k, v in base.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("bad", [dict(head_dim=96), dict(hidden=200), dict(n_q_heads=3),
                                 dict(kv_block_tokens=32), dict(attn_segment_keys=100),
                                 dict(max_tokens_per_call=0), dict(kv_dtype=7), dict(mode=9),
                                 dict(intermediate=700), dict(n_q_heads=128, n_kv_heads=1),
                                 dict(n_experts=65, top_k=2, expert_intermediate=128),
                                 dict(n_experts=64, top_k=9, expert_intermediate=128),
                                 dict(n_experts=8, top_k=2, expert_intermediate=100),
                                 dict(n_experts=8, top_k=2, expert_intermediate=128,
                                      n_shared_experts=2)])
def test_create_rejects_bad_config_before_any_device_call(lib, bad):
    from bitwise_consistent_rl_amd import _abi
    h = ctypes.c_void_p()
    st = lib.bci_create(ctypes.byref(_cfg(**bad)), 0, ctypes.byref(h))
    assert st == _abi.BCI_E_INVALID and not h.value


def test_bad_split_mode_rejected(lib):
    from bitwise_consistent_rl_amd import _abi
    h = ctypes.c_void_p()
    assert lib.bci_create(ctypes.byref(_cfg(attn_split_mode=3)), 0, ctypes.byref(h)) == _abi.BCI_E_INVALID


def test_null_context_calls_return_invalid(lib):
    from bitwise_consistent_rl_amd import _abi
    assert lib.bci_set_batch(None, None, None) == _abi.BCI_E_INVALID
    assert lib.bci_forward_logprobs(None, None, None) == _abi.BCI_E_INVALID
    assert lib.bci_op_gemm_bf16(None, None, None, None, 1, 128, 64, 0, None) == _abi.BCI_E_INVALID
    lib.bci_destroy(None)


def test_lmhead_noalloc_rejects_on_the_host(lib):
    """The allocation-free lm_head entry point checks every argument before any HIP
    call: bad pointers or shapes, and sizes beyond its fixed device array."""
    from bitwise_consistent_rl_amd import _abi
    f = lib.bci_lmhead_logprob_noalloc
    p = ctypes.c_void_p(256)          # never dereferenced: the checks come first
    assert f(None, p, p, 1, 2048, 151936, p, None) == _abi.BCI_E_INVALID
    assert f(p, p, p, 1, 2000, 151936, p, None) == _abi.BCI_E_INVALID      # H % 64
    assert f(p, p, p, -1, 2048, 151936, p, None) == _abi.BCI_E_INVALID
    assert f(p, p, p, 513, 2048, 151936, p, None) == _abi.BCI_E_WORKSPACE  # 513 x 594 pairs
    assert f(p, p, p, _abi.BCI_LMHEAD_NOALLOC_MAX_ROWS + 1, 2048, 256, p, None) == _abi.BCI_E_WORKSPACE
