"""The measured MFMA rate used as the sustained-peak denominator: finite, below the
datasheet peak, and no lower with all-zero operands (less switching power) than with
random ones."""
import pytest

pytestmark = pytest.mark.gpu


def test_measured_mfma_rate_is_sane():
    from bitwise_consistent_rl_amd import _abi
    rnd = _abi.bci_measure_mfma_rate(0, True)
    zer = _abi.bci_measure_mfma_rate(0, False)
    print(f"sustained bf16 MFMA rate: random {rnd:.1f}, zeros {zer:.1f} TFLOP/s", flush=True)
    assert 200.0 < rnd < 2600.0 and 200.0 < zer < 2600.0
    assert zer >= 0.95 * rnd
