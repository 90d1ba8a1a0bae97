"""Shared helpers of the GPU tests (no method arithmetic here)."""
import numpy as np
import torch

import synth
from oracle.codecs import bf16_decode

BF = torch.bfloat16


def f64(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> float64 numpy, by exact widening of the bits on the CPU."""
    return bf16_decode(synth.bf16_bits(t))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of the bf16 grid at |x| (2^-133 at zero)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(ax)).astype(np.int64) - 7)


def assert_bf16_close(got, ref, abs_bound=None, max_ulp=2, frac_exact=0.99, what=""):
    """got and ref on the bf16 grid: |got - ref| <= max_ulp ulps of the larger of the two
    (plus an optional absolute bound for cancellation), and at least ``frac_exact`` of
    them within 1 ulp."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    ulp = bf16_ulp(np.maximum(np.abs(got), np.abs(ref)))   # the coarser grid at a binade edge
    tol = max_ulp * ulp
    if abs_bound is not None:
        tol = tol + abs_bound
    bad = d > tol
    if bad.any():
        idx = np.argwhere(bad)[:5]
        pairs = [(tuple(int(v) for v in i), float(got[tuple(i)]), float(ref[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance, e.g. {pairs}")
    within1 = np.mean(d <= ulp + (0 if abs_bound is None else abs_bound))
    assert within1 >= frac_exact, (what, within1)


def cuda(t):
    return t.to("cuda")


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return bool(torch.equal(a.contiguous().view(torch.uint8 if a.element_size() == 1 else torch.int16
                                               if a.element_size() == 2 else torch.int32).cpu(),
                            b.contiguous().view(torch.uint8 if b.element_size() == 1 else torch.int16
                                                if b.element_size() == 2 else torch.int32).cpu()))
