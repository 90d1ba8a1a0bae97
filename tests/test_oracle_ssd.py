"""Pins of the state-space oracle (CPU only) against formulas other than the
recurrence itself: the quadratic (attention-like) form of the same sum evaluated by
brute force, closed forms for special inputs, and the algebra of carried state.
A wrong decay index (exp of dt at t instead of t..s+1), a dropped dt on the input, a
swapped B/C or a wrong head-to-group map fails at least one of these."""
import numpy as np
import pytest

from oracle import ssd


def _inputs(T=37, H=6, G=3, N=5, P=4, seed=0):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((T, H, P)), dt=np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), (T, H))),
                A=-np.exp(rng.uniform(0, np.log(16), H)), B=rng.standard_normal((T, G, N)),
                C=rng.standard_normal((T, G, N)), D=rng.standard_normal(H))


def _quadratic(x, dt, A, B, C, D):
    """y_t = sum_{s <= t} (C_t . B_s) exp(A * sum_{k=s+1..t} dt_k) dt_s x_s + D x_t."""
    T, H, P = x.shape
    G = B.shape[1]
    y = np.zeros((T, H, P))
    for h in range(H):
        g = h // (H // G)
        for t in range(T):
            acc = D[h] * x[t, h]
            for s in range(t + 1):
                decay = np.exp(A[h] * dt[s + 1:t + 1, h].sum())
                acc = acc + (C[t, g] @ B[s, g]) * decay * dt[s, h] * x[s, h]
            y[t, h] = acc
    return y


@pytest.mark.parametrize("seed", [0, 1])
def test_recurrence_equals_quadratic_form(seed):
    kw = _inputs(seed=seed)
    y, _ = ssd.ssd_recurrence(**kw)
    np.testing.assert_allclose(y, _quadratic(**kw), rtol=1e-11, atol=1e-11)


def test_no_decay_is_a_prefix_sum():
    kw = _inputs(seed=2)
    kw["A"] = np.zeros_like(kw["A"])
    y, h = ssd.ssd_recurrence(**kw)
    x, dt, B, C, D = kw["x"], kw["dt"], kw["B"], kw["C"], kw["D"]
    H, G = x.shape[1], B.shape[1]
    g = np.arange(H) // (H // G)
    Bh, Ch = B[:, g], C[:, g]                                     # [T, H, N]
    S = np.cumsum(dt[:, :, None, None] * Bh[..., None] * x[:, :, None, :], axis=0)   # [T, H, N, P]
    np.testing.assert_allclose(y, np.einsum("thn,thnp->thp", Ch, S) + D[None, :, None] * x, rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(h, S[-1], rtol=1e-12, atol=1e-12)


def test_zero_step_passes_only_the_skip():
    kw = _inputs(seed=3)
    kw["dt"] = np.zeros_like(kw["dt"])
    y, h = ssd.ssd_recurrence(**kw)
    np.testing.assert_array_equal(y, kw["D"][None, :, None] * kw["x"])
    assert not h.any()


def test_single_impulse_decays_geometrically():
    kw = _inputs(T=20, seed=4)
    kw["x"][1:] = 0.0
    kw["D"][:] = 0.0
    c = 0.05
    kw["dt"][:] = c
    y, _ = ssd.ssd_recurrence(**kw)
    H, G = kw["x"].shape[1], kw["B"].shape[1]
    for h in range(H):
        g = h // (H // G)
        t = np.arange(20)
        want = (kw["C"][:, g] @ kw["B"][0, g])[:, None] * np.exp(kw["A"][h] * c * t)[:, None] * c * kw["x"][0, h]
        np.testing.assert_allclose(y[:, h], want, rtol=1e-12, atol=1e-14)


def test_carried_state_splits_a_sequence():
    kw = _inputs(T=40, seed=5)
    y_all, h_all = ssd.ssd_recurrence(**kw)
    first = {k: (v[:17] if k in ("x", "dt", "B", "C") else v) for k, v in kw.items()}
    rest = {k: (v[17:] if k in ("x", "dt", "B", "C") else v) for k, v in kw.items()}
    y1, h1 = ssd.ssd_recurrence(**first)
    y2, h2 = ssd.ssd_recurrence(**rest, h0=h1)
    np.testing.assert_array_equal(np.concatenate([y1, y2]), y_all)
    np.testing.assert_array_equal(h2, h_all)


def test_heads_of_a_group_share_b_and_c():
    kw = _inputs(T=12, H=4, G=2, seed=6)
    # heads 0 and 1 (group 0) given identical x, dt, A, D produce identical outputs;
    # head 2 (group 1) with the same per-head inputs does not
    for k in ("x", "dt"):
        kw[k][:, 1] = kw[k][:, 0]
        kw[k][:, 2] = kw[k][:, 0]
    for k in ("A", "D"):
        kw[k][1] = kw[k][0]
        kw[k][2] = kw[k][0]
    y, _ = ssd.ssd_recurrence(**kw)
    np.testing.assert_array_equal(y[:, 1], y[:, 0])
    assert np.abs(y[:, 2] - y[:, 0]).max() > 1e-3
