"""A Mamba-2-style selective state-space layer (the recurrence only), in fp64 on the CPU.

Test infrastructure only.  Nothing on the product path imports this.

The report's second workload, Nemotron-3.5, mixes Mamba-2, attention and MoE layers
(page "Finish RL Training Faster" digest, section "两组结果，要连同分母一起读"), and
porting the method to it meant recursive arithmetic in which decode replays the
chunked computation order of prefill and training reuses the same operator, rather
than only asking that the final state come out close (same page, section
"一致性有多个层面，修好一处还不能验收").  The pages give no formula.  The reading is
the Mamba-2 selective state-space recurrence with a scalar decay per head:

    h_t = exp(A_h * dt[t,h]) * h_{t-1} + dt[t,h] * B[t,g] (outer) x[t,h]
    y[t,h] = C[t,g] . h_t + D_h * x[t,h]

per head h (state h_t of shape [N, P]), with the B and C inputs shared by the heads of
a group g = h // (H / G), and h_{-1} = 0 at the start of a sequence.  dt is the
per-head step after its softplus (given), A_h < 0 and D_h are per-head constants.

The oracle is that recurrence written out, one position after another; the chunked
form the product path uses is a reordering of the same sum and is not imitated here.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_round

bf = bf16_round


def ssd_recurrence(x, dt, A, B, C, D, h0=None):
    """The recurrence over positions 0..T-1.

    x [T, H, P], dt [T, H], A [H], B and C [T, G, N], D [H], h0 [H, N, P] (zero when
    None).  Returns (y [T, H, P] float64 -- not rounded, h_T [H, N, P])."""
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    g_of_h = np.arange(H) // (H // G)
    h = np.zeros((H, N, P)) if h0 is None else np.array(h0, dtype=np.float64)
    y = np.empty((T, H, P))
    for t in range(T):
        decay = np.exp(A * dt[t])                                    # [H]
        Bt, Ct = B[t][g_of_h], C[t][g_of_h]                          # [H, N]
        h = decay[:, None, None] * h + dt[t][:, None, None] * Bt[:, :, None] * x[t][:, None, :]
        y[t] = np.einsum("hn,hnp->hp", Ct, h) + D[:, None] * x[t]
    return y, h


def ssd_layer(x, dt, A, B, C, D, h0=None):
    """The layer's stored output: y rounded to bf16 (float64 values), and the state."""
    y, h = ssd_recurrence(x, dt, A, B, C, D, h0)
    return bf(y), h
