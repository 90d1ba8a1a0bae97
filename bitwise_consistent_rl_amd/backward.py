"""Gradients of the forward's operators, composed from C-ABI calls (no arithmetic here).

Every gradient GEMM is ``bci_op_gemm_bf16`` -- the forward's invariant GEMM -- on
transposed operands: for y = x . w^T,
    dx = dy . w       = GEMM(A = dy, W = w^T)           (contraction over w's rows)
    dw = dy^T . x     = GEMM(A = dy^T, W = x^T), fp32   (contraction over the tokens,
                                                          padded to 64 with zero rows)
so each element is one ascending fp32 MFMA chain and rows of dx do not depend on the
other rows of the batch.  The pieces around the GEMMs (transpose, add+RMSNorm,
SiLU*up and log-softmax backward) are kernels of the library.  torch provides the
buffers and the stream.
"""
from __future__ import annotations

import torch

from . import _abi as abi

BF = torch.bfloat16


def _pad64(n: int) -> int:
    return (n + 63) // 64 * 64


def transpose(ctx: int, x: torch.Tensor, ld: int = None) -> torch.Tensor:
    """x [R, C] bf16 -> [C, ld] bf16 with zero columns past R (ld defaults to R padded to 64)."""
    R, C = x.shape
    ld = _pad64(R) if ld is None else ld
    out = torch.empty(C, ld, dtype=BF, device=x.device)
    abi.bci_op_transpose_bf16(ctx, x, out, R, C, ld)
    return out


def gemm(ctx: int, a: torch.Tensor, w: torch.Tensor, epi: int, out_cols: int = None) -> torch.Tensor:
    M, K = a.shape
    N = w.shape[0]
    dtype = torch.float32 if epi == abi.BCI_EPI_F32 else BF
    c = torch.empty(M, out_cols or N, dtype=dtype, device=a.device)
    abi.bci_op_gemm_bf16(ctx, a, w, c, M, N, K, epi)
    return c


def linear_backward(ctx: int, x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, wT: torch.Tensor = None):
    """y = x . w^T (x [M, K], w [N, K], dy [M, N] bf16; N % 64 == 0).
    Returns dx [M, K] bf16 and dw [N, K] fp32."""
    M, K = x.shape
    N = w.shape[0]
    if N % 64:
        raise ValueError("the output width of the forward GEMM must be a multiple of 64")
    if wT is None:
        wT = transpose(ctx, w, ld=N)                     # [K, N]
    dx = gemm(ctx, dy, wT, abi.BCI_EPI_BF16)             # [M, K], contraction over N
    Mp = _pad64(M)
    dw = gemm(ctx, transpose(ctx, dy, Mp), transpose(ctx, x, Mp), abi.BCI_EPI_F32)   # [N, K]
    return dx, dw


def add_rmsnorm_backward(ctx: int, r: torch.Tensor, g: torch.Tensor, dh: torch.Tensor, eps: float,
                         dr_in: torch.Tensor = None):
    """Returns (dr [rows, H] bf16, dg [H] fp32, rstd [rows] fp32)."""
    rows, H = r.shape
    dr = torch.empty_like(r)
    rstd = torch.empty(rows, dtype=torch.float32, device=r.device)
    dg = torch.empty(H, dtype=torch.float32, device=r.device)
    abi.bci_op_add_rmsnorm_backward(ctx, r, g, dh, dr_in, dr, rstd, dg, rows, H, eps)
    return dr, dg, rstd


def mlp_backward(ctx: int, h: torch.Tensor, wgu: torch.Tensor, wd: torch.Tensor, dout: torch.Tensor,
                 inter: int):
    """The SiLU-gated MLP out = act . wd^T, act = bf(silu(g) u), [g u] = bf(h . wgu^T).
    The forward's gate/up outputs and activation are recomputed with the forward's own
    GEMMs (same bits).  Returns (dh bf16, dwgu fp32, dwd fp32, gu, act)."""
    M = h.shape[0]
    gu = gemm(ctx, h, wgu, abi.BCI_EPI_BF16)                       # [M, 2I]
    act = gemm(ctx, h, wgu, abi.BCI_EPI_SILU_MUL, out_cols=inter)  # [M, I]
    dact, dwd = linear_backward(ctx, act, wd, dout)
    dgu = torch.empty_like(gu)
    abi.bci_op_silu_mul_backward(ctx, gu, dact, dgu, M, inter)
    dh, dwgu = linear_backward(ctx, h, wgu, dgu)
    return dh, dwgu, dwd, gu, act


def logprob_backward(ctx: int, hf: torch.Tensor, emb: torch.Tensor, ids: torch.Tensor,
                     gout: torch.Tensor, embT: torch.Tensor = None):
    """lp = z[id] - logsumexp(z), z = hf . E^T (fp32 logits).  Returns (dhf bf16, dE fp32)."""
    M = hf.shape[0]
    V = emb.shape[0]
    z = gemm(ctx, hf, emb, abi.BCI_EPI_F32)                        # [M, V] fp32
    dz = torch.empty(M, V, dtype=BF, device=hf.device)
    abi.bci_op_logprob_backward_dz(ctx, z, ids, gout, M, V, dz)
    del z
    return linear_backward(ctx, hf, emb, dz, wT=embT)
