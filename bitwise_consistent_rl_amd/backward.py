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
VOCAB_SLICE = 4096   # contraction slice of the lm_head backward's dz . E


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


def gemm_ksplit(ctx: int, a: torch.Tensor, w: torch.Tensor, epi: int, k_split: int) -> torch.Tensor:
    """a . w^T with the contraction in fixed slices of k_split summed in slice order
    (for few output tiles over a long contraction)."""
    M, K = a.shape
    N = w.shape[0]
    dtype = torch.float32 if epi == abi.BCI_EPI_F32 else BF
    c = torch.empty(M, N, dtype=dtype, device=a.device)
    ws = torch.empty((K + k_split - 1) // k_split * M * N, dtype=torch.float32, device=a.device)
    abi.bci_op_gemm_bf16_ksplit(ctx, a, w, c, M, N, K, k_split, epi, ws)
    return c


def linear_backward(ctx: int, x: torch.Tensor, w: torch.Tensor, dy: torch.Tensor, wT: torch.Tensor = None,
                    dx_k_split: int = None):
    """y = x . w^T (x [M, K], w [N, K], dy [M, N] bf16; N % 64 == 0).
    Returns dx [M, K] bf16 and dw [N, K] fp32.  dx_k_split: contraction slice of the dx
    product (over N), for a long N with few output tiles."""
    M, K = x.shape
    N = w.shape[0]
    if N % 64:
        raise ValueError("the output width of the forward GEMM must be a multiple of 64")
    if wT is None:
        wT = transpose(ctx, w, ld=N)                     # [K, N]
    if dx_k_split:
        dx = gemm_ksplit(ctx, dy, wT, abi.BCI_EPI_BF16, dx_k_split)   # [M, K], slices of N
    else:
        dx = gemm(ctx, dy, wT, abi.BCI_EPI_BF16)         # [M, K], contraction over N
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
    """lp = z[id] - logsumexp(z), z = hf . E^T (fp32 logits).  Returns (dhf bf16, dE fp32).
    dhf = dz . E contracts over the whole vocabulary onto few output tiles, so it runs in
    fixed vocabulary slices of VOCAB_SLICE summed in slice order."""
    M = hf.shape[0]
    V = emb.shape[0]
    z = gemm(ctx, hf, emb, abi.BCI_EPI_F32)                        # [M, V] fp32
    dz = torch.empty(M, V, dtype=BF, device=hf.device)
    abi.bci_op_logprob_backward_dz(ctx, z, ids, gout, M, V, dz)
    del z
    return linear_backward(ctx, hf, emb, dz, wT=embT, dx_k_split=VOCAB_SLICE if V > VOCAB_SLICE else None)


def attention_backward(ctx: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                       do: torch.Tensor, split: bool = True):
    """Causal GQA attention backward of one sequence (positions 0..L-1): (dq, dk, dv) bf16.
    split: give the library its part buffer (fp32 [2, 4, L, nkv * d]) so the dK/dV pass
    can cut long sequences' rows into fixed parts summed in order."""
    L = q.shape[0]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(2 * 4 * k.numel(), dtype=torch.float32, device=q.device) if split else None
    abi.bci_op_attention_backward(ctx, q, k, v, o, do, L, dq, dk, dv, ws)
    return dq, dk, dv


def rope_backward(ctx: int, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor) -> torch.Tensor:
    """[R^T dq, R^T dk, dv] for the current batch, laid out as the forward's qkv rows."""
    T = dq.shape[0]
    dqkv = torch.empty(T, dq.shape[1] + dk.shape[1] + dv.shape[1], dtype=BF, device=dq.device)
    abi.bci_op_rope_backward(ctx, dq, dk, dv, dqkv)
    return dqkv


def decoder_layer_forward(ctx: int, layer: int, w: dict, r_in: torch.Tensor, m_prev: torch.Tensor = None,
                          *, nq: int, nkv: int, d: int, inter: int, eps: float) -> dict:
    """One pre-norm decoder layer over the current batch (one sequence at positions
    0..L-1, its cache bound), op by op with the forward's own entry points, keeping what
    the backward needs:
        r1, h = AddNorm(m_prev, r_in, attn_norm);  q, k, v = RoPE(split(h Wqkv^T)) -> cache
        o = Attn(q, cache);  a = o Wo^T;  r2, h2 = AddNorm(a, r1, mlp_norm);  m = MLP(h2)
    ``w``: attn_norm, wqkv, wo, mlp_norm, wgu, wd (bf16).  Returns the saved tensors and
    the outputs r (= r2) and m."""
    L, H = r_in.shape
    r = r_in.clone()
    h = torch.empty_like(r)
    abi.bci_op_add_rmsnorm(ctx, m_prev, r, h, w["attn_norm"], L, H, eps)
    r1 = r.clone()
    qkv = gemm(ctx, h, w["wqkv"], abi.BCI_EPI_BF16)
    q = torch.empty(L, nq * d, dtype=BF, device=r.device)
    abi.bci_op_rope_kv_write(ctx, qkv, q, layer)
    o = torch.empty_like(q)
    abi.bci_op_attention(ctx, q, layer, o)
    a = gemm(ctx, o, w["wo"], abi.BCI_EPI_BF16)
    h2 = torch.empty_like(r)
    abi.bci_op_add_rmsnorm(ctx, a, r, h2, w["mlp_norm"], L, H, eps)
    act = gemm(ctx, h2, w["wgu"], abi.BCI_EPI_SILU_MUL, out_cols=inter)
    m = gemm(ctx, act, w["wd"], abi.BCI_EPI_BF16)
    k = torch.empty(L, nkv * d, dtype=BF, device=r.device)
    v = torch.empty_like(k)
    abi.bci_op_kv_gather_dequant(ctx, 0, L, layer, k, v)    # the keys and values attended to
    return dict(r_mid=r1, h=h, q=q, K=k, V=v, o=o, r=r, h2=h2, m=m)


def decoder_layer_backward(ctx: int, w: dict, saved: dict, d_r: torch.Tensor, d_m: torch.Tensor, *,
                           inter: int, eps: float) -> dict:
    """Gradient of ``decoder_layer_forward``'s layer, the current batch still set: the
    layer run backwards, every rounding (and an FP8 cache's quantiser) taken as the
    identity.  d_r, d_m: gradients reaching the outputs r2 and m.  Returns d_r_in (also
    the gradient of m_prev) in bf16 and the weight gradients in fp32."""
    L = d_r.shape[0]
    dh2, dwgu, dwd, _, _ = mlp_backward(ctx, saved["h2"], w["wgu"], w["wd"], d_m, inter)
    dr2, dg2, _ = add_rmsnorm_backward(ctx, saved["r"], w["mlp_norm"], dh2, eps, d_r)
    do, dwo = linear_backward(ctx, saved["o"], w["wo"], dr2)
    dq, dk, dv = attention_backward(ctx, saved["q"], saved["K"], saved["V"], saved["o"], do)
    dqkv = rope_backward(ctx, dq, dk, dv)
    dh, dwqkv = linear_backward(ctx, saved["h"], w["wqkv"], dqkv)
    dr1, dg1, _ = add_rmsnorm_backward(ctx, saved["r_mid"], w["attn_norm"], dh, eps, dr2)
    return dict(d_r_in=dr1, attn_norm=dg1, wqkv=dwqkv, wo=dwo, mlp_norm=dg2, wgu=dwgu, wd=dwd)
