"""Gradients of the attention forward, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed
----------------
"FlashAttention 4: Atenção Mais Rápida e Eficiente em Memória para LLMs",
section "Principais Conclusões", and "FlashAttention-4 no Blackwell B200:
pipelining de kernels e o que FP4 realmente muda", section "Redução de
tráfego no backward", name the backward pass (the gradients of O with
respect to Q, K and V, which training needs) as the counterpart of the
forward kernel.
The pages give no formulas; the gradients are those of the plain definition
in ``attention.attention_forward`` (s = scale q k^T, p = softmax_j(s),
o = p v), obtained by the chain rule:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_c dO_ic O_ic            (= sum_j P_ij dP_ij)
    dS = P * (dP - D)                  (softmax Jacobian)
    dQ = scale dS K
    dK = scale dS^T Q

with P the normalised probabilities of the forward (masked keys have
P = 0).  Reading where the pages are silent: the gradient of the
log-sum-exp output is not propagated (it is an auxiliary output).
"""

import numpy as np

from .attention import attention_head_rows


def attention_backward_head(q, k, v, do, scale, causal):
    """One head: q, k, v, do float64 [N][d].  Returns (dq, dk, dv) [N][d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n = q.shape[0]
    s = scale * np.matmul(q, k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] <= np.arange(n)[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / e.sum(axis=1, keepdims=True)
    o = np.matmul(p, v)
    dv = np.matmul(p.T, do)
    dp = np.matmul(do, v.T)
    delta = (do * o).sum(axis=1, keepdims=True)
    ds = p * (dp - delta)
    dq = scale * np.matmul(ds, k)
    dk = scale * np.matmul(ds.T, q)
    return dq, dk, dv


def attention_backward(q, k, v, do, scale, causal):
    """[B][N][H][d] float64 tensors; returns (dq, dk, dv) of that shape."""
    q = np.asarray(q, dtype=np.float64)
    B, N, H, d = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(q)
    dv = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            a, bb, c = attention_backward_head(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h],
                                               scale, causal)
            dq[b, :, h], dk[b, :, h], dv[b, :, h] = a, bb, c
    return dq, dk, dv


def attention_delta(o, do):
    """D [B][H][N] = sum over d of dO * O, from [B][N][H][d] tensors."""
    return np.einsum("bnhd,bnhd->bhn", np.asarray(o, dtype=np.float64),
                     np.asarray(do, dtype=np.float64))
