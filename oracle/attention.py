"""The plain definition of the attention forward, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed
----------------
"FlashAttention-4 no Blackwell B200: pipelining de kernels e o que FP4
realmente muda", section "Por que o Blackwell exige mais do que
multiplicações rápidas", gives the operation as softmax(Q K^T / sqrt(d)) V;
"FlashAttention 4: Atenção Mais Rápida e Eficiente em Memória para LLMs",
section "Introdução", describes the same three steps (scores Q x K, a
softmax normalisation, a product with V); and the dev.to page "FlashAttention-4
em Blackwell B200", section 6 (FAQ, question 2), states that the tiled method
is exact, with the same softmax as the original attention.  So the oracle is
the definition written out, with no tiling:

    s_ij  = scale * sum_k q_ik k_jk          for every visible key j
    m_i   = max_j s_ij
    e_ij  = exp(s_ij - m_i)
    l_i   = sum_j e_ij
    o_i   = sum_j e_ij v_j / l_i
    lse_i = m_i + ln(l_i)

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * layout: Q, K, V, O are [B][N][H][d], as in the bfloat16 usage example of
    "FlashAttention-3: Pipeline Assíncrono ...", section "Implementando
    FlashAttention-3 em produção"; the log-sum-exp is [B][H][N];
  * lse uses the natural logarithm of the scaled scores;
  * causal: key j is visible to query i iff j <= i (square problem, so the
    top-left and bottom-right alignments coincide and every row sees key 0);
  * a row with no visible key (unreachable here) gives o = 0, lse = -inf;
  * subtracting the row maximum m_i before exponentiating is the usual
    overflow guard; it does not change the value.
A library matrix product (numpy.matmul, float64) serves as the dot-product
step; the score matrix is materialised one block of query rows at a time.
"""

import numpy as np

_ROW_BLOCK = 512


def attention_head_rows(q, k, v, scale, causal, rows=None):
    """Attention for one (batch, head): q, k, v are float64 [N][d].

    ``rows`` selects the query rows to evaluate (default: all).  Returns
    (o [R][d], lse [R]) in float64 for the selected rows, in the given order.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows, dtype=np.int64)
    o = np.empty((rows.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.empty(rows.shape[0], dtype=np.float64)
    keys = np.arange(k.shape[0])
    for r0 in range(0, rows.shape[0], _ROW_BLOCK):
        rb = rows[r0:r0 + _ROW_BLOCK]
        s = scale * np.matmul(q[rb], k.T)                    # s_ij
        if causal:
            s = np.where(keys[None, :] <= rb[:, None], s, -np.inf)
        m = s.max(axis=1)                                    # m_i
        empty = ~np.isfinite(m)
        m_safe = np.where(empty, 0.0, m)
        e = np.exp(s - m_safe[:, None])                      # e_ij
        l = e.sum(axis=1)                                    # l_i
        l_safe = np.where(empty, 1.0, l)
        o[r0:r0 + rb.shape[0]] = np.matmul(e, v) / l_safe[:, None]
        lse[r0:r0 + rb.shape[0]] = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return o, lse


def attention_forward(q, k, v, scale, causal, rows=None):
    """Full attention forward on [B][N][H][d] float64 tensors.

    Returns (o, lse).  Without ``rows``: o is [B][N][H][d] and lse [B][H][N].
    With ``rows`` (an int array [B][H][R], per-head query rows): o is
    [B][H][R][d] and lse [B][H][R], in the order of ``rows``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must all be [B][N][H][d] of one shape")
    B, N, H, d = q.shape
    if rows is None:
        o = np.empty((B, N, H, d), dtype=np.float64)
        lse = np.empty((B, H, N), dtype=np.float64)
    else:
        rows = np.asarray(rows, dtype=np.int64)
        if rows.shape[:2] != (B, H):
            raise ValueError("rows must be [B][H][R]")
        o = np.empty((B, H, rows.shape[2], d), dtype=np.float64)
        lse = np.empty((B, H, rows.shape[2]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            r = None if rows is None else rows[b, h]
            ob, lb = attention_head_rows(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :],
                                         scale, causal, r)
            if rows is None:
                o[b, :, h, :] = ob
                lse[b, h, :] = lb
            else:
                o[b, h] = ob
                lse[b, h] = lb
    return o, lse
