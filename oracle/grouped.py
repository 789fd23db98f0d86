"""Grouped-query and variable-length attention forward, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed
----------------
"FlashAttention 4: Atenção Mais Rápida e Eficiente em Memória para LLMs",
sections "Principais Conclusões" and "Compatibilidade e status atual", names
two forms of the same attention: grouped-query attention, where several query
heads share one key/value projection (multi-query attention when there is a
single one), and variable-length batches, where sequences of different
lengths are processed without padding.  Neither changes the arithmetic of
``attention.attention_forward``; each only chooses which keys a query row
sees, so both are written as that definition applied to the chosen keys:

  * grouped: query head h of H reads K/V head h // (H / Hkv); the K/V heads
    are repeated to H heads and the plain definition is applied;
  * variable-length: sequence b owns the packed token rows cu[b] .. cu[b+1]-1
    of every tensor and is its own attention problem (causal: its query i
    sees its keys 0..i).

Readings where the pages are silent: consecutive query heads share a K/V
head (h // (H / Hkv)), and the log-sum-exp of a packed batch is laid out
[H][total].
"""

import numpy as np

from .attention import attention_forward


def attention_forward_gqa(q, k, v, scale, causal, rows=None):
    """q: [B][N][H][d]; k, v: [B][N][Hkv][d] with H a multiple of Hkv.
    Returns (o, lse) shaped as by ``attention_forward``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    H, Hkv = q.shape[2], k.shape[2]
    if Hkv <= 0 or H % Hkv != 0 or k.shape != v.shape:
        raise ValueError("H must be a multiple of the K/V heads; k and v of one shape")
    g = H // Hkv
    return attention_forward(q, np.repeat(k, g, axis=2), np.repeat(v, g, axis=2), scale, causal,
                             rows)


def attention_forward_varlen(q, k, v, cu, scale, causal, rows=None):
    """Packed variable-length batch: q [total][H][d], k, v [total][Hkv][d],
    cu [B+1] token offsets.

    Without ``rows``: returns (o [total][H][d], lse [H][total]).  With
    ``rows`` (a list over sequences of int arrays [H][R_b] of row indices
    within the sequence): returns lists over sequences of o [H][R_b][d] and
    lse [H][R_b].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    cu = np.asarray(cu, dtype=np.int64)
    total, H, d = q.shape
    if rows is None:
        o = np.zeros((total, H, d), dtype=np.float64)
        lse = np.zeros((H, total), dtype=np.float64)
    else:
        o, lse = [], []
    for b in range(cu.shape[0] - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if rows is not None:
            r = np.asarray(rows[b], dtype=np.int64)
            if s1 == s0:
                o.append(np.zeros((H, 0, d)))
                lse.append(np.zeros((H, 0)))
                continue
            ob, lb = attention_forward_gqa(q[None, s0:s1], k[None, s0:s1], v[None, s0:s1], scale,
                                           causal, rows=r[None])
            o.append(ob[0])
            lse.append(lb[0])
        elif s1 > s0:
            ob, lb = attention_forward_gqa(q[None, s0:s1], k[None, s0:s1], v[None, s0:s1], scale,
                                           causal)
            o[s0:s1] = ob[0]
            lse[:, s0:s1] = lb[0]
    return o, lse
