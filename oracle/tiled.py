"""Online-softmax recurrence over key/value tiles, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the second, tiled route to the attention result, used to pin the
oracle (the two must agree to rounding) and to count how often the output
accumulator is rescaled.  It follows the recurrence of the Python simulator
in the dev.to page "FlashAttention-4 em Blackwell B200", section 4
("Implementação Completa em Python: Simulador do Algoritmo de Tiling e Online
Softmax"): for each block of query rows, running statistics m (row maximum,
initialised to -inf) and l (row sum, initialised to 0) and an output tile O
(initialised to 0) are carried across the key/value tiles; each tile's score
block is scale * Q K^T; when the running maximum moves from m_old to m_new the
earlier sum and output are multiplied by exp(m_old - m_new).

Two departures from the simulator, each a reading of the pages:
  * normalisation is deferred: O holds sum_j exp(s_ij - m_i) v_j and is divided
    by l once at the end (the simulator divides every step; same value);
  * the rescale is threshold-gated as described in "FlashAttention 4: Atenção
    Mais Rápida e Eficiente em Memória para LLMs", section "Reescalonamento
    Softmax Online Mais Inteligente": the reference maximum is only moved when
    a tile's row maximum exceeds it by more than ``tau`` (natural-log units).
    Between moves the exponentials exp(s - m_ref) may exceed 1 (by at most
    e^tau); the final result is unchanged in exact arithmetic.
  * the key tail is masked instead of truncated, and causal tiles that lie
    wholly above the diagonal are skipped (never visited); the others are
    masked element by element (key j visible to query i iff j <= i).
"""

import math

import numpy as np


def tiled_online_softmax_head(q, k, v, scale, causal, block_q, block_k, tau=0.0):
    """One head, q/k/v float64 [N][d].  Returns (o [N][d], lse [N], stats).

    ``tau`` = 0 rescales whenever a row maximum grows (the simulator's rule);
    ``tau`` = math.inf never moves a finite reference maximum.
    ``stats`` counts visited tiles, the simulator's QK^T flop count
    (2 * rows * cols * d per visited tile), and rescale events (a row whose
    finite reference maximum was moved).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    nk = k.shape[0]
    o_out = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse_out = np.zeros(n, dtype=np.float64)
    stats = {"q_blocks": 0, "kv_blocks": -(-nk // block_k), "tiles": 0,
             "qk_flops": 0, "rescales": 0, "row_tiles": 0}
    for q0 in range(0, n, block_q):
        qi = np.arange(q0, min(q0 + block_q, n))
        stats["q_blocks"] += 1
        m = np.full(qi.shape[0], -np.inf)                   # running max (reference)
        l = np.zeros(qi.shape[0])                           # running sum
        acc = np.zeros((qi.shape[0], v.shape[1]))           # unnormalised O
        for k0 in range(0, nk, block_k):
            kj = np.arange(k0, min(k0 + block_k, nk))
            if causal and kj[0] > qi[-1]:
                continue                                    # tile wholly above the diagonal
            stats["tiles"] += 1
            stats["qk_flops"] += 2 * block_q * block_k * d
            s = scale * np.matmul(q[qi], k[kj].T)           # score tile
            if causal:
                s = np.where(kj[None, :] <= qi[:, None], s, -np.inf)
            m_tile = s.max(axis=1)
            # the first finite maximum always becomes the reference; later
            # ones only when they exceed it by more than tau
            m_fin = np.where(np.isfinite(m), m, 0.0)
            move = (m_tile > m) & (~np.isfinite(m) | (m_tile > m_fin + tau))
            stats["rescales"] += int(np.sum(move & np.isfinite(m)))
            stats["row_tiles"] += qi.shape[0]
            m_new = np.where(move, m_tile, m)
            # exp(m_old - m_new) with exp(-inf - finite) = 0 on the first move
            alpha = np.where(move, np.exp(np.where(np.isfinite(m), m - m_new, -np.inf)), 1.0)
            l = l * alpha
            acc = acc * alpha[:, None]
            m_safe = np.where(np.isfinite(m_new), m_new, 0.0)
            p = np.exp(s - m_safe[:, None])
            p = np.where(np.isfinite(m_new)[:, None], p, 0.0)
            l = l + p.sum(axis=1)
            acc = acc + np.matmul(p, v[kj])
            m = m_new
        empty = l == 0.0
        o_out[qi] = acc / np.where(empty, 1.0, l)[:, None]
        lse_out[qi] = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
    return o_out, lse_out, stats


def simulator_counts(seq_len, block_size, d_model):
    """The three counters the dev.to simulator reports, obtained by running
    the tiled model above (non-causal, square blocks) on zero-valued tiles of
    the simulator's shape: number of blocks along the sequence, its QK^T flop
    count, and the size in MiB of an N x N 2-byte score matrix that tiling
    keeps out of HBM (rounded to 3 decimals, as the page prints it)."""
    z = np.zeros((seq_len, d_model))
    _, _, st = tiled_online_softmax_head(z, z, z, 1.0 / math.sqrt(d_model), False,
                                         block_size, block_size)
    return {
        "num_blocks": st["kv_blocks"],
        "total_flops_simulated": st["qk_flops"],
        "hbm_traffic_eliminated_mb": round(seq_len * seq_len * 2 / (1024 * 1024), 3),
    }
