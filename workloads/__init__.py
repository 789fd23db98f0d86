"""Seeded synthetic inputs for the attention forward.

This module is shared by the tests, the benchmark and the smoke check.  It
only draws and encodes inputs; it holds none of the attention arithmetic.  The
CPU oracle and the HIP library both receive exactly the arrays made here
(the oracle decodes them itself, the library gets device copies).

Workloads (shape B, H, N, d; data; mode):
  tiny      1, 2, 128, 64      bf16 N(0,1)                      non-causal and causal
  mha2k     4, 16, 2048, 128   bf16 N(0,1)                      non-causal and causal
  long8k    2, 16, 8192, 128   bf16 N(0,1)                      causal
  long8k64  2, 32, 8192, 64    bf16 N(0,1)                      causal
  ctx32k    1, 32, 32768, 128  bf16 N(0,1), 1% of K rows x8     causal
  fp8_8k    2, 16, 8192, 128   OCP e4m3 from N(0,1) with 0.1%
                               outliers x20, per-(b,h) descale  non-causal
  gqa8k     2, 32/8, 8192, 128 bf16 N(0,1); 32 query heads over
                               8 K/V heads                      causal
  varlen    8 sequences, 16/4 heads, d 128, bf16 N(0,1); packed
            lengths drawn in [2, 8192] with the first fixed at
            8192 and the second at 1 (about 33k tokens)         causal
The scale is 1/sqrt(d) everywhere.  Grouped-query workloads give K and V
Hkv heads ([B][N][Hkv][d]); variable-length workloads pack their sequences
along the token axis ([total][heads][d], offsets in "cu").

Recipe (all draws on the CPU with torch.Generator, so the same seed gives the
same bytes on every machine running this torch build):
  * seed = 1000 * workload_id + tensor_id, tensor ids Q=0, K=1, V=2,
    peaked K rows=3, outlier positions=4 (+ the tensor id * 10), row sample=5,
    sequence lengths=6, rotation signs=7, upstream gradient=9;
  * values: float32 standard normal, laid out [B][N][H][d];
  * ctx32k: per (b, h), round(0.01 * N) distinct key rows are multiplied by 8
    in float32 (a peaked softmax that exercises the rescale);
  * bf16: float32 -> bfloat16 round-to-nearest-even (torch's conversion);
  * outliers (fp8_8k, and its bf16 source for the quantiser): per tensor,
    round(0.001 * numel) distinct elements are multiplied by 20 in float32;
  * fp8: the outliers as above; then per (b, h): descale = amax / 448 and code = e4m3fn(x / descale)
    round-to-nearest-even (torch's float8_e4m3fn conversion, after a clamp
    to +-448 so rounding noise cannot overflow);
  * sampled rows (large workloads): per (b, h), rows 0 and N-1 plus 510
    distinct rows drawn uniformly from 1..N-2.
"""

import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "bf16" or "fp8"
    modes: tuple          # causal flags to run
    peaked_k: bool = False
    outliers: bool = False
    Hkv: int = 0          # K/V heads; 0: same as H
    lengths: tuple = ()   # variable-length batch: the sequence lengths (B = len, N = max)

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.d)

    @property
    def kv_heads(self):
        return self.Hkv or self.H

    @property
    def varlen(self):
        return bool(self.lengths)

    @property
    def total(self):
        return sum(self.lengths) if self.lengths else self.B * self.N

    def flops(self, causal):
        """4*B*H*N^2*d, halved when causal (the metric's convention); for a
        variable-length batch the sum of 4*H*n^2*d over its sequences."""
        if self.lengths:
            f = sum(4.0 * self.H * n * n * self.d for n in self.lengths)
        else:
            f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if causal else f


def varlen_lengths(wid, count, max_len):
    """Seeded sequence lengths for a variable-length workload: the first is
    max_len, the second 1, the rest uniform in [2, max_len]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * wid + 6)
    rest = torch.randint(2, max_len + 1, (count - 2,), generator=g).tolist()
    return tuple([max_len, 1] + rest)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 2, 128, 64, "bf16", (False, True)),
    "mha2k": Workload("mha2k", 2, 4, 16, 2048, 128, "bf16", (False, True)),
    "long8k": Workload("long8k", 3, 2, 16, 8192, 128, "bf16", (True,)),
    "long8k64": Workload("long8k64", 6, 2, 32, 8192, 64, "bf16", (True,)),
    "ctx32k": Workload("ctx32k", 4, 1, 32, 32768, 128, "bf16", (True,), peaked_k=True),
    "fp8_8k": Workload("fp8_8k", 5, 2, 16, 8192, 128, "fp8", (False,), outliers=True),
    "gqa8k": Workload("gqa8k", 7, 2, 32, 8192, 128, "bf16", (True,), Hkv=8),
}
_VL = varlen_lengths(8, 8, 8192)
WORKLOADS["varlen"] = Workload("varlen", 8, len(_VL), 16, max(_VL), 128, "bf16", (True,), Hkv=4,
                               lengths=_VL)

SAMPLE_ROWS = 512
E4M3_MAX = 448.0


def seed_for(wid, tensor_id):
    return 1000 * wid + tensor_id


def _randn(shape, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def _perm_prefix(n, count, seed):
    """``count`` distinct integers from range(n), seeded."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    if n <= 1 << 24:
        return torch.randperm(n, generator=g)[:count]
    # large n: rejection-free draw of distinct values by oversampling
    out = torch.empty(0, dtype=torch.int64)
    while out.numel() < count:
        cand = torch.randint(0, n, (2 * count,), generator=g)
        out = torch.unique(torch.cat([out, cand]))  # sorted, distinct
    # choose a seeded subset of exactly ``count`` of them
    return out[torch.randperm(out.numel(), generator=g)[:count]]


def bf16_bits(t):
    """float32 torch tensor -> numpy uint16 bit patterns of its bf16 rounding."""
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def cu_seqlens(lengths):
    """int32 offsets [B+1] of packed sequences."""
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _shapes(w, shape):
    """(B, N, H, d) and the per-tensor array shapes: [B][N][heads][d], or
    [1][total][heads][d] for a variable-length workload."""
    B, N, H, d = shape if shape is not None else (w.B, w.N, w.H, w.d)
    Hkv = w.Hkv or H
    if w.lengths:
        T = sum(w.lengths)
        return (B, N, H, d), {"q": (1, T, H, d), "k": (1, T, Hkv, d), "v": (1, T, Hkv, d)}
    return (B, N, H, d), {"q": (B, N, H, d), "k": (B, N, Hkv, d), "v": (B, N, Hkv, d)}


def _peak_rows(w, x, N):
    """Multiplies round(0.01 N) distinct key rows of every (b, K/V head) by 8."""
    Bx, _, Hx, _ = x.shape
    npk = int(round(0.01 * N))
    for b in range(Bx):
        for h in range(Hx):
            rows = _perm_prefix(N, npk, seed_for(w.wid, 3) * 7919 + b * Hx + h)
            x[b, rows, h, :] *= 8.0


def make_bf16(w, shape=None):
    """Q, K, V for a bf16 workload as uint16 bf16 bit arrays (shapes as in
    ``_shapes``), plus "cu" offsets for a variable-length workload."""
    (B, N, H, d), shp = _shapes(w, shape)
    out = {}
    for tid, name in enumerate(("q", "k", "v")):
        x = _randn(shp[name], seed_for(w.wid, tid))
        if name == "k" and w.peaked_k:
            _peak_rows(w, x, N)
        if w.outliers:
            _outliers(w, x, tid)
        out[name] = bf16_bits(x)
    if w.lengths:
        out["cu"] = cu_seqlens(w.lengths)
    return out


def _outliers(w, x, tid):
    """Multiplies round(0.001 * numel) distinct elements of x by 20."""
    n_out = int(round(0.001 * x.numel()))
    idx = _perm_prefix(x.numel(), n_out, seed_for(w.wid, 4) + 10 * tid)
    flat = x.view(-1)
    flat[idx] *= 20.0


def _quantize(x, descale_of):
    y = (x / descale_of).clamp(-E4M3_MAX, E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_fp8(w, shape=None):
    """Q, K, V for an fp8 workload: uint8 e4m3fn codes (shapes as in
    ``_shapes``) and float32 descales [B][heads] per tensor (per sequence for
    a variable-length workload), plus "cu" offsets when variable-length."""
    (B, N, H, d), shp = _shapes(w, shape)
    out = {}
    for tid, name in enumerate(("q", "k", "v")):
        x = _randn(shp[name], seed_for(w.wid, tid))
        if w.outliers:
            _outliers(w, x, tid)
        if w.lengths:
            cu = cu_seqlens(w.lengths)
            nh = x.shape[2]
            descale = torch.empty((len(w.lengths), nh), dtype=torch.float32)
            codes = np.empty(x.shape, dtype=np.uint8)
            for b in range(len(w.lengths)):
                seg = x[:, cu[b]:cu[b + 1]]
                amax = seg.abs().amax(dim=(0, 1, 3)) if seg.shape[1] else torch.zeros(nh)
                descale[b] = torch.clamp(amax, min=1e-30) / E4M3_MAX
                codes[:, cu[b]:cu[b + 1]] = _quantize(seg, descale[b][None, None, :, None])
            out[name] = codes
            out["d" + name] = descale.numpy()
        else:
            amax = x.abs().amax(dim=(1, 3))                       # [B][heads]
            descale = torch.clamp(amax, min=1e-30) / E4M3_MAX
            out[name] = _quantize(x, descale[:, None, :, None])
            out["d" + name] = descale.to(torch.float32).numpy()
    if w.lengths:
        out["cu"] = cu_seqlens(w.lengths)
    return out


def make_dout(w, shape=None):
    """Upstream gradient dO for a backward pass: bf16 bits of N(0,1),
    shaped like Q ([B][N][H][d]), seed tensor id 9."""
    (B, N, H, d), shp = _shapes(w, shape)
    return bf16_bits(_randn(shp["q"], seed_for(w.wid, 9)))


def rotation_signs(w):
    """Random signs s for the Hadamard rotation diag(s) H_d / sqrt(d):
    (float64 +-1 [d], uint32 [d/32] with bit i set where s_i = -1),
    seed tensor id 7."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(w.wid, 7))
    neg = (torch.randint(0, 2, (w.d,), generator=g) == 1).numpy()
    words = np.zeros(w.d // 32, dtype=np.uint32)
    for i in np.nonzero(neg)[0]:
        words[i // 32] |= np.uint32(1) << np.uint32(i % 32)
    return np.where(neg, -1.0, 1.0), words


def make_inputs(w, shape=None):
    return make_fp8(w, shape) if w.dtype == "fp8" else make_bf16(w, shape)


def sample_rows(w, count=SAMPLE_ROWS, N=None):
    """Per-(b, h) query rows to check: all rows when N <= count, else rows 0
    and N-1 plus ``count - 2`` distinct seeded rows.  Returns int64 [B][H][R]."""
    N = w.N if N is None else N
    if N <= count:
        return np.broadcast_to(np.arange(N, dtype=np.int64), (w.B, w.H, N)).copy()
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_for(w.wid, 5))
    rows = np.empty((w.B, w.H, count), dtype=np.int64)
    for b in range(w.B):
        for h in range(w.H):
            mid = torch.randperm(N - 2, generator=g)[:count - 2].numpy() + 1
            rows[b, h] = np.concatenate([[0, N - 1], np.sort(mid)])
    return rows
