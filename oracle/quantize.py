"""E4M3 quantisation of attention inputs, with the optional random Hadamard
rotation, in the precision the decisions are taken in.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed
----------------
"FlashAttention-3: Pipeline Assíncrono com Warp Specialization, WGMMA e FP8
no Hopper e Blackwell", section "Estabilidade em FP8: Algoritmo de 2 Passos
e Incoherent Processing", gives two defences for E4M3 (range +-448); the
second ("incoherent processing") multiplies the operands by random
orthogonal Hadamard matrices H_d so that a few large-magnitude outliers are
spread over all dimensions instead of saturating the format.  For attention
the rotation is applied to the rows of Q and K: with M orthogonal,
(Q M)(K M)^T = Q K^T, so the scores are unchanged while each rotated row has
a flatter magnitude profile.

Readings where the page is silent:
  * M = diag(s) H_d / sqrt(d): s a vector of random signs (an input: the
    caller draws it, so both sides see the same one), H_d the Sylvester
    Hadamard matrix, H[i][j] = (-1)^popcount(i & j); V is not rotated;
  * quantisation per (batch, head) as the FP8 entry point expects:
    descale = amax / 448, code = e4m3(x / descale), round to nearest even,
    clamped to +-448; with the rotation the returned descale is the one of
    x diag(s) H_d divided by sqrt(d), so that code * descale approximates
    x M;
  * a code is an integer decided by floating point, so the oracle takes the
    decision in the precision the kernel takes it in, binary32: the
    transform is the fast Walsh-Hadamard butterfly (strides 1, 2, 4, ...,
    d/2; a pair (a, b) becomes (a + b, a - b)) in binary32, then the
    maximum, descale = fl(amax / 448), v = fl(y / descale), the clamp and
    the rounding onto the E4M3 grid.
"""

import math

import numpy as np

E4M3_MAX = 448.0


def e4m3fn_encode(x):
    """float64 values -> OCP E4M3 (fn) codes, round to nearest even on the
    format's grid, saturating at +-448; NaN -> 0x7F.  Built from the format
    definition (exponent bias 7, 3 mantissa bits, subnormals m/8 * 2^-6)."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    a = np.minimum(np.abs(np.where(np.isnan(x), 0.0, x)), E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.uint8)
    sub = a < 2.0 ** -6
    # subnormals (and the rounding up into the smallest normal): m = a / 2^-9
    m_sub = np.rint(np.where(sub, a, 0.0) / 2.0 ** -9).astype(np.int64)    # 0..8
    code = np.where(sub, m_sub.astype(np.uint8), code)                       # m = 8 is 0x08 = 2^-6
    # normals: a = f 2^k, f in [0.5, 1): exponent e = k - 1, quantum 2^(e - 3)
    f, k = np.frexp(np.where(sub, 1.0, a))
    e = k.astype(np.int64) - 1
    q = np.rint(np.where(sub, 8.0, a) / np.ldexp(1.0, (e - 3).astype(np.int32)))  # 8..16
    up = q >= 16
    e = np.where(up, e + 1, e)
    q = np.where(up, 8.0, q)
    normal = (((e + 7) << 3) | (q.astype(np.int64) - 8)).astype(np.uint8)
    code = np.where(sub, code, normal)
    code = code | sign
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def hadamard(d):
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1."""
    i = np.arange(d)
    bits = np.bitwise_and(i[:, None], i[None, :])
    pop = np.zeros(bits.shape, dtype=np.int64)
    while bits.any():
        pop += bits & 1
        bits = bits >> 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def fwht32(y):
    """y @ H_d along the last axis by the iterative fast Walsh-Hadamard
    butterfly, every addition rounded to binary32."""
    y = np.asarray(y, dtype=np.float32)
    d = y.shape[-1]
    h = 1
    while h < d:
        z = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = z[..., 0, :], z[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(y.shape)
        h *= 2
    return y


def quantize_e4m3(x, signs=None):
    """x: float64 [B][N][H][d] holding binary32-exact values (bf16 inputs).
    signs: None (no rotation) or +-1 array [d].  Returns (codes uint8
    [B][N][H][d], descale float32 [B][H])."""
    x = np.asarray(x, dtype=np.float64)
    B, N, H, d = x.shape
    y = x.astype(np.float32)
    if signs is not None:
        y = y * np.asarray(signs, dtype=np.float32)           # exact
        y = fwht32(y)
    codes = np.empty(x.shape, dtype=np.uint8)
    descale = np.empty((B, H), dtype=np.float32)
    inv_sqrt_d = np.float32(1.0 / math.sqrt(d))
    for b in range(B):
        for h in range(H):
            yh = y[b, :, h, :]
            amax = np.float32(np.abs(yh).max()) if yh.size else np.float32(0.0)
            ds = np.float32(amax / np.float32(E4M3_MAX))
            div = ds if ds > 0 else np.float32(1.0)
            v = (yh / div).astype(np.float32)
            v = np.clip(v, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
            codes[b, :, h, :] = e4m3fn_encode(v.astype(np.float64))
            descale[b, h] = np.float32(ds * inv_sqrt_d) if signs is not None else ds
    return codes, descale
