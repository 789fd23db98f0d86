"""Bit-level decoders for the input formats the attention path consumes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the formats but do not define their encodings:
  * bf16 inputs follow the usage example in "FlashAttention-3: Pipeline
    Assíncrono com Warp Specialization, WGMMA e FP8 no Hopper e Blackwell",
    section "Implementando FlashAttention-3 em produção" (bfloat16 Q/K/V).
  * FP8 E4M3 is described in the same page, section "Estabilidade em FP8:
    Algoritmo de 2 Passos e Incoherent Processing": 1 sign bit, 4 exponent
    bits, 3 mantissa bits, dynamic range +-448.

The decoders below follow the public format definitions:
  * bfloat16 is the upper 16 bits of an IEEE-754 binary32 word.
  * OCP FP8 E4M3 ("fn" variant, the one whose largest finite value is 448):
    exponent bias 7; exponent field 0 encodes subnormals m/8 * 2^-6; the
    pattern S.1111.111 is NaN; there are no infinities.
Everything is decoded to float64 so that the oracle sees exactly the values
the GPU receives.
"""

import numpy as np


def bf16_bits_to_float64(bits):
    """Decode bfloat16 bit patterns (uint16 array) to float64, exactly."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError("bf16 bits must be a uint16 array, got %s" % b.dtype)
    word = b.astype(np.uint32) << np.uint32(16)
    return word.view(np.float32).astype(np.float64)


def e4m3fn_bits_to_float64(bits):
    """Decode OCP FP8 E4M3 (fn) bit patterns (uint8 array) to float64.

    Built from the format fields, not from a library conversion: value =
    (-1)^s * 2^(e-7) * (1 + m/8) for e in 1..15 (except e=15, m=7 = NaN), and
    (-1)^s * 2^-6 * (m/8) for e = 0.
    """
    b = np.asarray(bits)
    if b.dtype != np.uint8:
        raise TypeError("e4m3 bits must be a uint8 array, got %s" % b.dtype)
    s = (b >> 7).astype(np.int64)
    e = ((b >> 3) & 0xF).astype(np.int64)
    m = (b & 0x7).astype(np.float64)
    sign = np.where(s == 1, -1.0, 1.0)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    subnormal = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, subnormal, normal)
    nan = (e == 15) & ((b & 0x7) == 7)
    return np.where(nan, np.nan, out)


def dequantize_e4m3(codes, descale):
    """x = e4m3_value(code) * descale[b, h], in float64.

    ``codes`` is uint8 [B][N][H][d]; ``descale`` is float [B][H] (one factor
    per batch and head, the FP8 entry point's convention).  The product of an
    e4m3 value and an fp32 descale is exact in float64.
    """
    c = np.asarray(codes)
    ds = np.asarray(descale, dtype=np.float64)
    if c.ndim != 4:
        raise ValueError("codes must be [B][N][H][d]")
    B, N, H, d = c.shape
    if ds.shape != (B, H):
        raise ValueError("descale must be [B][H]")
    return e4m3fn_bits_to_float64(c) * ds[:, None, :, None]
