"""CPU oracle for the tiled exact scaled-dot-product attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call,
link or execute anything in this package: only ``tests/``, the smoke check
in ``__graft_entry__.py`` and the ``cpu_baseline`` leg of ``bench.py`` use
it.  It shares no code with the HIP library (no kernels, headers, helpers,
tables or pre/post-processing); the only thing both sides consume is the
seeded input generator in ``workloads/``, which holds none of the method's
arithmetic.

Modules
-------
formats     bit-level decoding of bf16 and OCP FP8 E4M3 ("fn") inputs to fp64.
attention   the plain definition of softmax(Q K^T * scale) V and its per-row
            log-sum-exp, in fp64, materialising the score rows.
tiled       the online-softmax recurrence over key/value tiles (running row
            max m, running row sum l, output accumulator O) with an optional
            rescale threshold, in fp64; used to pin the oracle's "tiled equals
            untiled" exactness property and to count rescales.
brute       a pure-Python (math.fsum) evaluation of the definition for tiny
            inputs, independent of NumPy.
grouped     grouped-query (K/V heads shared by groups of query heads) and
            variable-length (packed sequences) forms of the definition.
backward    the gradients dQ, dK, dV of the definition (chain rule), and the
            row quantity D = sum(dO * O).
quantize    E4M3 encoding and per-(batch, head) quantisation of attention
            inputs with the optional random Hadamard rotation.
"""

from .formats import bf16_bits_to_float64, e4m3fn_bits_to_float64, dequantize_e4m3
from .attention import attention_forward, attention_head_rows
from .tiled import tiled_online_softmax_head, simulator_counts
from .brute import attention_brute
from .grouped import attention_forward_gqa, attention_forward_varlen
from .backward import attention_backward, attention_backward_head, attention_delta
from .quantize import e4m3fn_encode, fwht32, hadamard, quantize_e4m3

__all__ = [
    "bf16_bits_to_float64",
    "e4m3fn_bits_to_float64",
    "dequantize_e4m3",
    "attention_forward",
    "attention_head_rows",
    "tiled_online_softmax_head",
    "simulator_counts",
    "attention_brute",
    "attention_forward_gqa",
    "attention_forward_varlen",
    "attention_backward",
    "attention_backward_head",
    "attention_delta",
    "e4m3fn_encode",
    "fwht32",
    "hadamard",
    "quantize_e4m3",
]
