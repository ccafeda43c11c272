"""CPU oracle for fused exact attention — TEST INFRASTRUCTURE ONLY.

This package is the slow, obviously-correct float64 statement of what the
GPU path computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product library never
does, and this package imports nothing from the product (no shared kernels,
helpers, tables or constants).

Sources. Three web pages describe the method:

* [FA4-news] "FlashAttention-4: cómo Together AI aceleró la atención en GPU
  Blackwell" (news.hamidun.com).
* [FA3-wiki] "FlashAttention-3 (ES)" (systems-analysis.ru).
* [FA4-gist] "FlashAttention-4: Algorithm and Kernel Pipelining Co-Design for
  Asymmetric Hardware Scaling" (gist.science summary of arXiv 2603.05451).

Tiling and fusion are exact ([FA3-wiki] "FlashAttention y FlashAttention-2"),
the orthogonal rotation leaves Q·Kᵀ unchanged ([FA3-wiki] innovation 3) and
conditional rescaling only skips work ([FA4-gist] technical summary 2.B), so
the oracle is the plain definition written out: S = scale·Q·Kᵀ (optionally
causally masked), P = row-softmax(S), O = P·V ([FA4-news] "Por qué el enfoque
estándar ya no funciona"), with the per-row log-sum-exp and the standard
softmax gradient.

Modules
-------
attention   float64 forward / backward materialising S, P, dP, dS.
brute       pure-Python triple loops (no BLAS) for tiny shapes.
hadamard    Sylvester Hadamard matrix, fast Walsh–Hadamard transform,
            SplitMix64 sign vector, the random-sign rotation.
e4m3        OCP FP8 E4M3FN decode/encode (round-to-nearest-even, saturating).
fp8_model   diagnostic model of the fp8 forward: rotate, amax scales (per row
            for Q', per head for K' and V), quantise, dequantise, then the
            float64 attention.

Parity pins: every function here is checked by ``tests/test_oracle_*.py``
against closed forms, invariants, brute force or library routines.
"""

from .attention import (attention_forward, attention_backward,
                        attention_forward_rows, softmax_rows)
from .hadamard import (sylvester, fwht, splitmix64, rotation_signs, rotate)
from .e4m3 import (E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_values)
from .fp8_model import (quantize_per_head, quantize_per_block, quantize_per_block_pow2,
                        quantize_per_row_split, fp8_attention_model)

__all__ = [
    "attention_forward", "attention_backward", "attention_forward_rows",
    "softmax_rows", "sylvester", "fwht", "splitmix64", "rotation_signs",
    "rotate", "E4M3_MAX", "e4m3_decode", "e4m3_encode", "e4m3_values",
    "quantize_per_head", "quantize_per_block", "quantize_per_block_pow2",
    "quantize_per_row_split", "fp8_attention_model",
]
