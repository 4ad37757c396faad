"""Plain CPU oracle for Jensen-bias-corrected attention over a quantized KV cache.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP library (no kernels, headers, helpers, tables or constants) and imports
nothing from it.

What it follows: *Quantized Keys Steal Attention: Bias Correction for KV-Cache
Compression in Video Diffusion* (Tuncer, Becker, Pfeil; arXiv 2605.26266). The
pages available are the abstract, §1 (with the captions of Figs. 1-3), §2 and
§3 (integer quantization, Eq. (1); quantization granularity; Hadamard
rotation). The paper's §4, where the correction is derived, is not among them;
the correction here is derived from the noise model stated in the Fig. 3
caption (uniform rounding noise on a score, exponentiated, biased upward by
convexity) and from the abstract's statement that the correction uses only the
step sizes of the cached keys and the query norm via a second-order Taylor
expansion. See ``correction.py`` for the derivation.

Precision: everything is float64 except the quantizer, which decides integer
codes and fp16 step sizes and therefore follows one fixed float32 operation
order (``quant.py``), the same order the kernel uses.

Modules
-------
hadamard    normalized Sylvester-Hadamard matrix and the float32 butterfly order
quant       asymmetric round-to-nearest quantizer, code layouts, dequantization
correction  Jensen-bias correction: second-order Taylor and exact forms
attention   chunk attention over [cached window ; current chunk], masses
"""
from . import hadamard, quant, correction, attention  # noqa: F401
from .attention import reference_call  # noqa: F401
