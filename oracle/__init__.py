"""CPU oracle for the SVDQuant W4A4 linear and the INT8 tensorwise W8A8 linear.

TEST INFRASTRUCTURE. Nothing in the product path imports, calls or links this
package. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it. It shares no code, table or helper with the HIP
library under ``bit_quantized_linear_amd/``; the two meet only through the
seeded input generators (``bit_quantized_linear_amd.workloads``), which hold
none of the method's arithmetic.

The oracle is plain numpy in float64 (float32 only where the method's own
rounding points say "round to fp32"). It is slow and meant to be read
against the pages:

* [HF-SVDQ]  "Hugging Face встроила Nunchaku в Diffusers: диффузия быстрее на
  30%, видеопамяти нужно до 50% меньше" (iitog.ru) -- the method paragraph
  ("Суть метода"): W4A4 main layers, activation outliers moved into the
  weights, the hardest part of each weight kept as a 16-bit low-rank branch,
  the remainder at 4 bits; the "Nunchaku Lite" paragraph: svdq_w4a4 layers
  for attention and MLP projections, INT4 variant.
* [KREA-SVDQ] "SVDQuant ускоряет Krea 2 вдвое даже на старых NVIDIA GPU --
  INT8/W4A4 вместо бесполезного FP8" (ainews.so) -- section "Решение: INT8 и
  W4A4": the INT8 tensorwise format and W4A4 + SVDQuant with low-rank
  branches that compensate quantization error without a calibration dataset.
* [DC-README] "Diffusion Compiler" README (CodeAlexx/diffusion-compiler) --
  the "Compiler" bullet listing the ``int4-group`` physical format.
* [HF-SVDQ] "Nunchaku Lite" paragraph, second layer type: awq_w4a16, 4-bit
  weights with 16-bit activations for normalization/modulation layers
  (``oracle/w4a16.py``); and the 4-bit float variant of svdq_w4a4, built as
  OCP MXFP4 (``oracle/mxfp4.py``).
* [HF-SVDQ] the same paragraphs: the MLP pair (up-projection, GELU,
  down-projection) with the down-projection's activation side produced from
  the up-projection's output (``oracle/mlp.py``).

Where the pages leave a step open, the reading taken is stated at the
function that takes it. Parity status of every function is listed in
``oracle/svdquant.py``, ``oracle/w8a8.py``, ``oracle/w4a16.py``,
``oracle/mxfp4.py`` and ``oracle/mlp.py`` headers.
"""

from . import mlp, mxfp4, svdquant, w4a16, w8a8  # noqa: F401
