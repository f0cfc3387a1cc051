"""CPU oracle for the ggml-style MUL_MAT at LLM-decode shapes.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, and nowhere else.  It shares
no code with the HIP library (``quantized_skinny_gemm_amd``) and does not
import it; the two meet only in ``workloads.py``, which draws the seeded
inputs and holds none of the method's arithmetic.

What it computes (plain NumPy, float64 unless a step is fixed to fp32):

* ``codec``   -- Q4_0 and Q8_0 quantize / dequantize / decode, as the exact
  sequence of IEEE fp32 operations the readings below fix, plus the per-block
  integer dot products.
* ``mul_mat`` -- ``dst[M, N] = src1[M, K] . src0[N, K]^T`` for Q4_0, Q8_0, F16
  and F32 ``src0``, in float64.

Sources (page title, section):

* llama.cpp PR 1632 "mulmat tune", Introduction: the three MUL_MAT kinds
  (f32 x f32, f16 x f32, quantized x f32) and the INIT stage that prepares
  ``src1`` before COMPUTE.
* Arm China article on llama.cpp NUMA optimisation (Neoverse N2), section
  on the MulMat operator: ``src1`` is quantized into the ``wdata`` buffer and
  the product is ``dst = src0 * wdata``.
* The block formats themselves are not printed on any page (they are only
  named: "Q4_0, Q4_1, ..."; "llama3_Q4_0").  This library is specified
  against the ggml block layouts: Q4_0 = 32 values, fp16 scale
  ``d = (signed absmax) / -8``, ``q = clamp(floor(x / d + 8.5), 0, 15)``;
  Q8_0 = 32 values, ``d = absmax / 127``, ``q = round(x / d)``.

Readings taken where that definition leaves a step open (each one pinned by
a test in ``tests/test_oracle_*.py``):

R1  byte layout: Q4_0 block = fp16 ``d`` (little endian) then 16 bytes of
    nibbles; Q8_0 block = fp16 ``d`` then 32 int8.  Blocks run along K.
R2  nibble order: byte ``i`` holds element ``i`` in its low nibble and
    element ``i + 16`` in its high nibble.
R3  signed absmax: the first element (lowest index) with the strictly
    largest ``|x|``; the scan starts from ``+0``, so an all-zero block has
    ``max = +0`` and ``d = +0 / -8 = -0.0``.
R4  codes are computed from the fp32 ``d``; only storage rounds it to fp16.
R5  ``x / d`` is evaluated as ``x * (1 / d)``: one correctly rounded fp32
    reciprocal per block (``0`` when ``d == 0``), then one fp32 product.
R6  Q4_0: ``t = fl32(fl32(x * id) + 8.5)`` then ``floor`` and clamp to
    ``[0, 15]``; no fused multiply-add.
R7  Q8_0: ``round`` is round-half-away-from-zero applied to ``fl32(x * id)``.
R8  fp32 -> fp16 is IEEE round-to-nearest-even with subnormals kept.
R9  ``dst`` is overwritten (not accumulated into).
R10 Q8_0 weights (src0): the Q8_0 block of R1, quantized from f32 weights
    by the same routine as src1 (R5, R7, R8); each block dot is the sum of
    the products of the two signed 8-bit code sets (no offset), scaled by
    both fp16 scales.
"""

from . import codec, mul_mat  # noqa: F401
