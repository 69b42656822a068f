"""CPU oracle for the NVFP4 W4A4 mixture-of-experts expert path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check of the build entry
point and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code
with the GPU library (no kernels, headers, tables or helpers) and imports only
numpy and the Python standard library.

The oracle is deliberately plain and slow: every step is written out in the
order the method defines it, floating point is FP64 wherever the method does
not fix a precision, and the FP32 steps that decide an integer (a scale byte or
an FP4 code) are evaluated with a single correctly rounded FP32 operation each,
so that the GPU path can be required to match those integers bit for bit.

Sources.  The method is described on three web pages:

* "Low-Bit Precision Training Is Ready for Production: What Engineering Leaders
  Need to Know Before Adopting NVFP4" (vector-labs.ai) -- cited as
  *Low-Bit Precision Training*.
* "The 4-bitter Lesson: Balancing Stability and Performance in NVFP4 RL"
  (humans&) -- cited as *The 4-bitter Lesson*.
* "miniTE identifies and closes the execution gap in native NVFP4 reinforcement
  learning" (n884.com) -- cited as *miniTE news item*.

The element and scale formats the pages name (FP4 E2M1, FP8 E4M3) are defined
by the Open Compute Project specifications "OCP Microscaling Formats (MX) v1.0"
(FP4 E2M1 element type) and "OCP 8-bit Floating Point Specification (OFP8)"
(E4M3 with maximum 448, no infinities).

Modules
-------
formats   BF16, FP8 E4M3 and FP4 E2M1 encode/decode.
nvfp4     NVFP4 two-level block quantisation (rows and columns) and dequant.
moe       routing, permutation, grouped GEMMs, SwiGLU and the weighted combine.
pipeline  the whole expert-layer forward and backward with the GPU's storage
          roundings mirrored (for end-to-end reporting).
philox    the Philox4x64-10 counter-based generator (stochastic rounding).

Parity status: every function is pinned by tests under ``tests/`` against
closed forms, invariants, brute force or exact rational arithmetic.  The
``pipeline`` functions are pinned through their stages and by two whole-path
identities: the single-expert top-1 layer equals a dense W4A4 SwiGLU MLP, and
every gradient of the quantised backward is the adjoint of its forward GEMM on
the backward's own operands.  End to end, the GPU pipeline and the oracle
pipeline agree only statistically: after an intermediate tensor is re-quantised,
an FP32-versus-FP64 accumulation difference upstream can move an element across an
FP4 rounding boundary, so the GPU tests compare stage by stage, each stage fed the
GPU's own inputs, and gate the whole layer only loosely.
"""

from . import formats, philox, nvfp4, moe, pipeline  # noqa: F401
