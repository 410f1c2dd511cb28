"""CPU oracle for the backward of block-scaled low-precision linear and
grouped matmuls.

TEST INFRASTRUCTURE, not part of the library: a plain, slow, obviously
correct numpy implementation in fp64 of what the GPU path computes (format
decoding, MX re-quantization and the dX / dW contractions).  It shares no
code with the HIP library and imports nothing from it.  Only `tests/`, the
smoke check in `__graft_entry__.py` and the CPU-baseline leg of `bench.py`
may use it.

Pins (tests/test_oracle_*.py, all CPU):
* formats: exhaustive E4M3 / E8M0 tables against torch's CPU float8 dtypes,
  E2M1 against the OCP value list and the eight magnitudes of the FP4 page;
  bf16 rounding against torch's CPU cast; RNE-onto-grid against torch's E4M3
  cast below the saturation point and a brute-force nearest search.
* dequant: hand-built blocks with closed-form values for every format,
  including the NVFP4 two-level scale and partial 128x128 blocks.
* MX quant: scale-exponent invariant, idempotence, special blocks.
* GEMMs: pure-Python triple loops on tiny shapes, the ones-gradient closed
  forms of the FP8-adapter page's tests, grouped == per-group dense.
* forwards: triple loops (the NVFP4 forward over scalar-decoded operands),
  the FP8-adapter page's formulation on its grouped test shapes and on
  partial 128-blocks, and the adjoint identity that ties each forward's
  orientation to the backward's.
* per-tensor FP8 (pertensor.py): the E5M2 table against torch's
  float8_e5m2, quantization against torch's casts below saturation and a
  brute-force nearest search, the scale formula and ring update of the
  AstrAI page, triple-loop GEMMs with the scales applied to the sums.

Parity unpinned by the source documents: the E2M1 nibble order and the NVFP4
tensor-scale reading (see formats.py).
"""
from . import formats, gemm, pertensor  # noqa: F401
