"""CPU oracle for the weight-only quantized skinny GEMM.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library never does, and the
library shares no code with it.  Everything here is plain NumPy in float64:

  formats   E2M1 / E4M3FN decoders and encoders from their bit layouts
  quantize  the NVFP4 and 128x128-block FP8 quantization rules
  gemm      y = x . dequant(W) in float64, per-row argmax, error metrics,
            and the SwiGLU of a gate/up pair of projections
  speculative  greedy verification of a speculative-decoding round

Every function is pinned by the CPU tests (tests/test_oracle_*.py) against
tables, library routines, brute force and closed-form cases.
"""

from .formats import e2m1_decode, e4m3_decode, e2m1_encode, e4m3_encode, E2M1_MAX, E4M3_MAX
from .quantize import nvfp4_quantize, nvfp4_global_scale, fp8_quantize
from .speculative import verify_greedy
from .gemm import (nvfp4_unpack_codes, nvfp4_dequant_unscaled, nvfp4_gemm, fp8_dequant, fp8_gemm,
                   silu, nvfp4_swiglu, argmax_rows, compare)
