"""CPU oracle for the microscaling quantize + block-scaled GEMM path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

The oracle is plain, slow and written to be checked by eye against the pages
it follows. It shares no code with the HIP kernels, the C ABI or the Python
binding. Floating-point steps that the method performs in binary32 are done
with ``numpy.float32`` (IEEE-754, round-to-nearest-even, subnormals kept);
everything else is exact FP64 or integer arithmetic.

Sources (cited by page title and section in every module):
  * "Miles Blackwell RL Cambia la Uniformidad BF16 por MXFP8 y NVFP4 Nativos"
    (remio.ai) -- MXFP8 blocks, per-token NVFP4, bit-exact quantizer contract,
    rowwise/columnwise copies, joint gate/up scale.
  * "NVIDIA presenta una metodologia de preentrenamiento de 4 bits utilizando
    NVFP4" (7minutos.es) -- E2M1 value set, UE8M0 power-of-two scales, NVFP4
    two-level scaling, random Hadamard transform.
  * "Miles Blackwell MXFP8/NVFP4 RL recipes" (aib.vote) -- MXFP8 block of 32,
    NVFP4 block of 16 with E4M3 scale plus FP32 tensor/token scale, dequantized
    backward, DeepSeek-V3 expert arithmetic.

Functions with no pin against the pages are marked "parity unpinned" in their
docstring. Present ones:
  * the E8M0 exponent-selection rule (round-up reading) is held in place only by
    invariants and hand-worked closed forms, not by a value printed on a page;
  * the NVFP4 FP32 operation order and the choice to store the decode scale;
  * the blockwise-FP8 scale choice s = amax / 448 and its zero-block scale.
"""

from . import formats, mxfp8, nvfp4, gemm, moe, rng  # noqa: F401
from . import mxfp4  # noqa: F401,E402
from . import fp8_block  # noqa: F401,E402
