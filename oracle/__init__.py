"""CPU oracle for symmetric round-to-nearest group quantization and the
weight-only dequantizing matmul.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test-suite (``tests/``), the smoke
check in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library (no kernels,
headers, helpers, tables or constants) and imports nothing from it.

The oracle is written from the definitions on the source pages, step by step
and without blocking, fusion or reordering, so that it can be checked by eye:

* ``rtn``     -- group absmax, fp32 scale, round-half-even codes, clip to
                 +-qmax, int8 bytes / int4 nibble packing, and unpacking
                 (page "量化推理：INT8/INT4 的体积、困惑度与速度为什么不同步",
                 script functions ``pack`` and ``unpack``; page "Huit bits,
                 puis quatre", section "Arrondir").
* ``gptq``    -- the calibration matrix H = sum x^T x, its damping, the
                 factor U of H^-1 = U^T U, and the column-by-column GPTQ
                 codes in the same payload / scale format (page "Huit bits,
                 puis quatre", section "Arrondir mieux : GPTQ").
* ``matmul``  -- the dequantizing products y = x . w_hat^T in fp64 and the
                 per-output error base sum |x . w_hat| used for tolerances
                 (page "Huit bits, puis quatre", section "Ranger des entiers
                 dans des f32", the QuantizedMatmul paragraph).

Every function is pinned by ``tests/test_oracle_pins.py`` against values the
pages print, closed forms, special cases and brute force on tiny inputs.
"""

from .rtn import (  # noqa: F401
    QMAX,
    quantize_pack,
    pack_codes,
    unpack,
    codes_from_payload,
    payload_bytes,
    num_scales,
    bits_per_weight,
)
from .matmul import (  # noqa: F401
    bf16_bits_to_f32,
    bf16_round,
    gemv_ref,
    gemm_ref,
    error_base,
)
from . import gptq  # noqa: F401,E402
