"""CPU oracle for the NVFP4 decode / speculative-verify weight pass.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct definition that the HIP path is checked against.  Only the test
suite (``tests/``), ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it.  The product path (``verify_gemm_amd``)
never imports, calls or falls back to anything here, and nothing here
imports the product path: the two share no code.

Contents
--------
``nvfp4``   closed-form E2M1 / E4M3 / bf16 decoding, nibble unpacking,
            dequantisation and the fp64 GEMM with its acceptance bound.
``lmhead``  the lm_head pass: per-row argmax (lowest index on ties),
            top-2 gap against the bound (near-tie classification), the
            greedy accept-prefix length, tree verify and the sliced head's
            row-to-token map.
``fp8``     FP8 (E4M3) weights with tensor and per-row scales.

Every function is pinned by ``tests/test_oracle_*.py`` against values that
do not come from the oracle itself (exact rational brute force, library
decoders, hand-worked cases, invariants).  No function here is
"parity unpinned".
"""
from .nvfp4 import (  # noqa: F401
    bf16_bits_to_f64,
    dequant,
    e2m1_table,
    e2m1_value,
    e4m3_table,
    e4m3_value,
    nvfp4_gemm_ref,
    nvfp4_gemm_ref_entries,
    unpack_codes,
    tolerance_bound,
)
from .fp8 import fp8_dequant, fp8_gemm_ref  # noqa: F401
from .lmhead import (  # noqa: F401
    accept_len_ref,
    lmhead_ref,
    top2_merge,
)
