"""CPU oracle for the fused affine-quantized matmul.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (``dequant_matmul_qmv_amd``) never imports it, and this package
imports nothing from the product path: the two share no code.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(hand-computed words and values, brute force with exact rationals on tiny
inputs, closed forms and special cases).  No function is "parity unpinned".
"""

from .qmv_oracle import (  # noqa: F401
    unpack_codes,
    widen_sb,
    widen_act,
    dequant_f64,
    matmul_ref,
    matmul_ref_rows,
    linear_ref,
    quantize_act_i8,
    matmul_ref_a8,
    dequant_ref_out,
    f32_to_bf16_bits,
)
