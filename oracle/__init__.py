"""CPU oracle for draft-tree verification (test infrastructure only).

A plain, slow, float64 numpy statement of what the verify step computes. Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it; the HIP library and
its binding never do, and this package imports nothing from them.
"""

from .kvquant import (  # noqa: F401
    dequantize_kv,
    dequantize_kv_mx4,
    e2m1_decode,
    e2m1_encode,
    e4m3_decode,
    e4m3_encode,
    mx4_block_exponent,
    mx4_block_exponents,
    quantize_kv,
    quantize_kv_mx4,
    row_scale_exponent,
)
from .sampling import philox4x32_10, sample_accept, sample_rows, uniforms  # noqa: F401
from .tree_verify import (  # noqa: F401
    accept,
    anc_bitmask_words,
    argmax_rows,
    bf16_bits_to_f64,
    kv_commit,
    tree_attention,
    tree_structure,
    validate_parent,
    verify,
    visibility_mask,
)
