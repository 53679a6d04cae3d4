"""CPU oracle for the q4_K x q8_1 quantized matrix multiply (MMQ), its q6_K variant and its
f16 comparator.

TEST INFRASTRUCTURE ONLY. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here. The HIP
path (``q4_q8_int8_amd``) never imports this package and this package never
imports it; the two share no code, headers, tables or constants.

Every function is a plain, slow, readable restatement of what the pages define
(see the docstrings for the page and section each step follows). Floating-point
results are computed in float64 except where the pages fix the precision (the
q8_1 scale and quantization steps are float32, the stored scale is float16).
"""
from .mmq_oracle import (  # noqa: F401
    QK8, QK_K, Q4K_BLOCK_BYTES,
    Q8, Q4K,
    f16_encode, f16_decode, round_half_away,
    quantize_q8_1,
    decode_q4_K, q4_K_scales, dequantize_q4_K,
    mmq, block_dots, mmq_terms,
)
from .f16_oracle import convert_f32_f16, dequantize_q4_K_f16, gemm_f16  # noqa: F401
from .q6k_oracle import (  # noqa: F401
    Q6K, Q6K_BLOCK_BYTES, decode_q6_K, q6_K_scales, dequantize_q6_K,
    mmq_q6K, block_dots_q6K, mmq_q6K_terms, mmq_q6K_fold_terms,
)
