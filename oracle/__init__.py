"""CPU oracle (test infrastructure only; see oracle/attention.py)."""
from .attention import (  # noqa: F401
    attention_backward_fp64,
    attention_bruteforce,
    attention_fp64,
    attention_online_fp64,
    attention_rows_fp64,
    attention_weights_fp64,
    merge_partials_fp64,
    score_matrix_bytes,
    score_matrix_gb,
)
from .fp8 import attention_fp8_fp64, dequantize_heads, e4m3_to_fp64  # noqa: F401
