"""fp64 CPU oracle for GQA flash attention (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package. It shares no code with the HIP path.
"""

from .attention import (  # noqa: F401
    alibi_slopes,
    attention_ref,
    combine_ref,
    decode_paged_ref,
    kv_append_ref,
    paged_gather_ref,
    partial_attention_ref,
    to_f64,
    visible_mask,
)
from .fp8 import (  # noqa: F401
    dequantize_e4m3,
    e4m3_table,
    e4m3_value,
    kv_append_fp8_ref,
    quantize_e4m3,
)
