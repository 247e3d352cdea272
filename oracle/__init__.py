"""fp64 CPU oracle for fused softmax attention over dense and paged KV.

TEST INFRASTRUCTURE ONLY. The product path (the HIP library and its Python
binding) never imports, calls, links or executes anything in this package.
Only the tests, the smoke check and the benchmark's CPU-baseline leg use it.

It shares no code with the GPU path: it is written from the pages' statement
of the problem, in plain numpy float64, materialising every score matrix.
"""

from .attention import (  # noqa: F401
    NEG_INF,
    widen_bf16,
    widen_e4m3fn,
    widen,
    attention_rows,
    window_key_start,
    gather_paged_rows,
    decode_paged,
    decode_paged_rows,
    prefill_dense,
    prefill_dense_fp8,
    prefill_dense_fp8_rows,
    prefill_paged,
    prefill_paged_rows,
    merge_lse,
    online_softmax_blocks,
)
from .plan_examples import (  # noqa: F401
    decode_task_mapping,
    page_stack_counts,
    fold_factor,
    packed_query_tiles,
    mla_packed_workspace_bytes,
    static_anchor_tau,
)
from .cache import (  # noqa: F401
    E4M3_MAX,
    quantize_e4m3fn,
    cache_rows_view,
    cache_append,
    mla_kv_pack,
)
