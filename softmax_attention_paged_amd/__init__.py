"""MI355X-native fused softmax attention forward (prefill, paged decode with
split-KV + log-sum-exp merge) behind a C ABI; see include/attn.h.

The Python layer only marshals torch tensors into the C ABI. The HIP library
must be built in-tree first (python -m softmax_attention_paged_amd.build).
"""

from .api import (  # noqa: F401
    cache_append, decode_paged, decode_paged_noalloc, decode_params, decode_plan, default_scale, merge_lse,
    mla_kv_pack_fp8, prefill,
    prefill_workspace_size,
)
from ._ffi import AttnError, LIB_PATH, load  # noqa: F401
