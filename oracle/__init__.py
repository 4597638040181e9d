"""CPU oracle (test infrastructure only; never imported by the product path)."""

from .attention import (  # noqa: F401
    attention,
    attention_rows,
    chunked_prefill,
    decode,
    gather_paged,
    kv_cache_write_expected,
    merge_lse,
    rope,
    round_bf16,
)
from .rmsnorm import residual_rms_norm  # noqa: F401
