"""fp64 CPU oracle for the attention forward pass and its gradients.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check of the
repository's graft entry point and by the benchmark's CPU-baseline leg, never
by the product path.  It shares no code with the HIP package.
"""
from .attention import (  # noqa: F401
    attention,
    visible_mask,
    block_summary,
    merge_summaries,
    finalize_summary,
    streamed_attention,
    split_attention,
    expand_kv_heads,
    varlen_attention,
)
from .backward import (  # noqa: F401
    attention_backward,
    grouped_attention_backward,
    kv_head_of,
    varlen_attention_backward,
)
from .dropout import (  # noqa: F401
    dropout_attention,
    dropout_attention_backward,
    dropout_keep,
    philox4x32_10,
)
