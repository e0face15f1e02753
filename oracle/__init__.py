"""fp64 CPU oracle (test infrastructure only; never called by the library)."""
from .pp_oracle import (  # noqa: F401
    attend,
    doc_prefix_len,
    oracle_decode,
    tail_lists,
    to_f64,
    visible_slots,
)
from .pp_step_oracle import (  # noqa: F401
    oracle_append_step,
    rope,
    round_bf16,
    shared_positions,
)
from .pp_prefill_oracle import oracle_prefill, prefill_visible  # noqa: F401
