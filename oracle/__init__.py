"""fp64 CPU oracle (test infrastructure only; see oracle.fp64, oracle.backward,
oracle.masks and oracle.monoids)."""
from .fp64 import (  # noqa: F401
    LOG2E,
    NEG_INF,
    attention,
    attention_base2,
    attention_selected_rows,
    block_state,
    combine,
    combine_partials,
    decode_partials,
    identity_state,
    inject,
    logsumexp_from_state,
    readout,
    safe_softmax_rows,
    split_bounds,
)
from .backward import (  # noqa: F401,E402
    attention_backward,
    attention_backward_dq_rows,
    attention_backward_row_block,
)
from .masks import attention_varlen, attention_window, visible  # noqa: F401,E402
from .monoids import (  # noqa: F401,E402
    log_sum_exp,
    moments,
    moments_scan,
    softmax_stats,
    softmax_stats_scan,
    variance,
)
