"""fp64 CPU oracle for exact attention — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the HIP library.
"""

from .attention import (  # noqa: F401
    attention_bwd,
    attention_bwd_head,
    attention_bwd_rows,
    attention_decode_head,
    attention_fwd,
    attention_fwd_head,
    causal_tiles_visited,
    tiled_fwd_fa1_head,
    tiled_fwd_head,
    visible,
)
from .dropout import (  # noqa: F401,E402
    attention_bwd_dropout_head,
    attention_dq_dropout_rows,
    attention_fwd_dropout_head,
    dropout_bytes,
    dropout_keep,
    dropout_threshold,
    philox4x32_10,
)
