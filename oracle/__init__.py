"""CPU oracle for exact scaled dot-product attention and its gradients.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this
package: only the test suite, the smoke check and the benchmark's CPU-baseline
leg call it.  It shares no code, tables or helpers with the HIP library.

Everything here is plain fp64 NumPy that materialises the score matrix S and
the probability matrix P one (sequence, head) at a time, i.e. the "standard
attention" the pages describe, written out from its definition.
"""

from .attention import (  # noqa: F401
    allowed_mask,
    attn_bwd,
    attn_bwd_sampled,
    attn_fwd,
    attn_fwd_rows,
    kv_head_of,
    probabilities,
    sequence_spans,
)
from .online_recurrence import online_attention  # noqa: F401
from .philox import drop_threshold, keep_mask, keep_scale, philox4x32_10  # noqa: F401
from . import fp8  # noqa: F401,E402
