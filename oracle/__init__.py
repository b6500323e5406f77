"""CPU fp64 oracle for packed variable-length attention.

TEST INFRASTRUCTURE.  Only ``tests/``, the smoke check in ``__graft_entry__``
and the CPU-baseline leg of ``bench.py`` may import anything here.  The HIP
library and its Python binding never import this package, and this package
never imports them.
"""

from .attention import (  # noqa: F401
    backward,
    bias_grad,
    bias_tile,
    forward,
    head_backward,
    head_forward,
    head_logit_grad,
    head_probs,
    sequence_group_backward,
    sequence_head_forward,
    visible,
)
from .brute import brute_forward  # noqa: F401
from .kvcache import gather_pages, kvcache_forward  # noqa: F401
from .packing import pack_metadata, pad, unpad  # noqa: F401
