"""Plain CPU float64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP library
in ``exact_io_aware_online_amd`` never imports, links or calls it, and this
package imports nothing from there.

Every function here materialises the full score matrix, exactly what the
IO-aware method avoids, because that is the plainest way to write the
definition down (FlashAttention: Part 2, section 6.2 "FlashAttention
Summary": ordinary attention forms Q K^T as an N x N matrix).
"""

from . import fp8  # noqa: F401
from . import sdpa  # noqa: F401
from .sdpa import (  # noqa: F401
    kv_head_of,
    visible_mask,
    scores,
    softmax_rows,
    attention,
    attention_rows,
    decode,
    merge_partials,
    online_softmax_attention,
)
