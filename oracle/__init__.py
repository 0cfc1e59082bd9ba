"""CPU oracle for the paged-KV attention forward and backward.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
package.  The library (``invariant_paged_kv_amd``) never imports it, and it
never imports the library: the two share no code.  Both are fed by the seeded
generators in ``pkv_inputs``, which hold none of the method's arithmetic.

The oracle is plain NumPy in float64.  It computes the mathematical definition
of the operation, with no blocking, chunking, online softmax or fixed-order
merging: those are how the GPU path reaches the same result, not what the
result is.

Pins (see ``tests/test_oracle.py``): every function here is checked against
something other than itself -- a pure-Python ``decimal`` brute force over a
nested-list pool, PyTorch's own float64 scaled-dot-product attention, closed
forms, and the invariances the pages state; the backward against PyTorch's
float64 autograd, central finite differences of the forward, and the
gradient identities of softmax (``tests/test_oracle_backward.py``).  No function in this package is
"parity unpinned".
"""

from .paged_kv import (  # noqa: F401
    Layout,
    attention,
    attention_chunks,
    bf16_bits_to_f64,
    cache_write,
    fp8e4m3_bits_to_f64,
    gather_kv,
    gather_sequence,
    masked_softmax,
    scores,
    row_positions,
    visible_keys,
)
from .backward import (  # noqa: F401
    attention_backward,
    attention_backward_bound,
    cu_seqlens_k_of,
)
