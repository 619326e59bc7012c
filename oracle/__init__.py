"""CPU oracle for exact scaled-dot-product attention (test infrastructure only).

This package is the slow, obviously-correct reference that the GPU kernels are
checked against. It is test infrastructure: only the test suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product library (``exact_io_aware_54_amd``) never imports or
calls anything here and shares no code with it.

Everything is float64 numpy. The score matrix S and the probability matrix P
are materialised (in full-row chunks when N is large), exactly as the
three-step "standard attention" the pages describe, never through the online
recurrence the kernels use.

Modules
-------
attention
    Forward (O and per-row logsumexp, also with fewer queries than keys) and
    backward (dQ, dK, dV) from the plain definition, and the merge of results
    over disjoint key sets. Pinned by tests/test_oracle.py and
    tests/test_oracle_splitkv.py.
online
    The blocked online-softmax recurrence of the pages' tiling algorithm, in
    both loop orders. Used only to pin the exactness of the oracle.
e4m3
    OCP FP8 E4M3 encode/decode written from the bit-level definition of the
    format. Pinned exhaustively over all 256 codes.

Every public function is pinned by a test that does not re-use its own
formula; there is no "parity unpinned" function in this package.
"""

from .attention import (  # noqa: F401
    scores,
    softmax_rows,
    attention_forward,
    attention_backward,
    attention_forward_rows,
    counted_flops,
    merge_partials,
)
from .e4m3 import e4m3_decode, e4m3_encode, E4M3_MAX  # noqa: F401
from .online import online_forward_kv_outer, online_forward_q_outer  # noqa: F401
