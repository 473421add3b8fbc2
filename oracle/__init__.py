"""CPU oracle for large-beam Gated DeltaNet decoding.

TEST INFRASTRUCTURE, not part of the product.  Only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may import, call or
execute anything here.  The HIP path never routes through it.

A plain, slow FullState implementation in float64: every beam materialises
its d_v x d_k state by eq. (4) of the OneLA reading note, states are copied
when beams are re-parented, and scoring, selection and ancestry are done by
brute force (full sort).  It imports nothing from the GPU package; both sides
share only the seeded input generators in synth/.

Parity status: every function here is pinned by tests/test_oracle_*.py:
exact-arithmetic identities and brute force (eqs. 3-9), closed forms, library
routines (scipy's log-softmax, a full sort), walks of the parent pointers (SID
prefixes, cumulative scores) and explicit per-value-head loops (grouped heads).
tests/test_oracle_mutations.py plants plausible mistakes in a copy of this
package and checks that a pin fails for each.  No function is "parity unpinned".
"""
from .gdn import gdn_token, prefill, rank1_transition  # noqa: F401
from .beam import (FullStateDecoder, ancestry_update, capacity_elements,  # noqa: F401
                   log_softmax_rows, step_scores, top_w)
from .run import decode_request, prefill_request  # noqa: F401
