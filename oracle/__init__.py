"""Plain fp64 CPU oracle for causal linear attention and the gated delta rule.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only the tests under ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call it.  It shares no code
with the HIP library (no kernels, headers, helpers or constants) and imports
nothing from it.

Every function works on numpy float64 arrays, one head at a time, with the
shapes the source page uses for its exercises: Q, K of shape (T, d_k), V of
shape (T, d_v), state S of shape (d_v, d_k), normaliser z of shape (d_k,).
Batched wrappers over [B, H, T, d] live in :mod:`oracle.batched`.

Source page, cited by title and section throughout: "Linear attention and
hybrids" (ai.flicky.cc, stage 5, module 5.5 long context, lesson 03).

Parity pins: every function here is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` against values printed on the page, closed forms,
invariants or brute force.  No function is "parity unpinned".
"""

from .linear_attention import (
    phi,
    la_parallel,
    la_recurrent,
    la_chunked,
    la_decode_step,
    decayed_recurrent,
    decayed_parallel,
    gated_recurrent,
    gated_parallel,
    gated_decode_step,
)
from .gated_delta import (
    gdn_recurrent,
    gdn_chunked,
    gdn_parallel,
    gdn_decode_step,
    gdn_bruteforce_states,
)
from .kda import (
    kda_recurrent,
    kda_chunked,
    kda_decode_step,
    kda_bruteforce_states,
)
from . import batched
from . import preops
from . import varlen

__all__ = [
    "phi",
    "la_parallel",
    "la_recurrent",
    "la_chunked",
    "la_decode_step",
    "decayed_recurrent",
    "decayed_parallel",
    "gdn_recurrent",
    "gdn_chunked",
    "gdn_parallel",
    "gdn_decode_step",
    "gdn_bruteforce_states",
    "kda_recurrent",
    "kda_chunked",
    "kda_decode_step",
    "kda_bruteforce_states",
    "batched",
    "preops",
    "varlen",
]
