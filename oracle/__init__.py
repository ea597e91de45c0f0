"""Plain CPU oracle for the DCP absorbed-MLA decode hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this package; only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code, table or constant with the HIP
library: it decodes the stored bytes itself, builds its own e4m3 table from
the format definition, and models the page layout with plain integers.

What it computes (each function cites the passage it follows):

* ``codecs``     bf16 and OCP e4m3fn decode to float64, per-token fp32 scale.
* ``layout``     the shared virtual allocator and slot map of the SGLang page
                 "Decode Context Parallelism" (section "Virtual KV layout"):
                 virtual capacity C*c, virtual page P*c, owner(v) = v mod c,
                 physical(v) = floor(v/c); page allocation, the new-row
                 scatter, and each rank's owned positions.
* ``attention``  full-context softmax attention in float64 (the plain result
                 that the method reaches up to reduction order), the same
                 attention restricted to one rank's striped positions, and the
                 exact log-sum-exp merge of the SGLang page (section "MLA
                 decode dataflow"), in base e or base 2.

Pins (tests under ``tests/`` marked ``not gpu``) tie each part to something
other than itself: library routines (torch's bf16/e4m3 casts, torch's
scaled-dot-product attention and logsumexp in float64), closed forms, the
pages' literal examples, invariants and brute-force enumeration.
"""
from . import codecs, layout, attention  # noqa: F401
