"""CPU oracle for continuous depth batching (CDB) — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything under this package.  The product library
(``continuous_depth_batching_amd``) never imports, calls or links it, and it
shares no code with that library: the only common module is ``cdb_synth``,
which holds seeded inputs and no arithmetic of the method.

The oracle is a plain, slow, per-sequence implementation written from
"Depth-adaptive Inference of Looped Language Models via Continuous Depth
Batching" (arXiv 2608.09444):

* ``layers``   – RMSNorm, rotary embedding, SwiGLU and softmax attention,
                 plus a brute-force triple-loop attention for tiny inputs.
* ``model``    – the looped LM of §2 decoded one sequence at a time, with the
                 depth-indexed cache and its last-exited fill of §4.2, the
                 shared single-slot cache of §4.2 / App. E.1, the lookahead
                 gate of §4.3 / §7, forced replay with decision margins, and a
                 single-row core step for synthetic cached context.
* ``unrolled`` – an independently written plain deep transformer (fp64,
                 torch CPU) that a gate-off looped model must equal.
* ``cdb_sim``  – the stage queues of §4.1 driven by Alg. 1 (no-refill) and
                 Alg. 2 (refill), and fixed-depth continuous batching.
* ``bounds``   – Eq. 1, Eq. 2, the latency fit of Eq. 4 and the KV footprint
                 of App. E.1.
* ``precision_floor`` – the oracle with bf16 rounding at the storage points
                 of a bf16 path (§6.1 runs in bfloat16), to measure how far
                 bf16 storage alone moves states and logits.
* ``calibrate_gate`` – the gate-bias bisection that fixes each
                 configuration's mean exit depth.

Parity status: every function has a pin in ``tests/test_oracle_*.py`` except
the numeric values of hidden states, logits and exit distributions of a
random-init model, for which the pages print no worked example (parity
unpinned beyond the invariants the tests check).
"""
