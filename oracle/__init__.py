"""Plain CPU oracle for the all-reduce family (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and nothing
here imports the product.  The two sides share no code: the only thing both
consume is the seeded input generator, which holds none of the arithmetic.

The oracle is written from the text of these web pages (cited by title and
section in every function):

* "NCCL collectives, ring all-reduce & launching TP/PP"
  (inference-learning-path) -- definitions of all-reduce, all-gather,
  reduce-scatter; ring = reduce-scatter + all-gather; the all-ones sanity test.
* "Collective communication: NCCL's algorithms and protocols, and custom
  all-reduce" (ai-infra-handbooks) -- ring / one-shot / two-shot, the
  alpha-beta model and its printed table, the LL / LL128 / Simple protocols,
  algbw / busbw, and the exercises.

Every result the method computes has a plain definition (an elementwise SUM
over ranks), so the oracle is that definition written out, in the fixed
association order each algorithm implies, in the precision the method fixes
(fp32 adds, int32 wrapping adds, bf16 widened to fp32 and rounded
to-nearest-even).  Modules:

``bf16``         bf16 <-> fp32 conversions (widen, RNE narrow).
``dtypes``       the three payload types and their SUM.
``geometry``     block / chunk geometry of the schedules.
``collectives``  one-shot, two-shot, ring all-reduce; direct and ring
                 reduce-scatter and all-gather.
``proto``        LL and LL128 line codecs and their byte counts.
``cost``         alpha-beta model, algbw / busbw, crossover.
``traffic``      link bytes per rank and HBM bytes per call, tallied by
                 walking each schedule's transfers.
``sim``          a dependency-graph walk of the schedules that reports the
                 first blocked (rank, step) when a signal is withheld.

Parity status: every function above is pinned by ``tests/test_oracle_*.py``
against something other than itself (closed forms, printed values, brute
force, a library conversion); none is "parity unpinned".
"""
