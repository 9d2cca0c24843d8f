"""fp64 oracle for the Gated DeltaNet layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything in this package.  It shares no code with the
HIP library (``gated_deltanet_linear_rule_amd``), and the library never
imports it: the product path has no CPU fallback.

* ``oracle.c_oracle``  -- plain C, fp64, sequential per token (gdn_oracle.c);
* ``oracle.reference`` -- numpy fp64: literal matrix form, unrolled closed
  form, and the chunk-wise WY/UT form, for tiny sizes.

Parity status: every function is pinned by the tests in
``tests/test_oracle_pins.py`` against closed forms and invariants of the
recurrence; the pages print no worked numeric example, so no value from the
pages themselves pins it.
"""
