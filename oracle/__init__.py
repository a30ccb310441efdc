"""CPU oracles for the frame-wise Gated DeltaNet forward (causal and
bidirectional) and the streaming attention block -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The HIP library and its
Python binding never import it, and it imports nothing from them: the only
code both sides share is the seeded input generator, which holds none of the
method's arithmetic.

Contents
--------
``recurrence``  plain fp64 token-by-token recurrence (C, threaded over the
                independent (batch, head) units) -- THE oracle.
``chunked``     fp64 chunked (UT / WY) form of the same recurrence, derived
                from it; pins the algebra the GPU path uses and exposes its
                per-chunk intermediates.
``exact``       exact-rational brute force of the product form on tiny inputs.
``attention``   fp64 softmax attention of the streaming chunk-causal attention
                block (sink frames + rolling cache of past blocks).
``bidirectional`` the dense checkpoint's bidirectional GDN: reverse scan of the
                same recurrence (decays on the same frame boundaries) plus the
                forward scan.

Every function pins to something other than itself in ``tests/test_oracle_*``:
hand-derived values, closed forms, exact rationals, limits and invariants.
"""
