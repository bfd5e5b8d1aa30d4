"""CPU oracle for the ball-tree / ball-attention / BSA hot path.

TEST INFRASTRUCTURE ONLY.  Plain, slow, obviously correct NumPy code (fp64 for
all floating-point attention arithmetic; fp32 only where the tree's split rule
is defined on fp32 coordinates).  It shares no code with the HIP library and
never imports it.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in here; the
product path never falls back to it.

Modules
-------
``tree``       recursive median-split ball tree, the rotated tree, and the
               padded tree of an uneven N.
``attention``  ball attention (scaled dot-product attention inside each ball),
               on a padded tree too, and full attention, in fp64.
``attention_bwd`` gradients of ball attention (dq, dk, dv), in fp64.
``bsa``        brute-force Ball Sparse Attention: ball, compression and
               selection branches merged by sigmoid gates (and the group
               compression variant), in fp64.
``bsa_bwd``    gradients of BSA (dq, dk, dv and the gate parameters), in fp64.
``pool``       coarsening (means of consecutive tree positions) and refinement.
``permute``    row gather / scatter between original and tree order, the
               inverse permutation, and their padded forms.
``checks``     tree invariant checkers (plain and padded), independent of
               ``tree``.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against closed forms, library routines, invariants
and hand-enumerated golden cases; none is "parity unpinned".
"""
