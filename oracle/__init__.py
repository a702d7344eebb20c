"""CPU oracle for speculative-draft branch attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in this package.  The product path
(the HIP library and its Python binding) never does, and this package imports
nothing from it: the two share no code.

What it computes is the plain definition of the operator: for every query row
(main-sequence rows and draft-branch rows) one softmax over the union of the
keys that row may see -- its sequence's causal main prefix and, for a branch
row, the allowed keys of its own branch -- with a dense boolean mask.  The
method on the pages reaches the same result by splitting the key set into a
main-sequence part and a rank-local branch part and merging the two partial
softmaxes with the log-sum-exp reduction (evolve.pub review, "Scope & Claims":
branch attention under CP, the online-softmax reduction of Eq. 2; rcap.io
explainer, paragraph on branch attention under context parallelism).  The
split itself is also written out here (``split_forward``) so tests can check
that split-then-merge equals the union softmax, and so is the ring form of the
main-key part (``ring_forward``: key windows merged one after another, as a
context-parallel ring delivers them).

Arithmetic is float64 unless a caller asks otherwise.

``oracle.tapchannel`` is a plain model of the tap mailbox (slots with sequence
stamps, one-way writes and reads; rcap.io explainer, the TapChannel paragraph),
pinned in ``tests/test_tapchannel_host.py`` by every interleaving of a small
writer and reader and by a hand-worked script.

Readings adopted where the pages are silent (each is also a test):
  * softmax scale 1/sqrt(head_dim); LSE is the natural log of sum(exp(scale*q.k));
  * a branch row sees main keys from its sequence start to its anchor,
    inclusive; TTT query j sees branch keys 1..j; block queries see all keys of
    their block; no row sees another anchor's branch; main rows never see
    branch keys;
  * the backward pass is the exact gradient of the union softmax;
  * an empty partial is (O=0, LSE=-inf) and merging with it is the identity.

Parity unpinned: none -- every function is pinned by tests in
``tests/test_oracle_pins.py`` (brute force, closed forms, library reductions,
finite differences, invariants).
"""
from .branch_attention import (  # noqa: F401
    TTT, BLOCK, Problem, row_keys, dense_mask, attend, attend_bwd, forward, backward,
    forward_rows, backward_rows, lse_merge, split_forward, ring_forward, pair_counts,
)
