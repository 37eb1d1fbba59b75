"""CPU oracle for the SparseGemv path (TEST INFRASTRUCTURE ONLY).

Plain, slow, obviously-correct NumPy (FP64 where floating point is involved)
implementation of what the SparseGemv path computes, written from the page
"Efficient large-model ad applications through model compression and parallel verification"
(an English gloss of its Chinese title; the page is a Chinese translation of
arXiv 2605.11582; cited below as P1) and from the
plainest readings where that page is silent.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in this package. The product library
(``sparse_weight_only_amd``) never imports it and shares no code with it;
both are fed the same seeded inputs from ``synth``.

Modules and what pins each one (tests under ``tests/test_oracle_*.py``):

* ``fp16``   - FP64 -> FP16 round-to-nearest-even; pinned against an exact
               rational rounding of every tie and of random doubles.
* ``prune``  - N:M selection along K (P1 §3.2 "Sparsification"), by |w| or
               by the activation-aware score |w| * ||x_k|| of eq. (3);
               pinned by brute force over every kept subset and a
               hand-worked group where the two scores disagree.
* ``groups`` - per-output-channel group size (P1 §3.2 "Adaptive group
               quantization", eq. (3) first term); pinned by exact rational
               sums and ranking on tiny matrices.
* ``quant``  - asymmetric INT4 group quantisation (P1 §1 "our core idea":
               FP16 -> INT4 weight-only); pinned by grid-exact round trips,
               hand-worked examples and the half-step error bound.
* ``pack``   - canonical 2bit-CSR arrays (P1 §1 contributions, first item);
               pinned by unpack(pack) round trips, closed-form sizes, a
               hand-packed example and the 30 % size claim.
* ``layout`` - the kernel's physical permutation of the canonical arrays;
               pinned by a bijection check and a hand-placed example.
* ``gemv``   - dense dequantise-then-dot in FP64 and the normalised error;
               pinned by exact rational sums, math.fsum and unit vectors.

Parity unpinned: nothing in this package. What the pages leave open (their
own bit layout, their sensitivity measure, their kernel) is replaced by
explicit readings, each stated with the function that takes it; those
readings are pinned, the pages' originals cannot be.
"""
from . import fp16, prune, groups, quant, pack, layout, gemv  # noqa: F401
