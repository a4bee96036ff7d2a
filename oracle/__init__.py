"""CPU oracle for the per-position verification pass (test infrastructure).

This package is a plain, slow, float64 reference of everything the GPU
library computes. It exists only to check the GPU path: the only code that
may import, call or execute anything under ``oracle/`` is the test suite
(``tests/``), ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``. The product path (the HIP library and its Python binding)
never touches it, and the oracle never touches the product path: the two
share no code, helpers, headers or constant tables.

Sources. Three web pages describe the method; they are cited by title and
section:

* [DualDiffusion] "DualDiffusion: A Speculative Decoding Strategy for Masked
  Diffusion Models" (gist.science summary of arXiv 2604.05250).
* [SPOT] "On the SPOT: Enhancing Speculative Decoding for Diffusion Language
  Models via Commit-Order Prediction" (paper review, blog.secrett2633.cloud).
* [COVER] "Stop the Flip-Flop: Context-Preserving Verification for Fast
  Revocable Diffusion Decoding" (gist.science summary of arXiv 2602.06161).

Modules:

* ``rowstats``  log-sum-exp, KL(p_verifier || p_drafter), verifier entropy,
  max-probability confidence and argmax, each by its textbook definition.
* ``noise``     the counter-based hash that keys the shared Gumbel noise and
  the Gumbel-max tokens of both models under that shared noise.
* ``decide``    the per-position rules (Trust, KL threshold, KL with its
  probabilistic clause, confidence threshold, confidence in the drafted
  token, COVER's KEEP/REPLACE/REMASK, coupled-noise acceptance) and the
  accepted prefix per candidate.
* ``select``    COVER's seed score and the per-sequence top-k / threshold
  selection.
* ``tree``      acceptance over a tree of candidate block states and the
  commit list it yields.
* ``attention`` COVER's influence d_in and drift sensitivity d_out from
  attention probabilities.
* ``dual_view`` COVER's attention with the KV-cache override of seed columns
  and the diagonal correction.

Every function is pinned by tests under ``tests/`` against closed forms,
library routines, invariants or brute force; none of the pages prints a
worked example, so no end-to-end value is pinned by the pages themselves.
"""

from . import rowstats, noise, decide, select, tree, attention, dual_view  # noqa: F401

__all__ = ["rowstats", "noise", "decide", "select", "tree", "attention", "dual_view"]
