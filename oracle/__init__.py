"""CPU oracle for the block-diffusion drafter hot path.

TEST INFRASTRUCTURE.  This package is a plain, slow, obviously correct CPU statement of what the
hot path computes, written from the pages' description of the method.  Only the tests, the smoke
check and the bench's CPU-baseline leg may import it; the HIP library and its Python binding never
do, and this package never imports them.  It shares no code, tables or constants with the HIP
path; the two meet only at the seeded inputs of ``synth``.

Modules:
  drafter  - the drafter forward pass in fp64 (mixing + RMSNorm, split context/draft K/V,
             bidirectional block attention over the context, SwiGLU MLP, shared LM head);
  dnc      - integer-exact sampling and selection probabilities (argmax, exp, weights, RNG);
  accept   - greedy verification and streak-score self-selection, plus the helpers used only to
             pin the oracle (acceptance rates, Monte Carlo, enumeration);
  refine   - iterative refinement of a drafted block (Mask-Predict on the integer confidences).

Pins (tests/test_oracle_*.py): every function is checked against closed forms, invariants,
special cases, Monte Carlo or brute force.  The composed forward pass has no printed worked
example on the pages: beyond the pins of its parts it is "parity unpinned".
"""
from . import accept, dnc, drafter, refine

__all__ = ["accept", "dnc", "drafter", "refine"]
