"""CPU oracle for the batched Walsh-Hadamard hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links anything in this package: only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark use it.  It shares no code, tables or
constants with the HIP library and never imports it.

Every function here is a plain, slow, fp64 statement of what the hot path
computes, written as the definition (explicit Sylvester matrix products,
naive round-to-nearest, dense adapter and dense stage matrices).

Sources, cited by short key in each docstring:

[QWHA-abs]  "QWHA: Quantization-Aware Walsh-Hadamard Adaptation for
            Parameter-Efficient Fine-Tuning on Large Language Models",
            authors' abstract (chatpaper.ai dashboard page).
[QWHA]      The gist.science explainer of the same paper; "technical
            summary" section 2.1 (the WHA adapter, Delta W = F H^-1, F
            built from a value vector c and an index list E, +-1 kernel,
            add/subtract-only fast transform) and 2.2 (AdaAlloc, refinement).
[HARP]      "HARP: Hadamard-Preconditioned Adaptive Rotation Processor for
            Extreme LLM Quantization", gist.science explainer; technical
            summary section 1 (RHT: fast, exactly orthogonal, O(d log d)),
            2.1 (mixed-radix schedule prod b_t = d, block-diagonal stages on
            stride-permuted groups), 2.2 (B_{t,c} = Q_{t,c} G_{b_t}, G the
            normalised Sylvester Hadamard; Theta = 0 recovers the fixed RHT
            up to a fixed permutation convention), 2.4 (O(d log d) cost).

Where the pages leave a convention open the oracle takes one reading and
says so in the docstring ("reading: ...").  Modules:

  hadamard  Sylvester matrix, orthonormal WHT, sign diagonal, RHT / inverse
  rtn       per-group absmax RTN quantiser, bit packing, dequant + inverse
  qwha      dense QWHA adapter forward
  harp      dense HARP stage matrices and rotation, block parametrisation
  gemv      low-bit weight x activation product with the rotation online
  qwha_init QWHA initialisation: error coefficients, AdaAlloc, refinement
  compare   parity rules used to compare a device result with the oracle
"""

from . import hadamard, rtn, qwha, harp, gemv, qwha_init, compare  # noqa: F401
