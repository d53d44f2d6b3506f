"""CPU oracle for MXFP4 UOS + PNQ attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy implementation of what the GPU path
computes, written from the MXAttention pages (the arXiv abstract page, the
Pith review with its referee report, axiom ledger and figure captions, the
Pith verdict record, and the 10100.com explainer).  Floating point is float64
except where a step is defined in fp32 for bit-exactness (the Hadamard
butterflies, and the fp32 value of P~ on which its codes are decided).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``mxfp4_bit_attention_amd``) and imports nothing from it; the product path
never calls it.

Modules:
  mxfp4      E2M1 grid, rounding, scale rules (UOS / OCP / CEIL q), block quantiser.
  hadamard   Sylvester Hadamard rotation, defined in fp32.
  attention  flash attention on MXFP4 operands with PNQ or direct placement,
             post-normalisation diagnostic, exact softmax attention.
  uos        E(x), D(x), Delta(q), J(q) of the data-free scale objective.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
against values or properties the pages and the mathematics fix (see
tests/test_oracle_*.py); none is "parity unpinned".
"""
from . import attention, hadamard, mxfp4, uos  # noqa: F401
