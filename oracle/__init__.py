"""CPU reference ("oracle") for continuous softmax attention, float64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The HIP library never calls it and shares no code with it: the oracle follows
the per-segment integrals of the derivation, the kernels follow the
correction-weight form; the two meet only in the tests.

Source: J. Su, "Continuous Softmax Attention" (Scientific Spaces; English
translation on tylerromero.com; Chinese original mirrored on
datasets.osmarks.net).

Every function here is pinned by ``tests/test_oracle_pins.py`` against
something other than itself (quadrature of the defining integral, an
independent high-precision evaluation of the simplified form, closed forms,
invariants and limits; the gradient against finite differences of the
defining integral).  No function is "parity unpinned".
"""

from .csa import (  # noqa: F401
    phi1,
    phi2,
    csa_row,
    csa_reference,
    std_row,
    std_reference,
)
from .first_order import csa1_reference, csa1_row  # noqa: F401
from .backward import csa_backward_reference, csa_backward_row, dphi1, dphi2  # noqa: F401
from .half_interval import csa_half_reference, csa_half_row, seg_integrals  # noqa: F401
