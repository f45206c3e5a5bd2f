"""CPU fp64 oracle for the fused SDPA path (test infrastructure, not product code).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything here.  The oracle shares no code with the HIP
library and never calls it.

* :mod:`oracle.sdpa_ref` -- forward and backward, full score matrix, float64.
* :mod:`oracle.philox_ref` -- Philox-4x32-10 and the dropout keep mask.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
facts that do not come from the oracle itself (closed forms, invariants,
finite differences, PyTorch's own CPU float64 attention, rocRAND's Philox
and the Random123 known-answer vectors).  The index convention of the dropout
mask is a reading, pinned by hand-worked examples in ``tests/golden``.
"""

from . import philox_ref, sdpa_ref  # noqa: F401
