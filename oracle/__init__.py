"""CPU oracle for the KDA engine -- TEST INFRASTRUCTURE, never part of the product path.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this package. It shares no code with the HIP library: no kernels, headers, helpers
or tables. Inputs come from ``kda_inputs``, which holds no KDA arithmetic.

* ``kda``     -- sequential float64 recurrence and the pool/ring/metadata model.
* ``chunked`` -- an independent float64 chunked (WY/UT) formulation, used to pin ``kda``.

Parity status: the pages print no worked example and no equation, so no function here is
pinned to a printed value. Each is pinned instead by closed forms, invariants and special
cases that reduce to textbook results (see ``tests/test_oracle_pins.py``).
"""
from .kda import KDAPool, kda_scan, kda_step, ERR_NACC_RANGE  # noqa: F401
from .chunked import kda_chunk, kda_chunked  # noqa: F401
