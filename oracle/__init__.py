"""CPU oracle for the routed MoE FFN forward.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  It shares no code with the
HIP path; both are fed from the seeded generators in ``workloads``.

Parity status: every function here is pinned by a CPU test against something
other than itself (closed forms, invariants, brute-force enumeration, library
routines, or numbers the pages print); none is "parity unpinned".
"""
from . import e4m3, moe  # noqa: F401
