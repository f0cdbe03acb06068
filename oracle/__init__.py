"""CPU oracle of the DFlash2 block-drafter forward pass (float64 NumPy).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code with
the HIP library.  Every function cites the page passage it follows; see
`oracle.dflash2` for the list of sources and readings.
"""
from . import dflash2  # noqa: F401
