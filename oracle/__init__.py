"""CPU oracle of the DFlash2 draft-block path: test infrastructure only.

Imported by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg,
never by the product path (the HIP library and its binding).
"""
from . import dflash_oracle  # noqa: F401
