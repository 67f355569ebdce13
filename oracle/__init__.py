"""CPU oracle of the sync-free MoE GroupGEMM + GLU path.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path (the HIP library and
its Python binding).  It shares no code with the GPU path.
"""
from . import formats, moe  # noqa: F401
