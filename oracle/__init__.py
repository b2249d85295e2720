"""CPU oracle for the Medusa decode step (test infrastructure only).

Importable by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg,
never by the library itself.
"""
from . import medusa_oracle  # noqa: F401
