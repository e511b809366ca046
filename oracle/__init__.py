"""fp64 CPU oracle of the SLA2 forward: test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the GPU path never does.
"""
from . import codecs, sla2  # noqa: F401
