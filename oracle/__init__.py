"""CPU oracle of the compressed sparse attention path (float64 numpy).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg.  The product path never imports it.
"""
from . import codecs, csa_ref  # noqa: F401
