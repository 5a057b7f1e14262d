"""CPU oracle for the decomposed-layer forward pass (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package. The HIP path never imports, links or calls it.
"""
from .ref import *  # noqa: F401,F403
