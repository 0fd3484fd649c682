"""CPU oracle for the GDN state update (and the Mamba2 replay variant) -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the library never does.
"""
from .gdn_oracle import *  # noqa: F401,F403
from .mamba2_oracle import *  # noqa: F401,F403
