"""CPU oracle for the MXFP4 linear-layer triple -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
or run anything in this package. The product path (the HIP library and its
Python binding) never calls it, and it shares no code with that path.

Parity status of every function here: pinned (see oracle/mx_oracle.py's
header for what pins each one). No function is "parity unpinned".
"""
from .mx_oracle import *  # noqa: F401,F403
from .mx_oracle import __all__  # noqa: F401
