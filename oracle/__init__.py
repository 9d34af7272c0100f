"""CPU oracle (fp64 NumPy) for the latent-KV decode attention path.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. It shares no code with the HIP path.
"""
from .palu_oracle import *  # noqa: F401,F403
from .palu_oracle import __all__  # noqa: F401
