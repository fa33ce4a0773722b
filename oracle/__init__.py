"""fp64 CPU oracle for the Differential Attention V2 forward pass (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  The product path (``differential_attention_v2_amd``)
never does.
"""
from .diffattn_oracle import *  # noqa: F401,F403
from .diffattn_oracle import __all__  # noqa: F401
