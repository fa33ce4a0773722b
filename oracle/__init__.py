"""fp64 CPU oracle for the Differential Attention V2 forward and backward passes
(test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package.  The product path (``differential_attention_v2_amd``)
never does.
"""
from .diffattn_oracle import *  # noqa: F401,F403
from .diffattn_oracle import __all__ as _fwd_all
from .diffattn_backward import *  # noqa: F401,F403
from .diffattn_backward import __all__ as _bwd_all
from .projections import *  # noqa: F401,F403
from .projections import __all__ as _proj_all

__all__ = list(_fwd_all) + list(_bwd_all) + list(_proj_all)
