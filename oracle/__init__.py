"""fp64 CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this package.  It shares no code with the GPU library.
"""
from .mhla_oracle import *  # noqa: F401,F403
from .mhla_oracle import __all__ as _forward_all
from .mhla_backward import backward, dphi_map, mala_backward, mhla_backward_blockwise  # noqa: F401

__all__ = list(_forward_all) + ["backward", "dphi_map", "mala_backward", "mhla_backward_blockwise"]
