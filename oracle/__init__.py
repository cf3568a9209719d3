"""fp64 CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this package.  It shares no code with the GPU library.
"""
from .mhla_oracle import *  # noqa: F401,F403
from .mhla_oracle import __all__ as _forward_all
from .mhla_backward import backward, dphi_map, mala_backward, mhla_backward_blockwise  # noqa: F401
from .mhla_causal import (causal_blockwise, causal_plain, causal_sampled, forward_causal,  # noqa: F401
                          forward_causal_sampled)

__all__ = list(_forward_all) + ["backward", "dphi_map", "mala_backward", "mhla_backward_blockwise",
                                "causal_blockwise", "causal_plain", "causal_sampled", "forward_causal",
                                "forward_causal_sampled"]
