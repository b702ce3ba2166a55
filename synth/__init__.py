"""Seeded synthetic inputs for the ZeRO-3 shard step.

This package holds no arithmetic of the method: only workload shapes
(``configs``) and seeded random inputs (``gen``).  It is the one module that
both the HIP path's tests/bench and the CPU oracle's checks draw inputs from.
"""

from .configs import CONFIGS, Config, ParamSpec, get_config  # noqa: F401
