"""Test infrastructure: the fp64 CPU oracle of the owner-side Muon step.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything under ``oracle/``.  The product path (the HIP
library and its Python binding) never does, and this package never imports the
product path.
"""

from .muon_oracle import (  # noqa: F401
    NS_COEFFS,
    frobenius_normalize,
    gram_newton_schulz,
    momentum,
    muon_step,
    newton_schulz,
    ns_cost,
    ns_iteration,
    apply_update,
    update_scale,
    round_to_bf16,
    round_to_f32,
)
from .plan_oracle import plan_reference, tile_granularity  # noqa: F401
from .adamw_oracle import ADAMW_DEFAULTS, adamw_step  # noqa: F401
