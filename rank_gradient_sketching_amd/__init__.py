"""MI355X-native LoGRA low-rank gradient sketching: the data-parallel hot path.

The work runs in liblogra.so (hand-written HIP for gfx950) behind a C ABI
(include/logra.h); this package only marshals torch tensors into it.
"""
from .api import (GAUSSIAN, MAX_SWEEP, RADEMACHER, kl_budget_schedule,  # noqa: F401
                  kl_sweep_ws_bytes, kl_ws_bytes, merge, predicted_kl, predicted_kl_sweep,
                  regen_A, sketch_accumulate, sketch_ws_bytes, sketch_workspace)
