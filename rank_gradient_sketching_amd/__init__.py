"""MI355X-native LoGRA low-rank gradient sketching: the data-parallel hot path.

The work runs in liblogra.so (hand-written HIP for gfx950) behind a C ABI
(include/logra.h); this package only marshals torch tensors into it.
"""
from .api import (GAUSSIAN, RADEMACHER, kl_ws_bytes, merge, predicted_kl,  # noqa: F401
                  regen_A, sketch_accumulate, sketch_ws_bytes, sketch_workspace)
