"""MI355X-native LoGRA low-rank gradient sketching: the data-parallel hot path.

The work runs in liblogra.so (hand-written HIP for gfx950) behind a C ABI
(include/logra.h); this package only marshals torch tensors into it.
"""
from .api import (GAUSSIAN, MAX_SHARED, MAX_SWEEP, RADEMACHER, SKETCH_OVERWRITE,  # noqa: F401
                  MAX_GROUPS, MAX_LAYER_OUT, MAX_MERGE, SKETCH_DEFER, SKETCH_PENDING,
                  UPDATE_ADAM, UPDATE_MOMENTUM, UPDATE_SGD,
                  CHOICE_ACC_WIDE, CHOICE_AUTO, CHOICE_PROJECT_TILE, kernel_choice,
                  set_kernel_choice,
                  kl_budget_schedule, kl_sweep_ws_bytes, kl_ws_bytes, merge, predicted_kl,
                  predicted_kl_sweep, regen_A, sketch_accumulate, sketch_accumulate_shared,
                  sketch_accumulate_layer, sketch_layer_ws_bytes, sketch_layer_workspace,
                  merge_many, sketch_shared_ws_bytes, sketch_update, sketch_ws_bytes, sketch_workspace,
                  sketch_p_bytes, sketch_project, sketch_project_ws_bytes, sketch_accumulate_p,
                  sketch_accumulate_p_ws_bytes)
from . import sync  # noqa: F401,E402
