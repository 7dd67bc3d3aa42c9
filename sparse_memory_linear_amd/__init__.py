"""SDM (Sparse Delta Memory) hot path on MI355X: product-key addressing and the
sparse gated delta scan as hand-written HIP kernels behind a C ABI
(include/sdm.h). This package holds the Python binding (``binding``), the
in-tree build (``build``) and the seeded synthetic inputs (``inputs``)."""
from . import inputs  # noqa: F401
from .binding import (SDM_BF16, SDM_DELTA_EQ4, SDM_DELTA_FIG2, SDM_F32,  # noqa: F401
                      SdmError, sdm_abi_version, sdm_address, sdm_debug_half_scores,
                      sdm_last_error, sdm_scan_backward, sdm_scan_backward_workspace_bytes,
                      sdm_scan_forward, sdm_scan_forward_gated, sdm_scan_forward_noalloc, sdm_scan_forward_save,
                      sdm_scan_gated_workspace_bytes, sdm_scan_snapshot_bytes,
                      sdm_scan_workspace_bytes, sdm_state_init, sdm_state_init_backward,
                      sdm_status_string, sdm_gates, sdm_output_gate)
