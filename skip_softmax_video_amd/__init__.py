"""skip_softmax_video_amd: skip-softmax (BLASST) attention for MI355X (gfx950).

The compute path is the HIP C-ABI library libssa.so (include/ssa.h); this
package is its thin Python binding. Build the library with
`python -m skip_softmax_video_amd.build` (or __graft_entry__.build()).
"""
from ._binding import (  # noqa: F401
    DTYPE_BF16,
    DTYPE_FP8_E4M3,
    DTYPE_MXFP8_QK,
    EXPORTED,
    GATE_BASE,
    GATE_IGNORED,
    GATE_OVERRIDE,
    GATE_TIMESTEP,
    SSA_ERR_FIT_DEGENERATE,
    SSA_ERR_HIP,
    SSA_ERR_INVALID_ARG,
    SSA_ERR_NO_FORMULA,
    SSA_ERR_THRESHOLD_RANGE,
    SSA_ERR_UNSUPPORTED,
    SSA_OK,
    SSA_WARN_EXTRAPOLATED,
    CalibrationPool,
    SSAError,
    attn_calibrate,
    attn_fwd,
    calib_num_workgroups,
    calibration_fit,
    calibration_sparsity,
    flow_timesteps,
    gate_dense_steps,
    gate_layer,
    load_library,
    make_problem,
    resolve_threshold,
    status_string,
    tile_mask_dims,
)
