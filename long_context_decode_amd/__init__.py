"""JSSA decode hot path on MI355X (gfx950): Python binding of libjssa.so.

The names mirror the C ABI in include/jssa.h; the library's HIP kernels do all
of the work.  Importing this package fails if libjssa.so has not been built.
"""
from ._lib import (  # noqa: F401
    OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_ALIGN,
    KIND_GQA, KIND_MLA, SELECT_AUTO, SELECT_EXACT_STREAM, SELECT_SPLIT, SELECT_FUSED,
    STAGE_PROLOGUE, STAGE_STREAM, STAGE_FINISH, STAGE_ALL,
    SCALE_FP32, SCALE_E8M0, SCALE_NONE, KEYS_BF16, SCALE_FORMATS, MLA_LATENT, MLA_ROPE, EXPORTED, LIB_PATH,
    JSSAError, Shape, make_shape, shape_for, status_string, workspace_bytes, decode_single_launch, kp_page_bytes,
    attend_splits,
    alloc_workspace,
    alloc_scoring_cache, jssa_store, jssa_select, jssa_attend, jssa_attend_noalloc, jssa_decode, jssa_full_decode, jssa_gather_attend,
    calib_workspace_bytes, jssa_calib_moments, jssa_basis, raw_library,
)
