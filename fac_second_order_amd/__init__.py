"""MI355X-native single-GPU K-FAC step (HIP kernels for gfx950 behind a C ABI).

The functions below carry the names of the C entry points in include/kfac.h and only
marshal arguments. Importing this package loads libkfac.so and fails loudly if it has
not been built (python fac_second_order_amd/build.py)."""
from ._lib import (  # noqa: F401
    KFAC_F16, KFAC_F32, KFAC_F64, KfacError, LIB_PATH, kfac_version,
    kfac_factors_workspace, kfac_factors, kfac_factors_full,
    kfac_pack_sym_workspace, kfac_pack_sym,
    kfac_invert_workspace, kfac_invert_schedule, kfac_invert,
    kfac_invert_refine_workspace, kfac_invert_refine,
    kfac_precondition_workspace, kfac_precondition, kfac_precondition_update, kfac_precondition_ex,
    kfac_bn_diag_workspace, kfac_bn_diag, kfac_bn_update, kfac_bn_diag_noalloc,
    kfac_timing_kernels, kfac_kernel_name, kfac_timing_enable, kfac_timing_only, kfac_timing_reset,
    kfac_timing_read,
)
from .step import KfacStep  # noqa: F401
