"""MI355X-native DSpark-style draft sampling, verification and confidence scheduling.

The compute path is the HIP library ``libdspark.so`` (C ABI in
``include/dspark.h``); this package is its thin Python binding plus the seeded
synthetic workload generators.
"""
from .binding import (  # noqa: F401
    DSPARK_BF16,
    DSPARK_F32,
    KERNELS,
    DsparkError,
    LIB_PATH,
    dspark_draft_sample,
    dspark_draft_sample_noalloc,
    dspark_draft_workspace_bytes,
    dspark_profile_begin,
    dspark_profile_end,
    dspark_schedule,
    dspark_schedule_workspace_bytes,
    dspark_verify,
    dspark_verify_workspace_bytes,
    dspark_version,
    header_functions,
    lib,
)
