"""Frame-structured block-sparse attention for AMD MI355X (gfx950).

The compute path is the HIP library libfsattn.so (C ABI in include/fsattn.h);
this package is its thin Python binding."""
from .fsattn import (Bounds, DevicePlan, FsattnError, Mask, abi_version, device_plan,  # noqa: F401
                     forward, head_bounds, head_bounds_noalloc, head_bounds_workspace_bytes, launch_info, lib,
                     make_flags, mfma_probe, noalloc_max_workspace,
                     prior_art_forward, prior_art_workspace_bytes, produce,
                     plan, plan_on_device, plan_size, status_string, to_mask)
from .fsattn import (BF16, F32, MODE_AUTO, MODE_FORCE_FIXED, MODE_FORCE_ONLINE,  # noqa: F401
                     SHIFT_PER_ROW, DEFAULT_GAP_NATS)
