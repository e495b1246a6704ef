"""MI355X-native Mamba-3 SSM recurrence: chunked prefill and decode step in HIP.

The compute lives in libm3.so (C ABI in include/m3.h); this package is its thin
Python binding plus the seeded synthetic input generators.
"""
from ._binding import (  # noqa: F401
    M3Error, M3Prologue, M3Shape, M3_BF16, M3_FP32, EXPORTS, LIB_PATH, decode_step, decode_step_gated, decode_step_prologue, load_library,
    make_shape, prefill_chunk_used, prefill_workspace_bytes, scan_prefill, scan_prefill_gated, scan_prefill_prologue,
    prefill_max_chunk, prefill_status, debug_set_spin_limit, STATUS, scan_backward, backward_workspace_bytes,
    prefill_kernel_used, debug_set_prefill_kernel, M3_KERNEL_PER_CHUNK, M3_KERNEL_STREAM,
    prefill_prologue_mode, prefill_prologue_workspace_bytes, prefill_prologue_kernel_used, prefill_gated_kernel_used, M3_PROLOGUE_FUSED, M3_PROLOGUE_STAGED,
)
