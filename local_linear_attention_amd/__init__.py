"""liblla: causal Local Linear Attention forward and decode, and the Parallax forward, decode
and backward with a given probe, for AMD Instinct MI355X (gfx950).

The compute lives in ``liblla.so`` (hand-written HIP kernels behind a C ABI declared in
``include/lla.h``); ``lla`` is the ctypes binding.
"""
from .lla import (  # noqa: F401
    LLAError, library_path, lla_decode, lla_decode_workspace_size, lla_decode_ws, lla_forward, lla_forward_ex,
    lla_forward_fallback_rows, lla_forward_ws, lla_parallax_decode,
    lla_parallax_backward, lla_parallax_backward_workspace_size,
    lla_parallax_decode_workspace_size, lla_parallax_decode_ws, lla_parallax_forward, lla_parallax_forward_stats,
    lla_parallax_forward_ex, lla_parallax_forward_ws, lla_parallax_path_available,
    lla_parallax_workspace_size, lla_path_available, lla_profile_collect, lla_profile_enable,
    lla_status_string, lla_version, lla_workspace_size,
    load_library,
)
