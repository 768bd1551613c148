"""liblla: causal Local Linear Attention forward for AMD Instinct MI355X (gfx950).

The compute lives in ``liblla.so`` (hand-written HIP kernels behind a C ABI declared in
``include/lla.h``); ``lla`` is the ctypes binding.
"""
from .lla import (  # noqa: F401
    LLAError, lla_forward, lla_forward_ex, lla_path_available, lla_status_string, lla_version,
    library_path,
    load_library,
)
