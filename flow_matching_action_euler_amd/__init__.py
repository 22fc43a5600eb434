"""MI355X (gfx950) flow-matching action-expert denoise loop behind a C-ABI (include/ae.h).

``ActionExpert`` wraps one library handle; every step of the path runs in the
HIP library ``libae.so`` built by ``flow_matching_action_euler_amd.build``.
"""
from .binding import ActionExpert, AEError, load_library, LIB_PATH, EXPORTS  # noqa: F401
