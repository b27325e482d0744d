"""MI355X-native Q4 expert: gate/up + SwiGLU, down projection, whole expert.

The computation lives in hand-written HIP kernels for gfx950 behind the C ABI
of ``include/q4moe.h`` (``libq4moe.so`` in this package directory).  This
package only marshals arguments to it (``_lib``) and allocates aligned device
buffers with PyTorch (``device``).
"""
from ._lib import (  # noqa: F401
    OFFSET_ABSENT,
    Q4Error,
    Q4_OK,
    Q4_ERR_INVALID_ARGUMENT,
    Q4_ERR_ALIGNMENT,
    Q4_ERR_RANGE,
    Q4_ERR_UNSUPPORTED,
    Q4_ERR_HIP,
    Q4_ERR_WORKSPACE,
    LIB_PATH,
    load,
    last_error,
    abi_version,
    grouped_workspace_bytes,
    expert_gate_up,
    expert_gate_up_grouped,
    expert_gate_up_grouped_noalloc,
    validate_gate_up,
    validate_grouped,
    expert_down,
    expert_down_grouped,
    expert_forward,
    expert_forward_grouped,
    validate_down,
    validate_down_grouped,
    stream_read,
)
