"""ctypes binding of libq4moe.so: argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI
declared in include/q4moe.h.  This module turns tensors into device pointers,
passes the current HIP stream, and raises on a non-zero status.  It never
computes a result itself and has no fallback: without the built library every
call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libq4moe.so")

OFFSET_ABSENT = (1 << 64) - 1

Q4_OK = 0
Q4_ERR_INVALID_ARGUMENT = -1
Q4_ERR_ALIGNMENT = -2
Q4_ERR_RANGE = -3
Q4_ERR_UNSUPPORTED = -4
Q4_ERR_HIP = -5
Q4_ERR_WORKSPACE = -6

STATUS_NAMES = {
    Q4_OK: "OK",
    Q4_ERR_INVALID_ARGUMENT: "INVALID_ARGUMENT",
    Q4_ERR_ALIGNMENT: "ALIGNMENT",
    Q4_ERR_RANGE: "RANGE",
    Q4_ERR_UNSUPPORTED: "UNSUPPORTED",
    Q4_ERR_HIP: "HIP_ERROR",
    Q4_ERR_WORKSPACE: "WORKSPACE",
}


class Q4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class SlotLayoutC(ctypes.Structure):
    _fields_ = [
        ("slot_bytes", ctypes.c_uint64),
        ("gate_weight_offset", ctypes.c_uint64),
        ("up_weight_offset", ctypes.c_uint64),
        ("gate_scale_offset", ctypes.c_uint64),
        ("up_scale_offset", ctypes.c_uint64),
        ("down_weight_offset", ctypes.c_uint64),
        ("down_scale_offset", ctypes.c_uint64),
    ]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_SZ = ctypes.c_size_t
_LAYOUT = ctypes.POINTER(SlotLayoutC)

_SIGNATURES = {
    "q4_expert_gate_up": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P]),
    "q4_expert_gate_up_probe": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "q4_grouped_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "q4_stream_read": (ctypes.c_int, [_P, _U64, _I64, _U64, _U64, _I64, _I64, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, _P, _P]),
    "q4_expert_gate_up_grouped": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                 _P, _P, _SZ, _P]),
    "q4_expert_gate_up_grouped_probe": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64,
                                                       _I64, _P, _P, _P, _P, _SZ, _P]),
    "q4_expert_gate_up_grouped_noalloc": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64,
                                                         _I64, _P, _P, _P]),
    "q4_validate_gate_up": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P]),
    "q4_validate_grouped": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64, _P, _P,
                                           _SZ]),
    "q4_expert_down": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P]),
    "q4_expert_down_probe": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P]),
    "q4_expert_down_grouped": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                              _P, _P, _SZ, _P]),
    "q4_expert_down_grouped_probe": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                    _P, _P, _P, _SZ, _P]),
    "q4_expert_forward": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P]),
    "q4_expert_forward_grouped": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                 _P, _P, _P, _SZ, _P]),
    "q4_validate_down": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P]),
    "q4_validate_down_grouped": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64, _P,
                                                _P, _SZ]),
    "q4_last_error": (ctypes.c_char_p, []),
    "q4_abi_version": (ctypes.c_int, []),
    "q8_expert_gate_up": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P]),
    "q8_expert_gate_up_probe": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "q8_expert_gate_up_grouped": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                 _P, _P, _SZ, _P]),
    "q8_expert_gate_up_grouped_probe": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64,
                                                       _I64, _P, _P, _P, _P, _SZ, _P]),
    "q8_validate_gate_up": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P]),
    "q8_validate_grouped": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64, _P, _P,
                                           _SZ]),
    "q8_expert_down": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P]),
    "q8_expert_down_probe": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P]),
    "q8_expert_down_grouped": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                              _P, _P, _SZ, _P]),
    "q8_expert_down_grouped_probe": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                    _P, _P, _P, _SZ, _P]),
    "q8_expert_forward": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P]),
    "q8_expert_forward_grouped": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                 _P, _P, _P, _SZ, _P]),
    "q8_validate_down": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P]),
    "q8_validate_down_grouped": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64, _P,
                                                _P, _SZ]),
    "q4_expert_gate_up_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P]),
    "q4_expert_gate_up_probe_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "q4_expert_gate_up_grouped_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                 _P, _P, _SZ, _P]),
    "q4_expert_gate_up_grouped_probe_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64,
                                                       _I64, _P, _P, _P, _P, _SZ, _P]),
    "q4_validate_gate_up_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P]),
    "q4_validate_grouped_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64, _P, _P,
                                           _SZ]),
    "q4_expert_down_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P]),
    "q4_expert_down_probe_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P]),
    "q4_expert_down_grouped_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                              _P, _P, _SZ, _P]),
    "q4_expert_down_grouped_probe_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                    _P, _P, _P, _SZ, _P]),
    "q4_expert_forward_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P]),
    "q4_expert_forward_grouped_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                 _P, _P, _P, _SZ, _P]),
    "q4_validate_down_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P]),
    "q4_validate_down_grouped_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64, _P,
                                                _P, _SZ]),
    "q8_expert_gate_up_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P]),
    "q8_expert_gate_up_probe_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "q8_expert_gate_up_grouped_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                 _P, _P, _SZ, _P]),
    "q8_expert_gate_up_grouped_probe_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64,
                                                       _I64, _P, _P, _P, _P, _SZ, _P]),
    "q8_validate_gate_up_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P]),
    "q8_validate_grouped_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64, _P, _P,
                                           _SZ]),
    "q8_expert_down_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P]),
    "q8_expert_down_probe_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P]),
    "q8_expert_down_grouped_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                              _P, _P, _SZ, _P]),
    "q8_expert_down_grouped_probe_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                    _P, _P, _P, _SZ, _P]),
    "q8_expert_forward_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P, _P, _P]),
    "q8_expert_forward_grouped_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64,
                                                 _P, _P, _P, _SZ, _P]),
    "q8_validate_down_f32": (ctypes.c_int, [_P, _LAYOUT, _P, _I64, _I64, _I64, _P]),
    "q8_validate_down_grouped_f32": (ctypes.c_int, [_P, _U64, _I64, _LAYOUT, _P, _I64, _P, _I64, _I64, _I64, _P,
                                                _P, _SZ]),
}

_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libq4moe.so from the package directory (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m quantized_moe_expert_q4_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _fn(lib, fmt: str, name: str, xdtype: str = "bf16"):
    """Entry point ``<fmt>_<name>[_f32]`` of the library: ``fmt`` is "q4"
    (packed nibbles) or "q8" (int8 weights); ``xdtype`` is "bf16" or "f32"
    (activations and outputs)."""
    if fmt not in ("q4", "q8"):
        raise ValueError(f"weight format must be 'q4' or 'q8', not {fmt!r}")
    if xdtype not in ("bf16", "f32"):
        raise ValueError(f"activation dtype must be 'bf16' or 'f32', not {xdtype!r}")
    return getattr(lib, f"{fmt}_{name}" + ("_f32" if xdtype == "f32" else ""))


def last_error() -> str:
    return load().q4_last_error().decode()


def abi_version() -> int:
    return load().q4_abi_version()


def layout_c(layout) -> SlotLayoutC:
    """Marshal any object with the seven offset attributes into the C struct."""
    return SlotLayoutC(
        int(layout.slot_bytes), int(layout.gate_weight_offset), int(layout.up_weight_offset),
        int(layout.gate_scale_offset), int(layout.up_scale_offset),
        int(getattr(layout, "down_weight_offset", OFFSET_ABSENT)),
        int(getattr(layout, "down_scale_offset", OFFSET_ABSENT)))


def _check(status: int) -> int:
    if status != Q4_OK:
        raise Q4Error(status, last_error())
    return status


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


_XDTYPE_NAMES = {"bf16": "bfloat16", "f32": "float32"}


def _args(*specs) -> None:
    """Reject tensor arguments the kernels would misread.  Each spec is
    (name, tensor, dtype, numel): the tensor must have that dtype, be
    contiguous, hold at least ``numel`` elements and live in device memory
    (dtype, layout and size of every argument are checked before any
    device).  Raw integer pointers pass unchecked; None is left to the
    library's own checks (required pointers) or means "skip" (probes)."""
    live = [sp for sp in specs if sp[1] is not None and not isinstance(sp[1], int)]
    for name, t, dtype, numel in live:
        got = str(t.dtype).replace("torch.", "")
        if got != dtype:
            raise ValueError(f"{name} must be a {dtype} tensor, not {got}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() < numel:
            raise ValueError(f"{name} holds {t.numel()} elements, fewer than the {numel} the call reads or writes")
    for name, t, _, _ in live:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device (cuda) tensor, not on {t.device.type}")


def _slots_spec(name: str, t, num_slots: int, stride: int, layout):
    return (name, t, "uint8", (int(num_slots) - 1) * int(stride) + int(layout.slot_bytes))


def grouped_workspace_bytes(M: int, K: int, num_slots: int) -> int:
    return int(load().q4_grouped_workspace_bytes(M, K, num_slots))


def expert_gate_up(slot, layout, x, M: int, H: int, I: int, out, gate_probe=None, up_probe=None,
                   stream=None, fmt: str = "q4", xdtype: str = "bf16") -> None:
    """Enqueue the single-expert kernel (see q4_expert_gate_up in include/q4moe.h)."""
    lib = load()
    fn = _fn(lib, fmt, "expert_gate_up_probe" if (gate_probe is not None or up_probe is not None)
             else "expert_gate_up", xdtype)
    xt = _XDTYPE_NAMES[xdtype]
    _args(_slots_spec("slot", slot, 1, layout.slot_bytes, layout), ("x", x, xt, M * H), ("out", out, xt, M * I),
          ("gate_probe", gate_probe, "float32", M * I), ("up_probe", up_probe, "float32", M * I))
    lay = layout_c(layout)
    if gate_probe is None and up_probe is None:
        st = fn(_ptr(slot), ctypes.byref(lay), _ptr(x), M, H, I, _ptr(out), _stream(stream))
    else:
        st = fn(_ptr(slot), ctypes.byref(lay), _ptr(x), M, H, I, _ptr(out), _ptr(gate_probe), _ptr(up_probe),
                _stream(stream))
    _check(st)


def _grouped_specs(slots_base, slot_stride, num_slots, layout, x, M, slot_ids, K, n_in, out, n_out, workspace,
                   workspace_bytes, xdtype, in_name="x"):
    xt = _XDTYPE_NAMES[xdtype]
    return [_slots_spec("slots_base", slots_base, num_slots, slot_stride, layout), (in_name, x, xt, n_in),
            ("slot_ids", slot_ids, "int32", M * K), ("out", out, xt, n_out),
            ("workspace", workspace, "uint8", workspace_bytes)]


def expert_gate_up_grouped(slots_base, slot_stride: int, num_slots: int, layout, x, M: int, slot_ids, K: int,
                           H: int, I: int, out, workspace, workspace_bytes: int, gate_probe=None,
                           up_probe=None, stream=None, fmt: str = "q4", xdtype: str = "bf16") -> None:
    """Enqueue the grouped kernel (see q4_expert_gate_up_grouped in include/q4moe.h)."""
    lib = load()
    probes = gate_probe is not None or up_probe is not None
    fn = _fn(lib, fmt, "expert_gate_up_grouped_probe" if probes else "expert_gate_up_grouped", xdtype)
    _args(*_grouped_specs(slots_base, slot_stride, num_slots, layout, x, M, slot_ids, K, M * H, out, M * K * I,
                          workspace, workspace_bytes, xdtype),
          ("gate_probe", gate_probe, "float32", M * K * I), ("up_probe", up_probe, "float32", M * K * I))
    lay = layout_c(layout)
    if not probes:
        st = fn(_ptr(slots_base), slot_stride, num_slots, ctypes.byref(lay), _ptr(x), M, _ptr(slot_ids), K, H, I,
                _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream))
    else:
        st = fn(_ptr(slots_base), slot_stride, num_slots, ctypes.byref(lay), _ptr(x), M, _ptr(slot_ids), K, H, I,
                _ptr(out), _ptr(gate_probe), _ptr(up_probe), _ptr(workspace), workspace_bytes, _stream(stream))
    _check(st)


def expert_gate_up_grouped_noalloc(slots_base, slot_stride: int, num_slots: int, layout, x, M: int, slot_ids,
                                   K: int, H: int, I: int, out, invalid_count=None, stream=None) -> None:
    """Enqueue the grouped call on the library's static scratch (see
    q4_expert_gate_up_grouped_noalloc in include/q4moe.h): no workspace, no
    device allocation; ``invalid_count`` (int32 device tensor or None)
    receives the number of out-of-range ids."""
    lib = load()
    _args(_slots_spec("slots_base", slots_base, num_slots, slot_stride, layout), ("x", x, "bfloat16", M * H),
          ("slot_ids", slot_ids, "int32", M * K), ("out", out, "bfloat16", M * K * I),
          ("invalid_count", invalid_count, "int32", 1))
    lay = layout_c(layout)
    _check(lib.q4_expert_gate_up_grouped_noalloc(_ptr(slots_base), slot_stride, num_slots, ctypes.byref(lay), _ptr(x),
                                                 M, _ptr(slot_ids), K, H, I, _ptr(out), _ptr(invalid_count),
                                                 _stream(stream)))


def validate_gate_up(slot, layout, x, M: int, H: int, I: int, out, fmt: str = "q4", xdtype: str = "bf16") -> int:
    """Host-only argument check; returns the status (0 or negative)."""
    lay = None if layout is None else layout_c(layout)
    return _fn(load(), fmt, "validate_gate_up", xdtype)(_ptr(slot), None if lay is None else ctypes.byref(lay), _ptr(x), M, H, I,
                                      _ptr(out))


def validate_grouped(slots_base, slot_stride, num_slots, layout, x, M, slot_ids, K, H, I, out, workspace,
                     workspace_bytes, fmt: str = "q4", xdtype: str = "bf16") -> int:
    lay = None if layout is None else layout_c(layout)
    return _fn(load(), fmt, "validate_grouped", xdtype)(_ptr(slots_base), slot_stride, num_slots,
                                      None if lay is None else ctypes.byref(lay), _ptr(x), M, _ptr(slot_ids), K,
                                      H, I, _ptr(out), _ptr(workspace), workspace_bytes)


def expert_down(slot, layout, mid, M: int, H: int, I: int, out, down_probe=None, stream=None, fmt: str = "q4",
                xdtype: str = "bf16") -> None:
    """Enqueue the down projection of one slot (see q4_expert_down in include/q4moe.h)."""
    lib = load()
    fn = _fn(lib, fmt, "expert_down" if down_probe is None else "expert_down_probe", xdtype)
    xt = _XDTYPE_NAMES[xdtype]
    _args(_slots_spec("slot", slot, 1, layout.slot_bytes, layout), ("mid", mid, xt, M * I), ("out", out, xt, M * H),
          ("down_probe", down_probe, "float32", M * H))
    lay = layout_c(layout)
    if down_probe is None:
        st = fn(_ptr(slot), ctypes.byref(lay), _ptr(mid), M, H, I, _ptr(out), _stream(stream))
    else:
        st = fn(_ptr(slot), ctypes.byref(lay), _ptr(mid), M, H, I, _ptr(out), _ptr(down_probe), _stream(stream))
    _check(st)


def expert_down_grouped(slots_base, slot_stride: int, num_slots: int, layout, mid, M: int, slot_ids, K: int,
                        H: int, I: int, out, workspace, workspace_bytes: int, down_probe=None,
                        stream=None, fmt: str = "q4", xdtype: str = "bf16") -> None:
    """Enqueue the grouped down projection (see q4_expert_down_grouped in include/q4moe.h)."""
    lib = load()
    fn = _fn(lib, fmt, "expert_down_grouped" if down_probe is None else "expert_down_grouped_probe", xdtype)
    _args(*_grouped_specs(slots_base, slot_stride, num_slots, layout, mid, M, slot_ids, K, M * K * I, out, M * K * H,
                          workspace, workspace_bytes, xdtype, in_name="mid"),
          ("down_probe", down_probe, "float32", M * K * H))
    lay = layout_c(layout)
    if down_probe is None:
        st = fn(_ptr(slots_base), slot_stride, num_slots, ctypes.byref(lay), _ptr(mid), M, _ptr(slot_ids), K, H, I,
                _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream))
    else:
        st = fn(_ptr(slots_base), slot_stride, num_slots, ctypes.byref(lay), _ptr(mid), M, _ptr(slot_ids), K, H, I,
                _ptr(out), _ptr(down_probe), _ptr(workspace), workspace_bytes, _stream(stream))
    _check(st)


def expert_forward(slot, layout, x, M: int, H: int, I: int, mid, out, stream=None, fmt: str = "q4",
                   xdtype: str = "bf16") -> None:
    """Enqueue the whole expert of one slot (see q4_expert_forward in include/q4moe.h)."""
    fn = _fn(load(), fmt, "expert_forward", xdtype)
    xt = _XDTYPE_NAMES[xdtype]
    _args(_slots_spec("slot", slot, 1, layout.slot_bytes, layout), ("x", x, xt, M * H), ("mid", mid, xt, M * I),
          ("out", out, xt, M * H))
    lay = layout_c(layout)
    _check(fn(_ptr(slot), ctypes.byref(lay), _ptr(x), M, H, I, _ptr(mid), _ptr(out), _stream(stream)))


def expert_forward_grouped(slots_base, slot_stride: int, num_slots: int, layout, x, M: int, slot_ids, K: int,
                           H: int, I: int, mid, out, workspace, workspace_bytes: int, stream=None, fmt: str = "q4",
                           xdtype: str = "bf16") -> None:
    """Enqueue the grouped whole expert (see q4_expert_forward_grouped in include/q4moe.h)."""
    fn = _fn(load(), fmt, "expert_forward_grouped", xdtype)
    _args(*_grouped_specs(slots_base, slot_stride, num_slots, layout, x, M, slot_ids, K, M * H, out, M * K * H,
                          workspace, workspace_bytes, xdtype),
          ("mid", mid, _XDTYPE_NAMES[xdtype], M * K * I))
    lay = layout_c(layout)
    _check(fn(_ptr(slots_base), slot_stride, num_slots, ctypes.byref(lay), _ptr(x), M, _ptr(slot_ids), K, H, I,
              _ptr(mid), _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)))


def validate_down(slot, layout, mid, M: int, H: int, I: int, out, fmt: str = "q4", xdtype: str = "bf16") -> int:
    """Host-only argument check of the down call; returns the status."""
    lay = None if layout is None else layout_c(layout)
    return _fn(load(), fmt, "validate_down", xdtype)(_ptr(slot), None if lay is None else ctypes.byref(lay), _ptr(mid), M, H, I,
                                   _ptr(out))


def validate_down_grouped(slots_base, slot_stride, num_slots, layout, mid, M, slot_ids, K, H, I, out, workspace,
                          workspace_bytes, fmt: str = "q4", xdtype: str = "bf16") -> int:
    lay = None if layout is None else layout_c(layout)
    return _fn(load(), fmt, "validate_down_grouped", xdtype)(_ptr(slots_base), slot_stride, num_slots,
                                           None if lay is None else ctypes.byref(lay), _ptr(mid), M,
                                           _ptr(slot_ids), K, H, I, _ptr(out), _ptr(workspace), workspace_bytes)


def stream_read(slots_base, slot_stride: int, num_slots: int, offset_a: int, offset_b: int, rows: int,
                row_bytes: int, sink, pattern: int = 0, waves: int = 8, depth: int = 4, stream=None) -> None:
    """Enqueue the read-only streaming kernel (see q4_stream_read in include/q4moe.h)."""
    _args(("slots_base", slots_base, "uint8", (num_slots - 1) * slot_stride + max(offset_a, offset_b) + rows * row_bytes),
          ("sink", sink, "int32", 1))
    _check(load().q4_stream_read(_ptr(slots_base), slot_stride, num_slots, offset_a, offset_b, rows, row_bytes,
                                 pattern, waves, depth, _ptr(sink), _stream(stream)))
