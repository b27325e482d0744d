"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects invalid arguments with the documented status and message
(validation of page 52 validateCall / page 51 validateRange rules).  No GPU
is touched: only the host-only validators and pure queries are called."""
import ctypes
import os
import re

import pytest

import synth
import quantized_moe_expert_q4_amd as q4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(q[48]_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(q4.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 59, names
    for n in names:
        assert hasattr(lib, n), n
    assert q4.abi_version() == 5


def test_workspace_size_is_aligned_and_positive():
    for M, K, H, I, E in ((1, 1, 8, 1, 1), (32, 8, 6144, 2048, 64), (4096, 16, 7168, 4096, 65535)):
        b = q4.grouped_workspace_bytes(M, K, E)
        assert b >= 256 and b % 256 == 0
    assert q4.grouped_workspace_bytes(0, 1, 1) == 0
    assert q4.grouped_workspace_bytes(1, 1, 0) == 0


SLOT = 1 << 20           # fake, 4096-aligned "device" addresses: validation never dereferences them
X = 1 << 24
OUT = 1 << 26
IDS = 1 << 27
WS = 1 << 28


def _lay(H=4096, I=1536):
    return synth.contiguous_layout(H, I)


def _single(**kw):
    a = dict(slot=SLOT, layout=_lay(), x=X, M=1, H=4096, I=1536, out=OUT)
    a.update(kw)
    st = q4.validate_gate_up(a["slot"], a["layout"], a["x"], a["M"], a["H"], a["I"], a["out"])
    return st, q4.last_error()


def test_single_valid_arguments_pass():
    assert _single() == (0, "")


@pytest.mark.parametrize("kw,status,msg", [
    (dict(M=0), q4.Q4_ERR_INVALID_ARGUMENT, "requires input [M,H] with M >= 1"),
    (dict(H=0), q4.Q4_ERR_INVALID_ARGUMENT, "hidden size must be a positive integer"),
    (dict(I=0), q4.Q4_ERR_INVALID_ARGUMENT, "intermediate size must be a positive integer"),
    (dict(H=4100), q4.Q4_ERR_INVALID_ARGUMENT, "divisible by 8"),
    (dict(slot=0), q4.Q4_ERR_INVALID_ARGUMENT, "non-null"),
    (dict(slot=SLOT + 512), q4.Q4_ERR_ALIGNMENT, "page-aligned"),
    (dict(x=0), q4.Q4_ERR_INVALID_ARGUMENT, "input x"),
    (dict(x=X + 8), q4.Q4_ERR_ALIGNMENT, "16-byte"),
    (dict(out=0), q4.Q4_ERR_INVALID_ARGUMENT, "output"),
    (dict(out=OUT + 1), q4.Q4_ERR_ALIGNMENT, "2-byte"),
    (dict(layout=None), q4.Q4_ERR_INVALID_ARGUMENT, "layout"),
    (dict(H=65544, I=8, layout=synth.contiguous_layout(65544, 8)), q4.Q4_ERR_UNSUPPORTED, "65536"),
    (dict(M=70000), q4.Q4_ERR_UNSUPPORTED, "65535"),
    (dict(H=65536, I=65536, layout=synth.contiguous_layout(65536, 65536)), q4.Q4_ERR_UNSUPPORTED, "2^31"),
])
def test_single_rejections(kw, status, msg):
    st, err = _single(**kw)
    assert st == status, err
    assert msg in err


def _bad_layout(**kw):
    from dataclasses import replace
    return replace(_lay(), **kw)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(slot_bytes=0), q4.Q4_ERR_INVALID_ARGUMENT, "slot bytes"),
    (dict(gate_weight_offset=_lay().slot_bytes - 4096 * 1536 // 2 + 16), q4.Q4_ERR_RANGE, "gate weights exceeds the canonical expert slot"),
    (dict(up_weight_offset=(1 << 64) - 16), q4.Q4_ERR_RANGE, "up weights exceeds"),
    (dict(gate_scale_offset=_lay().slot_bytes - 4), q4.Q4_ERR_RANGE, "gate scales exceeds"),
    (dict(up_scale_offset=_lay().slot_bytes), q4.Q4_ERR_RANGE, "up scales exceeds"),
    (dict(down_weight_offset=_lay().slot_bytes - 16), q4.Q4_ERR_RANGE, "down weights exceeds"),
    (dict(down_scale_offset=_lay().slot_bytes - 8), q4.Q4_ERR_RANGE, "down scales exceeds"),
    (dict(gate_weight_offset=8, slot_bytes=_lay().slot_bytes + 4096), q4.Q4_ERR_ALIGNMENT, "multiples of 16"),
    (dict(up_scale_offset=_lay().up_scale_offset + 2, slot_bytes=_lay().slot_bytes + 4096), q4.Q4_ERR_ALIGNMENT,
     "multiples of 4"),
])
def test_layout_rejections(kw, status, msg):
    st, err = _single(layout=_bad_layout(**kw))
    assert st == status, err
    assert msg in err


def test_down_fields_in_range_are_accepted():
    lay = synth.contiguous_layout(4096, 1536)
    from dataclasses import replace
    lay = replace(lay, slot_bytes=lay.slot_bytes + 2 * 4096 * 1536 // 2 + 4 * 4096,
                  down_weight_offset=lay.slot_bytes, down_scale_offset=lay.slot_bytes + 4096 * 1536 // 2)
    assert _single(layout=lay)[0] == 0


def _grouped(**kw):
    lay = _lay(6144, 2048)
    a = dict(base=SLOT, stride=lay.slot_bytes, E=64, layout=lay, x=X, M=32, ids=IDS, K=8, H=6144, I=2048,
             out=OUT, ws=WS, wsb=q4.grouped_workspace_bytes(32, 8, 64))
    a.update(kw)
    st = q4.validate_grouped(a["base"], a["stride"], a["E"], a["layout"], a["x"], a["M"], a["ids"], a["K"], a["H"],
                             a["I"], a["out"], a["ws"], a["wsb"])
    return st, q4.last_error()


def test_grouped_valid_arguments_pass():
    assert _grouped() == (0, "")


@pytest.mark.parametrize("kw,status,msg", [
    (dict(K=0), q4.Q4_ERR_INVALID_ARGUMENT, "top-k"),
    (dict(E=0), q4.Q4_ERR_INVALID_ARGUMENT, "number of slots"),
    (dict(E=70000), q4.Q4_ERR_UNSUPPORTED, "65535 slots"),
    (dict(M=9000), q4.Q4_ERR_UNSUPPORTED, "routed pairs"),
    (dict(stride=12599296 + 100), q4.Q4_ERR_ALIGNMENT, "stride"),
    (dict(stride=4096), q4.Q4_ERR_RANGE, "stride is shorter"),
    (dict(base=SLOT + 64), q4.Q4_ERR_ALIGNMENT, "page-aligned"),
    (dict(ids=0), q4.Q4_ERR_INVALID_ARGUMENT, "slot ids"),
    (dict(ids=IDS + 2), q4.Q4_ERR_ALIGNMENT, "slot ids"),
    (dict(ws=0), q4.Q4_ERR_WORKSPACE, "workspace"),
    (dict(wsb=0), q4.Q4_ERR_WORKSPACE, "smaller"),
    (dict(ws=WS + 16), q4.Q4_ERR_ALIGNMENT, "workspace"),
    (dict(M=0), q4.Q4_ERR_INVALID_ARGUMENT, "M >= 1"),
])
def test_grouped_rejections(kw, status, msg):
    st, err = _grouped(**kw)
    assert st == status, err
    assert msg in err


def test_entry_points_reject_before_touching_the_device():
    # the enqueueing entry points run the same validation first; with invalid
    # arguments they return an error without any HIP call
    with pytest.raises(q4.Q4Error) as ei:
        q4.expert_gate_up(SLOT + 8, _lay(), X, 1, 4096, 1536, OUT, stream=0)
    assert ei.value.status == q4.Q4_ERR_ALIGNMENT
    with pytest.raises(q4.Q4Error) as ei:
        q4.expert_gate_up_grouped(SLOT, 4096, 1, _lay(), X, 1, IDS, 1, 4096, 1536, OUT, WS, 256, stream=0)
    assert ei.value.status == q4.Q4_ERR_RANGE


def test_noalloc_entry_point_rejects_before_touching_the_device():
    # sizes beyond the grouped limits, a misaligned count output and invalid
    # slots are rejected on the host before the static scratch is resolved
    with pytest.raises(q4.Q4Error) as ei:
        q4.expert_gate_up_grouped_noalloc(SLOT, 12599296, 64, _lay(), X, 9000, IDS, 8, 4096, 1536, OUT, stream=0)
    assert ei.value.status == q4.Q4_ERR_UNSUPPORTED and "routed pairs" in str(ei.value)
    lib = q4.load()
    st = lib.q4_expert_gate_up_grouped_noalloc(SLOT, 12599296, 64, ctypes.byref(q4._lib.layout_c(_lay())), X, 1,
                                               IDS, 8, 4096, 1536, OUT, WS + 2, 0)
    assert st == q4.Q4_ERR_ALIGNMENT and "invalid_count" in q4.last_error()
    with pytest.raises(q4.Q4Error) as ei:
        q4.expert_gate_up_grouped_noalloc(SLOT, 4096, 1, _lay(), X, 1, IDS, 1, 4096, 1536, OUT, stream=0)
    assert ei.value.status == q4.Q4_ERR_RANGE


# ---- down projection and whole expert (page 52 DOWN_SOURCE / validateCall) ----

def _down(**kw):
    a = dict(slot=SLOT, layout=synth.expert_layout(4096, 1536), mid=X, M=1, H=4096, I=1536, out=OUT)
    a.update(kw)
    st = q4.validate_down(a["slot"], a["layout"], a["mid"], a["M"], a["H"], a["I"], a["out"])
    return st, q4.last_error()


def test_down_valid_arguments_pass():
    assert _down() == (0, "")
    assert _down(M=65535) == (0, "")


def _shift_down(lay, dw=0, ds=0):
    from dataclasses import replace
    return replace(lay, down_weight_offset=lay.down_weight_offset + dw, down_scale_offset=lay.down_scale_offset + ds)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(I=1540, layout=synth.expert_layout(4096, 1540)), q4.Q4_ERR_INVALID_ARGUMENT, "divisible by 8"),
    (dict(layout=synth.contiguous_layout(4096, 1536)), q4.Q4_ERR_INVALID_ARGUMENT, "down weight and scale"),
    (dict(layout=_shift_down(synth.expert_layout(4096, 1536), dw=8)), q4.Q4_ERR_ALIGNMENT, "down weight offset"),
    (dict(layout=_shift_down(synth.expert_layout(4096, 1536), ds=-2)), q4.Q4_ERR_ALIGNMENT, "down scale offset"),
    (dict(layout=_shift_down(synth.expert_layout(4096, 1536), dw=1 << 24)), q4.Q4_ERR_RANGE,
     "down weights exceeds the canonical expert slot"),
    (dict(layout=_shift_down(synth.expert_layout(4096, 1536), ds=1 << 24)), q4.Q4_ERR_RANGE,
     "down scales exceeds the canonical expert slot"),
    (dict(mid=X + 8), q4.Q4_ERR_ALIGNMENT, "16-byte"),
    (dict(M=0), q4.Q4_ERR_INVALID_ARGUMENT, "M >= 1"),
    (dict(slot=SLOT + 4096 + 64), q4.Q4_ERR_ALIGNMENT, "page-aligned"),
])
def test_down_rejections(kw, status, msg):
    st, err = _down(**kw)
    assert st == status, err
    assert msg in err


def _down_grouped(**kw):
    lay = synth.expert_layout(6144, 2048)
    a = dict(base=SLOT, stride=lay.slot_bytes, E=64, layout=lay, mid=X, M=32, ids=IDS, K=8, H=6144, I=2048,
             out=OUT, ws=WS, wsb=q4.grouped_workspace_bytes(32, 8, 64))
    a.update(kw)
    st = q4.validate_down_grouped(a["base"], a["stride"], a["E"], a["layout"], a["mid"], a["M"], a["ids"], a["K"],
                                  a["H"], a["I"], a["out"], a["ws"], a["wsb"])
    return st, q4.last_error()


def test_down_grouped_valid_and_rejected():
    assert _down_grouped() == (0, "")
    st, err = _down_grouped(layout=synth.contiguous_layout(6144, 2048), stride=synth.contiguous_layout(6144, 2048).slot_bytes)
    assert st == q4.Q4_ERR_INVALID_ARGUMENT and "down" in err
    st, err = _down_grouped(M=65536, K=1, wsb=q4.grouped_workspace_bytes(65535, 1, 64))
    assert st == q4.Q4_ERR_UNSUPPORTED
    st, err = _down_grouped(wsb=0)
    assert st == q4.Q4_ERR_WORKSPACE


def test_down_and_forward_entry_points_reject_before_touching_the_device():
    lay = synth.expert_layout(4096, 1536)
    with pytest.raises(q4.Q4Error) as ei:
        q4.expert_down(SLOT + 8, lay, X, 1, 4096, 1536, OUT, stream=0)
    assert ei.value.status == q4.Q4_ERR_ALIGNMENT
    # forward validates both steps before enqueueing either: a gate/up-only layout fails
    with pytest.raises(q4.Q4Error) as ei:
        q4.expert_forward(SLOT, synth.contiguous_layout(4096, 1536), X, 1, 4096, 1536, X + (1 << 20), OUT, stream=0)
    assert ei.value.status == q4.Q4_ERR_INVALID_ARGUMENT
    with pytest.raises(q4.Q4Error) as ei:
        q4.expert_forward_grouped(SLOT, lay.slot_bytes, 2, lay, X, 1, IDS, 2, 4096, 1536, X + 8, OUT, WS, 256,
                                  stream=0)
    assert ei.value.status == q4.Q4_ERR_ALIGNMENT
    with pytest.raises(q4.Q4Error) as ei:
        q4.expert_down_grouped(SLOT, 4096, 1, lay, X, 1, IDS, 1, 4096, 1536, OUT, WS, 256, stream=0)
    assert ei.value.status == q4.Q4_ERR_RANGE


# ---- the Q8 family (page 52, Q8_GATE_UP_SOURCE / Glm52CanonicalQ8MetalExecutor) ----

def test_q8_validation_sizes_weights_one_per_byte():
    lay8 = synth.contiguous_layout(4096, 1536, fmt="q8")
    assert q4.validate_gate_up(SLOT, lay8, X, 1, 4096, 1536, OUT, fmt="q8") == 0
    # a Q4-sized slot is too short for int8 weights
    st = q4.validate_gate_up(SLOT, synth.contiguous_layout(4096, 1536), X, 1, 4096, 1536, OUT, fmt="q8")
    assert st == q4.Q4_ERR_RANGE and "exceeds the canonical expert slot" in q4.last_error()
    st = q4.validate_gate_up(SLOT, lay8, X, 1, 4100, 1536, OUT, fmt="q8")
    assert st == q4.Q4_ERR_INVALID_ARGUMENT and "Q8 expert dimensions" in q4.last_error()
    el8 = synth.expert_layout(4096, 1536, fmt="q8")
    assert q4.validate_down(SLOT, el8, X, 1, 4096, 1536, OUT, fmt="q8") == 0
    assert q4.validate_down_grouped(SLOT, el8.slot_bytes, 4, el8, X, 2, IDS, 2, 4096, 1536, OUT, WS, 256,
                                    fmt="q8") == 0
    assert q4.validate_grouped(SLOT, lay8.slot_bytes, 4, lay8, X, 2, IDS, 2, 4096, 1536, OUT, WS, 256,
                               fmt="q8") == 0
    # a projection above 2^31 - 16 bytes
    st = q4.validate_gate_up(SLOT, synth.contiguous_layout(65536, 32768, fmt="q8"), X, 1, 65536, 32768, OUT,
                             fmt="q8")
    assert st == q4.Q4_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        q4.validate_gate_up(SLOT, lay8, X, 1, 4096, 1536, OUT, fmt="q5")


# ---- f32 activations (page 52: validateCall accepts float32 input) ----

def test_f32_validation_and_output_alignment():
    lay = synth.contiguous_layout(4096, 1536)
    assert q4.validate_gate_up(SLOT, lay, X, 1, 4096, 1536, OUT, xdtype="f32") == 0
    assert q4.validate_gate_up(SLOT, lay, X, 1, 4096, 1536, OUT + 2) == 0          # bf16 output: 2-byte aligned
    st = q4.validate_gate_up(SLOT, lay, X, 1, 4096, 1536, OUT + 2, xdtype="f32")  # f32 output needs 4
    assert st == q4.Q4_ERR_ALIGNMENT and "4-byte" in q4.last_error()
    el = synth.expert_layout(4096, 1536)
    assert q4.validate_down(SLOT, el, X, 1, 4096, 1536, OUT, xdtype="f32") == 0
    assert q4.validate_down_grouped(SLOT, el.slot_bytes, 4, el, X, 2, IDS, 2, 4096, 1536, OUT, WS, 256,
                                    xdtype="f32") == 0
    with pytest.raises(ValueError):
        q4.validate_gate_up(SLOT, lay, X, 1, 4096, 1536, OUT, xdtype="f16")


def test_huge_top_k_is_rejected_before_the_pair_product():
    # K * M would wrap a signed 64-bit product; K alone is already out of range
    st, err = _grouped(M=4, K=1 << 62)
    assert st == q4.Q4_ERR_UNSUPPORTED, err
    assert "routed pairs" in err
    assert q4.grouped_workspace_bytes(4, 1 << 62, 64) == 0
    assert q4.grouped_workspace_bytes(1, 65537, 64) == 0


def test_stream_read_rejects_invalid_arguments_on_the_host():
    lib = q4.load()
    cases = [
        (dict(row_bytes=100), q4.Q4_ERR_INVALID_ARGUMENT),
        (dict(pattern=8), q4.Q4_ERR_INVALID_ARGUMENT),
        (dict(waves=4), q4.Q4_ERR_UNSUPPORTED),
        (dict(depth=8), q4.Q4_ERR_UNSUPPORTED),
        (dict(offset_a=8), q4.Q4_ERR_ALIGNMENT),
        (dict(offset_b=1 << 30), q4.Q4_ERR_RANGE),
        (dict(num_slots=0), q4.Q4_ERR_INVALID_ARGUMENT),
    ]
    for kw, status in cases:
        a = dict(base=SLOT, stride=6303744, num_slots=4, offset_a=0, offset_b=3145728, rows=1536, row_bytes=2048,
                 pattern=0, waves=8, depth=4, sink=WS)
        a.update(kw)
        st = lib.q4_stream_read(a["base"], a["stride"], a["num_slots"], a["offset_a"], a["offset_b"], a["rows"],
                                a["row_bytes"], a["pattern"], a["waves"], a["depth"], a["sink"], None)
        assert st == status, (kw, q4.last_error())


def test_binding_rejects_tensors_the_kernels_would_misread():
    """The binding checks dtype, contiguity, size and device of every tensor
    argument before the C call (CPU tensors: the device rule fires last)."""
    torch = pytest.importorskip("torch")
    lay = _lay(256, 128)
    H, I, M, K, E = 256, 128, 2, 2, 3
    slots = torch.zeros(E * lay.slot_bytes, dtype=torch.uint8)
    x = torch.zeros(M, H, dtype=torch.bfloat16)
    ids = torch.zeros(M, K, dtype=torch.int32)
    out = torch.zeros(M, K, I, dtype=torch.bfloat16)
    ws = torch.zeros(q4.grouped_workspace_bytes(M, K, E), dtype=torch.uint8)

    def call(**kw):
        a = dict(slots=slots, x=x, ids=ids, out=out, ws=ws, gate_probe=None, xdtype="bf16")
        a.update(kw)
        with pytest.raises(ValueError) as ei:
            q4.expert_gate_up_grouped(a["slots"], lay.slot_bytes, E, lay, a["x"], M, a["ids"], K, H, I, a["out"],
                                      a["ws"], ws.numel(), gate_probe=a["gate_probe"], xdtype=a["xdtype"])
        return str(ei.value)

    assert "slot_ids must be a int32" in call(ids=ids.to(torch.int64))
    assert "x must be a bfloat16" in call(x=x.float())
    assert "x must be a float32" in call(xdtype="f32")
    assert "out must be a bfloat16" in call(out=out.float())
    assert "gate_probe must be a float32" in call(gate_probe=torch.zeros(M, K, I, dtype=torch.bfloat16))
    assert "gate_probe holds" in call(gate_probe=torch.zeros(M * K * I - 1, dtype=torch.float32))
    assert "out holds" in call(out=out[:1])
    assert "x must be contiguous" in call(x=torch.zeros(H, M, dtype=torch.bfloat16).t())
    assert "slots_base holds" in call(slots=slots[:-1])
    assert "workspace holds" in call(ws=ws[:1])
    assert "must be a device (cuda) tensor" in call()
    # single-expert and down calls check their own shapes
    with pytest.raises(ValueError, match="out holds"):
        q4.expert_gate_up(slots, lay, x, M, H, I, torch.zeros(M * I - 1, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="mid must be a bfloat16"):
        q4.expert_down(slots, lay, torch.zeros(M, I, dtype=torch.float32), M, H, I, torch.zeros(M, H, dtype=torch.bfloat16))
