"""Planted mistakes in the CPU oracle must each fail at least one pin.

Every pin module checks the oracle against something other than itself
(rational brute force, closed forms, library conversions, invariants, a
hand-worked example).  This module shows that those pins would notice a
plausible slip: it rewrites one expression in one oracle function (a wrong
nibble order, a dropped zero point, a sign in the sigmoid, a dropped rounding
point, a transposed operand, ...), installs the rewritten function in the
oracle for the duration of the test, runs every pin of the four pin modules
against it, and asserts that at least one of them fails.

Each mistake is applied to the oracle only, on the CPU.
"""
import inspect
import textwrap
import warnings

import numpy as np
import pytest

import oracle
from oracle import q4_oracle
from tests import test_oracle_down_pins, test_oracle_f32_pins, test_oracle_pins, test_oracle_q8_pins

PIN_MODULES = (test_oracle_pins, test_oracle_down_pins, test_oracle_q8_pins, test_oracle_f32_pins)

# (name, oracle function, expression as written, planted mistake)
MUTANTS = [
    # nibble p of a word is weight 8w + p (page 52, GATE_UP_SOURCE's unpack)
    ("nibble_order_reversed", "q4_weights",
     "(words >> np.uint32(4 * p))", "(words >> np.uint32(4 * (7 - p)))"),
    # the zero point is 8
    ("zero_point_7", "q4_weights", "- np.int8(8)", "- np.int8(7)"),
    # Q8 weights are signed bytes
    ("q8_unsigned_bytes", "q8_weights", "dtype=np.int8", "dtype=np.uint8"),
    # bf16 rounding: ties to even (page 54, trellis_bf16)
    ("bf16_ties_away", "f32_to_bf16",
     "(d_hi == d_lo) & ((lo_bits & np.uint32(1)) == np.uint32(1))", "(d_hi == d_lo)"),
    ("bf16_truncates", "f32_to_bf16", "take_hi &= d_lo != 0.0", "take_hi &= False"),
    # F32 rounding of the scaled sum: ties to even
    ("f32_ties_away", "f32_round_dyadic", "(r == half and (m & 1))", "(r == half)"),
    ("f32_no_subnormals", "f32_round_dyadic", "max(top - 23, -149)", "top - 23"),
    # the scale multiplies the reduced sum
    ("scale_exponent_dropped", "scaled_f32", "exps[m] + se", "exps[m]"),
    ("scale_sign_dropped", "scaled_f32", "nums[i][m] * sn", "nums[i][m] * abs(sn)"),
    ("zero_takes_the_scale_sign_only", "scaled_f32",
     "zero_sign=s if nums[i][m] >= 0 else -s", "zero_sign=s"),
    # exact dot products
    ("limb_sign_dropped", "exact_dots",
     "np.where(d >= 0, left, right)) * sign", "np.where(d >= 0, left, right))"),
    ("limb_weight_wrong", "exact_dots", "(1 << (l * _LIMB_BITS))", "(1 << (l * (_LIMB_BITS - 1)))"),
    ("bf16_subnormal_exponent", "bf16_integer_parts",
     "np.where(ef == 0, 1, ef) - 127 - 7", "ef - 127 - 7"),
    ("bf16_hidden_bit_dropped", "bf16_integer_parts", "frac | 0x80", "frac"),
    ("f32_subnormal_exponent", "f32_integer_parts",
     "np.where(ef == 0, 1, ef) - 127 - 23", "ef - 127 - 23"),
    # the tail: sT = bf16(1 / (1 + exp(-gT))) in F32, five bf16 rounding points
    ("sigmoid_exp_sign", "swiglu_tail", "_exp_f32(-float(g))", "_exp_f32(float(g))"),
    ("sigmoid_one_minus", "swiglu_tail", "d = one + e", "d = one - e"),
    ("gate_rounding_dropped", "swiglu_tail",
     "gT = bf16_to_f32(f32_to_bf16(gate))", "gT = gate"),
    ("up_rounding_dropped", "swiglu_tail",
     "uT = bf16_to_f32(f32_to_bf16(up))", "uT = up"),
    ("sigmoid_rounding_dropped", "swiglu_tail",
     "sT = bf16_to_f32(f32_to_bf16(sig))", "sT = sig"),
    ("silu_rounding_dropped", "swiglu_tail",
     "siluT = bf16_to_f32(f32_to_bf16(gT * sT))", "siluT = gT * sT"),
    ("f32_tail_exp_sign", "swiglu_tail_f32", "_exp_f32(-float(g))", "_exp_f32(float(g))"),
    ("f32_tail_gate_times_up", "swiglu_tail_f32", "silu = gate * sig", "silu = gate"),
    # operands of the gate/up call
    ("gate_up_scales_swapped", "expert_gate_up",
     "sg = row_scales(slot, layout.gate_scale_offset, I)",
     "sg = row_scales(slot, layout.up_scale_offset, I)"),
    ("gate_up_tail_operands_swapped", "expert_gate_up",
     "swiglu_tail(gate, up)", "swiglu_tail(up, gate)"),
    # grouped call: invalid ids are counted
    ("invalid_ids_not_counted", "expert_gate_up_grouped", "invalid += 1", "invalid += 0"),
    # down projection (page 52, DOWN_SOURCE): row h of the down matrix is I/8 words
    ("down_matrix_transposed", "expert_down",
     "wd = decode_weights(slot, layout.down_weight_offset, H, I, fmt)",
     "wd = decode_weights(slot, layout.down_weight_offset, I, H, fmt).T"),
    ("down_output_unrounded", "expert_down",
     "f32_to_bf16(down) if xdtype", "f32_to_bf16(down.astype(np.float16)) if xdtype"),
    # grouped down: each routed pair reads its own mid row
    ("down_grouped_first_row", "expert_down_grouped",
     "np.stack([midbits[t, j] for t, j in pairs])", "np.stack([midbits[t, 0] for t, j in pairs])"),
]


def _pins():
    """Every pin of the pin modules as (name, zero-argument callable), slow ones left out."""
    out = []
    for mod in PIN_MODULES:
        for name, fn in sorted(vars(mod).items()):
            if not (name.startswith("test_") and inspect.isfunction(fn)):
                continue
            marks = getattr(fn, "pytestmark", [])
            if any(m.name == "slow" for m in marks):
                continue
            params = [m for m in marks if m.name == "parametrize"]
            if not params:
                out.append((f"{mod.__name__}.{name}", fn))
                continue
            argname, values = params[0].args
            for v in values:
                out.append((f"{mod.__name__}.{name}[{v}]", (lambda f, a, v: lambda: f(**{a: v}))(fn, argname, v)))
    return out


def _mutated(fname, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(q4_oracle, fname)))
    assert src.count(old) == 1, f"{fname}: expression to mutate found {src.count(old)} times"
    ns = dict(vars(q4_oracle))
    exec(compile(src.replace(old, new), f"<mutant of {fname}>", "exec"), ns)
    return ns[fname]


def _failing_pins(monkeypatch, fname, fn):
    monkeypatch.setattr(q4_oracle, fname, fn)
    if hasattr(oracle, fname):
        monkeypatch.setattr(oracle, fname, fn)
    failed = []
    with warnings.catch_warnings(), np.errstate(all="ignore"):
        warnings.simplefilter("ignore")
        for name, pin in _pins():
            try:
                pin()
            except (AssertionError, ValueError, IndexError, TypeError, ArithmeticError):
                failed.append(name)
            except pytest.skip.Exception:
                pass
    return failed


def test_pins_pass_on_the_unmutated_oracle(monkeypatch):
    fn = getattr(q4_oracle, "swiglu_tail")
    assert _failing_pins(monkeypatch, "swiglu_tail", fn) == []


def test_rewriting_without_a_change_keeps_every_pin_green(monkeypatch):
    # the rewrite machinery itself (re-compiling the source in the module's
    # namespace) does not change any result
    fn = _mutated("exact_dots", "* sign", "* sign")
    assert _failing_pins(monkeypatch, "exact_dots", fn) == []


@pytest.mark.parametrize("name,fname,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(monkeypatch, name, fname, old, new):
    fn = _mutated(fname, old, new)
    failed = _failing_pins(monkeypatch, fname, fn)
    assert failed, f"planted mistake {name} in {fname} passed every pin"
