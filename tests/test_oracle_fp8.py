"""CPU tests of the FP8 oracle (oracle/fp8.py) against its pins, with
planted mistakes that some pin must catch."""

import types

import numpy as np
import pytest

from oracle import fp8 as F
from tests import oracle_pins_fp8 as pins


@pytest.mark.parametrize("check", pins.FP8_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(F)


def _mutant(**overrides):
    """A copy of oracle/fp8.py whose functions see `overrides` in place of
    the named globals (the real module is untouched)."""
    m = types.ModuleType("fp8_mutant")
    m.__dict__.update({k: v for k, v in F.__dict__.items() if not k.startswith("__")})
    m.__dict__["__builtins__"] = F.__dict__["__builtins__"]
    for name, obj in list(m.__dict__.items()):
        if isinstance(obj, types.FunctionType) and obj.__module__ == F.__name__:
            m.__dict__[name] = types.FunctionType(obj.__code__, m.__dict__, name,
                                                  obj.__defaults__, obj.__closure__)
    m.__dict__.update(overrides)
    return m


def _caught(mutant):
    for check in pins.FP8_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(mutant)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            return True
    return False


def _decode_bias8(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    e, m = (c >> 3) & 0xF, c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -10, (1.0 + m / 8.0) * 2.0 ** (e - 8.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return np.where(c & 0x80, -1.0, 1.0) * mag


def _encode_truncate(x):
    """Round toward zero instead of to nearest even."""
    x = np.asarray(x, dtype=np.float64)
    vals = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(x), 448.0)
    i = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, 0x7E).astype(np.uint8)
    return np.where(x < 0, i | np.uint8(0x80), i).astype(np.uint8)


def _encode_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    vals = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(vals, a), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    c = np.where(vals[hi] - a <= a - vals[lo], hi, lo).astype(np.uint8)
    return np.where(x < 0, c | np.uint8(0x80), c).astype(np.uint8)


def _encode_flush_subnormals(x):
    c = F.e4m3_encode_rne(x)
    return np.where((c & 0x78) == 0, c & np.uint8(0x80), c).astype(np.uint8)


def _rotate_unnormalised(x, signs):
    x = np.asarray(x, dtype=np.float64)
    return (x * np.asarray(signs)) @ F.sylvester_hadamard(x.shape[-1])


def _rotate_without_signs(x, signs):
    x = np.asarray(x, dtype=np.float64)
    return x @ F.sylvester_hadamard(x.shape[-1]) / np.sqrt(x.shape[-1])


def _dequantize_block32(codes, scales, block=32):
    return F.dequantize(codes, scales, block=32)


def _dequantize_heads_reversed(codes, scales, block=64):
    return F.dequantize(codes, np.asarray(scales)[:, ::-1], block)


def _dequantize_divides(codes, scales, block=64):
    return F.dequantize(codes, 1.0 / np.asarray(scales, np.float64), block)


def _quantize_block32(x, signs=None, block=64):
    return F.quantize_blocks(x, signs, block=32)


MUTATIONS = {
    "decode_bias_8": dict(e4m3_decode=_decode_bias8),
    "encode_truncates": dict(e4m3_encode_rne=_encode_truncate),
    "encode_ties_away": dict(e4m3_encode_rne=_encode_ties_away),
    "encode_flushes_subnormals": dict(e4m3_encode_rne=_encode_flush_subnormals),
    "rotation_unnormalised": dict(rotate=_rotate_unnormalised),
    "rotation_ignores_signs": dict(rotate=_rotate_without_signs),
    "dequantize_blocks_of_32": dict(dequantize=_dequantize_block32),
    "dequantize_heads_reversed": dict(dequantize=_dequantize_heads_reversed),
    "dequantize_divides_by_scale": dict(dequantize=_dequantize_divides),
    "quantize_blocks_of_32": dict(quantize_blocks=_quantize_block32),
    "p_headroom_8": dict(P_HEADROOM_LOG2=8.5),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name):
    assert _caught(_mutant(**MUTATIONS[name])), name


def test_mutant_harness_is_faithful():
    assert not _caught(_mutant())
