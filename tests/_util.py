"""Small helpers shared by the tests (no method arithmetic)."""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32_from_hex(vals):
    return np.array([int(v, 16) for v in vals], dtype=np.uint32).view(np.float32)


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def bf16_ordered(bits):
    """bf16 bit patterns mapped to integers that order like the values
    (+0 and -0 both map to 0), so |a - b| counts bf16 ulps between them."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_diff(a, b):
    return np.abs(bf16_ordered(a) - bf16_ordered(b))
