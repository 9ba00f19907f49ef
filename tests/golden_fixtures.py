"""Readers of the hand-worked fixtures under tests/golden/ (no arithmetic of
the method: they parse the stored values)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f32(hex_bits: str) -> np.float32:
    return np.array([int(hex_bits, 16)], np.uint32).view(np.float32)[0]


def global_scale_examples():
    """(amax, g, g_inv, fl(2688 / amax)) rows of global_scale_examples.txt."""
    rows = []
    for line in open(os.path.join(GOLDEN, "global_scale_examples.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        amax, g, gi, alt = [f.strip() for f in line.split("|")]
        rows.append((np.float32(amax), _f32(g), _f32(gi), _f32(alt)))
    return rows
