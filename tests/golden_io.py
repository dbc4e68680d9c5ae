"""Readers for the text fixtures under tests/golden/ (no arithmetic of the method)."""
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_magnitudes():
    """Fractions for codes 0..7 from the page's constants table."""
    mags = {}
    with open(os.path.join(GOLDEN, "e2m1_magnitudes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code, val = line.split()
            mags[int(code)] = Fraction(val)
    return [mags[i] for i in range(8)]


def e2m1_fraction(code):
    """Exact value of an E2M1 code from the golden table plus the sign bit 3."""
    v = e2m1_magnitudes()[code & 7]
    return -v if code & 8 else v


def hand_examples():
    out = []
    with open(os.path.join(GOLDEN, "hand_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, k, A, sfA, x, sfx, alpha, S, c = line.split()
            k = int(k)
            out.append(dict(
                name=name, k=k,
                A=np.frombuffer(bytes.fromhex(A), dtype=np.uint8).reshape(1, 1, k // 2),
                sfA=np.frombuffer(bytes.fromhex(sfA), dtype=np.uint8).reshape(1, 1, k // 16),
                x=np.frombuffer(bytes.fromhex(x), dtype=np.uint8).reshape(1, k // 2),
                sfx=np.frombuffer(bytes.fromhex(sfx), dtype=np.uint8).reshape(1, k // 16),
                alpha=np.array([float(alpha)], dtype=np.float32),
                S=Fraction(S), c=int(c, 16)))
    return out


def quant_examples():
    """Hand-derived one-block quantiser examples: dicts with name, rule, gs,
    values (float32 (16,)), sf (int) and packed (uint8 (8,))."""
    out = []
    with open(os.path.join(GOLDEN, "quant_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, rule, gs, vals, sf, packed = line.split()
            values = np.array([float(Fraction(v)) if v != "-0" else -0.0 for v in vals.split(",")],
                              dtype=np.float32)
            assert len(values) == 16
            out.append(dict(name=name, rule=rule, gs=np.float32(float(Fraction(gs))), values=values,
                            sf=int(sf, 16), packed=np.frombuffer(bytes.fromhex(packed), dtype=np.uint8)))
    return out
