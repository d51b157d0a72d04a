"""Writes quant_division_blocks.json: activation blocks whose codes depend on
taking fp32(x / sx) as a correctly rounded division.

Every expected value is derived here with exact rational arithmetic
(fractions.Fraction) from the scheme's definition: sx = RN32(amax / 127),
q = clamp(round_half_even(RN32(x / sx)), -127, 127), where RN32 rounds a real
number to the nearest fp32 value, ties to even.  Nothing here calls the oracle
or the GPU library.  Each block is chosen so that at least one of three
plausible shortcuts gives different codes or a different scale:
  * x * RN32(1 / sx)       (a reciprocal multiply instead of the division),
  * RN32(amax * RN32(1/127)) as the scale,
  * x * RN32(127 / amax)   (the reciprocal scale in one step).
Run: python tests/golden/make_quant_division_blocks.py
"""
import json
import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def rn32(v: Fraction) -> Fraction:
    """v rounded to the nearest fp32 value, ties to even (normal range only)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2^e <= a < 2^(e+1); fp32 keeps 24 significant bits
    assert -126 <= e <= 127
    unit = Fraction(2) ** (e - 23)
    m = a / unit
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * unit


def rint_even(v: Fraction) -> int:
    lo = v.numerator // v.denominator
    rem = v - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return lo


def clamp(q):
    return max(-127, min(127, q))


def codes(xs, amax):
    sx = rn32(Fraction(amax) / 127)
    return sx, [clamp(rint_even(rn32(Fraction(x) / sx))) for x in xs]


def codes_reciprocal(xs, amax):
    sx = rn32(Fraction(amax) / 127)
    r = rn32(1 / sx)
    return sx, [clamp(rint_even(rn32(Fraction(x) * r))) for x in xs]


def codes_scale_by_reciprocal127(xs, amax):
    sx = rn32(Fraction(amax) * rn32(Fraction(1, 127)))
    return sx, [clamp(rint_even(rn32(Fraction(x) / sx))) for x in xs]


def codes_inverse_scale(xs, amax):
    sx = rn32(Fraction(amax) / 127)
    r = rn32(Fraction(127) / Fraction(amax))
    return sx, [clamp(rint_even(rn32(Fraction(x) * r))) for x in xs]


def fp16_grid_near(v: Fraction):
    """The fp16 values just below and above v (v positive, within fp16 normals)."""
    f = np.float16(float(v))
    return {float(np.nextafter(f, np.float16(0))), float(f), float(np.nextafter(f, np.float16(np.inf)))}


def near_tie_candidates(amax):
    """fp16 values x in (0, amax] that sit next to (k + 1/2) * sx."""
    sx = rn32(Fraction(amax) / 127)
    out = set()
    for k in range(127):
        for x in fp16_grid_near((k + Fraction(1, 2)) * sx):
            if 0 < x <= amax:
                out.add(x)
    return sorted(out)


def main():
    rng = np.random.default_rng(20261203)
    amaxes = [9.359375, 1999.0, 2.498046875, 343.25, 3.734375, 6.14453125, 180.5, 0.0123443603515625]
    blocks = []
    for amax in amaxes:
        sx = rn32(Fraction(amax) / 127)
        assert sx.numerator & (sx.numerator - 1) or sx.denominator & (sx.denominator - 1)  # not a power of two
        cands = near_tie_candidates(amax)
        _, good = codes(cands, amax)
        _, rcp = codes_reciprocal(cands, amax)
        _, inv = codes_inverse_scale(cands, amax)
        picked = [x for x, g, r, i in zip(cands, good, rcp, inv) if g != r or g != i]
        picked = picked[:12]
        # fill the block: the amax element (negated half the time), the picked
        # near-tie values with random signs, then random values below amax
        xs = [amax if rng.integers(2) else -amax]
        xs += [x if rng.integers(2) else -x for x in picked]
        while len(xs) < 32:
            v = float(np.float16(rng.uniform(-amax, amax)))
            xs.append(v)
        order = rng.permutation(32)
        xs = [xs[i] for i in order]
        assert all(float(np.float16(x)) == x for x in xs)
        sx, q = codes(xs, amax)
        _, q_rcp = codes_reciprocal(xs, amax)
        s_alt, q_alt = codes_scale_by_reciprocal127(xs, amax)
        _, q_inv = codes_inverse_scale(xs, amax)
        blocks.append({
            "name": f"amax_{amax}",
            "x": xs,
            "sx": float(sx),
            "q": q,
            "q_if_reciprocal_multiply": q_rcp,
            "q_if_scale_times_rcp127": q_alt,
            "sx_if_scale_times_rcp127": float(s_alt),
            "q_if_inverse_scale": q_inv,
        })
        assert float(sx) == sx  # sx is an fp32 value, exact in a Python float
    n_rcp = sum(b["q"] != b["q_if_reciprocal_multiply"] for b in blocks)
    n_inv = sum(b["q"] != b["q_if_inverse_scale"] for b in blocks)
    n_alt = sum(b["q"] != b["q_if_scale_times_rcp127"] or b["sx"] != b["sx_if_scale_times_rcp127"] for b in blocks)
    doc = {
        "about": ("Activation blocks with non-power-of-two scales whose codes depend on the division x / sx "
                  "being correctly rounded in fp32. Scheme: sx = fp32(max|x| / 127), q = clamp(round_half_even("
                  "fp32(x / sx)), -127, 127) (the pinned reading of in-kernel block-32 activation quantisation: "
                  "ML Drift explainer, tech.dede.sh, section 'Stage-aware optimization for large language models'). "
                  "Expected values derived with exact rational arithmetic by make_quant_division_blocks.py; the "
                  "q_if_* fields are what three shortcuts would give, kept to show that each block tells them apart."),
        "blocks_differing": {"reciprocal_multiply": n_rcp, "inverse_scale": n_inv, "scale_times_rcp127": n_alt},
        "blocks": blocks,
    }
    with open(os.path.join(HERE, "quant_division_blocks.json"), "w") as f:
        json.dump(doc, f, indent=1)
    print(doc["blocks_differing"])


if __name__ == "__main__":
    main()
