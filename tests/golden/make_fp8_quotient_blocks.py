"""Write fp8_quotient_blocks.json: 128-channel bf16 blocks whose E4M3 codes
depend on how the quotient x / scale is formed, with the codes that the
definition gives, derived in exact rational arithmetic.

The definition (the BF16-to-FP8 conversion inside dispatch, "Balancing and
Beyond: Communication-Centric Optimizations in Expert Parallelism" digest,
section 3.1; scale rule: block max |x| over 448, nearest-even, saturating):
    s = RNE32(amax / 448)          float32, correctly rounded
    q = RNE32(x / s)               float32, correctly rounded
    code = E4M3FN(clamp(q, +-448)) nearest-even
Rejected forms, which the blocks are chosen to tell apart from it:
    x * RNE32(448 / amax)          and          x * RNE32(1 / s).

Expected values come from fractions.Fraction (exact rationals, rounded to
float32 by hand below) and torch's float8_e4m3fn cast of the exact float32
quotient after the clamp (a library routine). The search for telling blocks
uses numpy float32 arithmetic only to pick candidates; nothing here calls the
oracle or the HIP library.

Run from the repository root:  python tests/golden/make_fp8_quotient_blocks.py
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "fp8_quotient_blocks.json")
SEED = 20261203


def bf16_value(b: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern."""
    sign = -1 if b & 0x8000 else 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    assert e != 0xFF
    if e == 0:
        return sign * Fraction(m, 1) * Fraction(2) ** (-133)
    return sign * Fraction(128 + m, 1) * Fraction(2) ** (e - 134)


def rne32(r: Fraction) -> Fraction:
    """r rounded to the nearest float32 value, ties to even (no overflow here)."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    r = abs(r)
    e = r.numerator.bit_length() - r.denominator.bit_length()   # 2^e <= r < 2^(e+2)
    if Fraction(2) ** e > r:
        e -= 1
    while Fraction(2) ** (e + 1) <= r:
        e += 1
    e = max(e, -126)                       # subnormals share the step of 2^-126
    step = Fraction(2) ** (e - 23)
    n = r / step
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    out = fl * step
    assert out < Fraction(2) ** 128
    return sign * out


def f32_bits(r: Fraction) -> int:
    """Bits of a float32 value given exactly (it must be representable)."""
    v = np.float32(float(r))               # exact: every float32 is a double
    assert Fraction(float(v)) == r
    return int(v.view(np.uint32))


def e4m3_codes(vals_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(vals_f32, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def exact_block(amax_bits: int, xs: list[int]) -> tuple[int, list[int]]:
    """Scale bits and the 128 codes of a block [amax, *xs] by the definition."""
    vals = [bf16_value(amax_bits)] + [bf16_value(b) for b in xs]
    a = max(abs(v) for v in vals)
    if a == 0:
        return 0, [0x80 if b & 0x8000 else 0x00 for b in [amax_bits] + xs]
    s = rne32(a / 448)
    # a quotient that is zero (x = +-0) or rounds to zero keeps the sign of x
    # (IEEE; s > 0), which an exact rational cannot carry
    q = np.array([float(rne32(v / s)) or (-0.0 if b & 0x8000 else 0.0)
                  for v, b in zip(vals, [amax_bits] + xs)], np.float32)
    return f32_bits(s), [int(c) for c in e4m3_codes(q)]


def _np_bf16(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def pick_blocks():
    rng = np.random.Generator(np.random.PCG64(SEED))
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        # amax bit patterns: normal blocks across many binades, blocks whose
        # scale is below 2^-100 (tiny amax) and whose scale is subnormal
        normal = rng.choice(np.arange(0x2000, 0x5F00), 44, replace=False)
        tiny = rng.choice(np.arange(0x0080, 0x0C80), 12, replace=False)   # 2^-126 .. 2^-103
        sub = rng.choice(np.arange(0x0001, 0x0080), 8, replace=False)     # bf16 subnormal amax
        blocks = []
        for ab in [int(v) for v in np.concatenate([normal, tiny, sub])]:
            a = _np_bf16(np.array([ab]))[0]
            s = np.float32(a) / np.float32(448.0)
            xb = np.arange(0, ab + 1, dtype=np.uint32)
            x = _np_bf16(xb)
            q = e4m3_codes(x / s)
            q1 = e4m3_codes(x * (np.float32(448.0) / a))
            q2 = e4m3_codes(x * (np.float32(1.0) / s))
            both = np.nonzero((q != q1) & (q != q2))[0]
            one = np.nonzero((q != q1) ^ (q != q2))[0]
            pick = list(rng.permutation(both)[:80]) + list(rng.permutation(one)[:40])
            pick = pick[:127]
            while len(pick) < 127:
                pick.append(int(rng.integers(0, ab + 1)))
            xs = [int(xb[i]) | (0x8000 if rng.random() < 0.5 else 0) for i in pick]
            amax_bits = ab | (0x8000 if rng.random() < 0.5 else 0)
            blocks.append((amax_bits, xs))
    return blocks


def alt_codes(amax_bits: int, xs: list[int]) -> tuple[list[int], list[int]]:
    """Codes of the two rejected quotient forms (numpy float32), for the record."""
    vals = _np_bf16(np.array([amax_bits] + xs, np.uint32))
    a = np.float32(np.abs(vals).max())
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        s = a / np.float32(448.0)
        q1 = e4m3_codes(vals * (np.float32(448.0) / a))
        q2 = e4m3_codes(vals * (np.float32(1.0) / s))
    return [int(c) for c in q1], [int(c) for c in q2]


def main():
    out = {
        "source": ("Balancing and Beyond (digest), section 3.1: BF16 activations converted to "
                   "FP8 inside dispatch; scale rule amax/448, nearest-even, saturating; "
                   "OCP E4M3FN"),
        "definition": "s = RNE32(amax/448); code = E4M3_RNE(clamp(RNE32(x/s), -448, 448))",
        "derivation": ("fractions.Fraction exact rationals rounded to float32 by hand; "
                       "torch float8_e4m3fn cast of the exact float32 quotient"),
        "generator": "tests/golden/make_fp8_quotient_blocks.py",
        "seed": SEED,
        "blocks": [],
    }
    for amax_bits, xs in pick_blocks():
        sbits, codes = exact_block(amax_bits, xs)
        a1, a2 = alt_codes(amax_bits, xs)
        out["blocks"].append({"bf16": [amax_bits] + xs, "scale_bits": sbits, "codes": codes,
                              "codes_mul_448_over_amax": a1, "codes_mul_reciprocal": a2})
    with open(OUT, "w") as f:
        json.dump(out, f, separators=(",", ":"))
        f.write("\n")
    n1 = sum(sum(c != d for c, d in zip(b["codes"], b["codes_mul_448_over_amax"])) for b in out["blocks"])
    n2 = sum(sum(c != d for c, d in zip(b["codes"], b["codes_mul_reciprocal"])) for b in out["blocks"])
    print(f"wrote {OUT}: {len(out['blocks'])} blocks; codes differing from x*(448/amax): {n1}, "
          f"from x*(1/s): {n2}")


if __name__ == "__main__":
    main()
