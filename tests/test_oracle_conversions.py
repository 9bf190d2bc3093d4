"""Oracle storage conversions pinned to library routines (exhaustive / edge cases)."""
import math
import struct
from fractions import Fraction

import numpy as np
import torch

import oracle


def test_fp8_e4m3_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        got = oracle.fp8_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == float(ref[c]), (c, got, ref[c])


def _edge_f32():
    pats = [0x00000000, 0x80000000, 0x00000001, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0xFF7FFFFF,
            0x7F800000, 0xFF800000, 0x3F808000, 0x3F818000, 0x3F80FFFF, 0x3F807FFF, 0x3F808001,
            0x7F7F8000, 0x7F7F7FFF, 0x00008000, 0x00018000, 0xBF808000, 0xBF818000]
    return [struct.unpack("<f", struct.pack("<I", p))[0] for p in pats]


def test_bf16_rounding_of_floats_matches_torch():
    rng = np.random.default_rng(0)
    vals = list(rng.standard_normal(20000).astype(np.float32))
    vals += list((rng.standard_normal(2000) * 1e-39).astype(np.float32))   # subnormals
    vals += list(rng.integers(0, 2**32, 5000, dtype=np.uint64).astype(np.uint32).view(np.float32))
    vals += _edge_f32()
    vals = [v for v in vals if not math.isnan(v)]
    ref = torch.tensor(np.array(vals, dtype=np.float32)).to(torch.bfloat16).view(torch.int16)
    ref = ref.numpy().view(np.uint16)
    got = np.array([oracle.bf16_bits(float(v)) for v in vals], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(vals[i], hex(got[i]), hex(ref[i])) for i in bad[:5]]


def _bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def test_bf16_rounding_of_doubles_is_nearest_even():
    """Brute force: the result is the nearest bf16 neighbour, ties to the even pattern.
    Inputs include doubles just off a bf16 tie, where float-then-bf16 double rounding errs."""
    rng = np.random.default_rng(1)
    xs = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000))
    for _ in range(2000):   # tie + tiny perturbation
        b = int(rng.integers(0x0080, 0x7F00)) | (int(rng.integers(0, 2)) << 15)
        lo, hi = _bf16_value(b), _bf16_value(b + 1)
        mid = (lo + hi) / 2.0
        xs += [mid, math.nextafter(mid, math.inf), math.nextafter(mid, -math.inf),
               mid + (hi - lo) * 2.0 ** -30]
    for x in xs:
        bits = oracle.bf16_bits(x)
        v = _bf16_value(bits)
        fx = Fraction(x)
        # neighbours of the result
        cands = [bits - 1, bits, bits + 1]
        dist = {c: abs(Fraction(_bf16_value(c & 0xFFFF)) - fx) for c in cands
                if not math.isinf(_bf16_value(c & 0xFFFF)) and not math.isnan(_bf16_value(c & 0xFFFF))}
        best = min(dist.values())
        assert dist[bits] == best, (x, hex(bits))
        winners = [c for c in dist if dist[c] == best]
        if len(winners) > 1:
            assert bits % 2 == 0, (x, hex(bits))
        assert math.copysign(1.0, v) == math.copysign(1.0, x) or v == 0.0


def test_f32_rounding_is_numpy_cast():
    rng = np.random.default_rng(2)
    xs = rng.standard_normal(5000) * 10.0 ** rng.integers(-40, 38, 5000)
    for x in xs:
        assert oracle.round_to("f32", float(x)) == float(np.float32(x))
