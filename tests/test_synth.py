"""Seeded generator: determinism, ranges, counter-based access and bf16 rounding (CPU only)."""
from fractions import Fraction
import math
import struct

import numpy as np

import synth


def _exact_bf16_rne(v: float) -> int:
    """Reference RNE to bf16 by exact rational arithmetic over the neighbouring bf16 values."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    f = Fraction(v)
    sign = 0x8000 if f < 0 else 0
    a = abs(f)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)
    lo = (a // ulp) * ulp
    hi = lo + ulp
    if a - lo < hi - a:
        r = lo
    elif a - lo > hi - a:
        r = hi
    else:
        r = lo if ((lo / ulp) % 2 == 0) else hi
    bits = struct.unpack("<I", struct.pack("<f", float(r)))[0]
    assert bits & 0xFFFF == 0
    return sign | (bits >> 16)


def test_bf16_rne_matches_exact_rounding():
    L = synth.host_lib()
    rng = np.random.default_rng(0)
    vals = list(rng.uniform(-0.1, 0.1, 2000)) + list(rng.standard_normal(2000) * 0.02)
    # exact ties: midpoint between two neighbouring bf16 values (both parities)
    for base in (1.0, 1.0078125, 0.001953125, -0.0390625):
        ulp = 2.0 ** (math.floor(math.log2(abs(base))) - 7)
        vals += [base + ulp / 2, base + 1.5 * ulp, base - ulp / 4]
    for v in vals:
        assert L.bq_bf16_rne(float(v)) == _exact_bf16_rne(float(v)), v


def test_codes_determinism_and_range():
    w = synth.WORKLOADS["decode4"]
    k = synth.key(w, w.weight_family, 0, synth.T_CODES, 17, synth.GATE)
    a = synth.codes(k, 4, 100_000)
    b = synth.codes(k, 4, 100_000)
    assert np.array_equal(a, b)
    assert a.min() == 0 and a.max() == 15
    # counter-based: any window equals the same slice of the full stream
    assert np.array_equal(synth.codes(k, 4, 1000, start=54_321), a[54_321:55_321])
    # roughly uniform
    counts = np.bincount(a, minlength=16)
    assert counts.min() > 0.9 * len(a) / 16 and counts.max() < 1.1 * len(a) / 16
    c2 = synth.codes(k, 2, 64_000)
    assert c2.max() == 3 and np.bincount(c2).min() > 0.9 * 16_000


def test_streams_are_distinct():
    w = synth.WORKLOADS["decode4"]
    ks = {synth.key(w, w.weight_family, l, t, e, m) for l in (0, 1) for t in (4, 5, 6) for e in (-1, 0, 1)
          for m in (0, 1, 2)}
    assert len(ks) == 2 * 3 * 3 * 3


def test_uniform_ranges():
    for name in ("decode4", "decode2"):
        w = synth.WORKLOADS[name]
        s = synth.bf16_to_f32(synth.uniform_bf16(synth.key(w, 1, 0, synth.T_SCALE, 0, 0), *w.scale_range, 50_000))
        b = synth.bf16_to_f32(synth.uniform_bf16(synth.key(w, 1, 0, synth.T_BIAS, 0, 0), *w.bias_range, 50_000))
        # bf16 rounding can move an endpoint by half an ulp (2^-8 relative)
        assert s.min() >= w.scale_range[0] * (1 - 2 ** -8) and s.max() <= w.scale_range[1] * (1 + 2 ** -8)
        assert b.min() >= w.bias_range[0] * (1 + 2 ** -8) and b.max() <= w.bias_range[1] * (1 - 2 ** -8)
        assert abs(s.mean() - np.mean(w.scale_range)) < 0.02 * np.mean(w.scale_range)


def test_normals():
    w = synth.WORKLOADS["decode4"]
    x = synth.tokens_x(w, 0, 50)
    assert x.dtype == np.float32 and x.shape == (50, 4096)
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1.0) < 0.02
    # token t is independent of how many tokens are generated with it
    assert np.array_equal(synth.tokens_x(w, 7, 1)[0], x[7])
    R = synth.bf16_to_f32(synth.router_weights(w))
    assert R.shape == (512, 4096) and abs(R.std() - 0.02) < 0.0005
