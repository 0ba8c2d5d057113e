"""Pins of the oracle's MXFP8 activation quantisation (oracle/route_ref.py:
e4m3_code, mxfp8_quantize): hand-worked codes of the E4M3 format, torch's
own float8_e4m3fn conversion (a library routine) on every in-range
representable value and midpoint, and the closed forms of the E8M0 scale."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def test_hand_worked_codes():
    assert O.e4m3_code(1.0) == 0x38
    assert O.e4m3_code(448.0) == 0x7E and O.e4m3_code(-448.0) == 0xFE
    assert O.e4m3_code(1000.0) == 0x7E                 # saturates
    assert O.e4m3_code(2.0 ** -6) == 0x08               # smallest normal
    assert O.e4m3_code(2.0 ** -9) == 0x01               # smallest subnormal
    assert O.e4m3_code(0.0) == 0x00 and O.e4m3_code(-0.0) == 0x80
    assert O.e4m3_code(1.0625) == 0x38                  # tie -> even mantissa 0
    assert O.e4m3_code(1.1875) == 0x3A                  # tie -> even mantissa 2
    assert O.e4m3_code(2.0 ** -10) == 0x00              # tie below the smallest subnormal
    assert O.e4m3_code(3 * 2.0 ** -10) == 0x02          # tie -> even subnormal 2
    assert O.e4m3_code(464.0) == 0x7E                   # above the top: saturate


def _finite_codes():
    return [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_values_round_trip():
    for c in _finite_codes():
        assert O.e4m3_code(O.e4m3_value(c)) == c


def test_matches_torch_float8_e4m3fn():
    vals = sorted({O.e4m3_value(c) for c in _finite_codes()})
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    rng = np.random.default_rng(5)
    rand = list(rng.uniform(-448, 448, 4000)) + list(rng.standard_normal(4000) * 0.01)
    xs = np.array(vals + mids + rand, dtype=np.float32)   # all exact in binary32
    want = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_code(float(x)) for x in xs], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(xs[i]), int(got[i]), int(want[i])) for i in bad[:5]]


def _bits(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_scale_closed_forms():
    ones = _bits(np.ones((1, 32)))
    q, s = O.mxfp8_quantize(ones)
    assert s.tolist() == [[119]] and (q == 0x78).all()    # 1 = 256 * 2^-8
    zeros = _bits(np.zeros((1, 64)))
    q, s = O.mxfp8_quantize(zeros)
    assert s.tolist() == [[0, 0]] and (q == 0).all()
    blk = np.zeros((1, 32), np.float32)
    blk[0, 7] = -3.0                                      # amax 3: floor(log2 3) = 1
    q, s = O.mxfp8_quantize(_bits(blk))
    assert s.tolist() == [[127 + 1 - 8]] and q[0, 7] == O.e4m3_code(-3.0 * 2 ** 7)


def test_dequantisation_error_bound():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((3, 256)) * np.exp(rng.uniform(-20, 20, (3, 1)))).astype(np.float32)
    bits = _bits(x)
    v = O.bf16_bits_to_f64(bits)
    q, s = O.mxfp8_quantize(bits)
    for t in range(3):
        for b in range(8):
            shared = int(s[t, b]) - 127
            blk = v[t, 32 * b:32 * b + 32]
            assert shared == math.frexp(float(np.abs(blk).max()))[1] - 1 - 8
            for i in range(32):
                d = O.e4m3_value(int(q[t, 32 * b + i])) * 2.0 ** shared
                # half a quantum: 2^-4 relative in the normal range, else 2^(shared-10)
                assert abs(d - blk[i]) <= max(abs(blk[i]) * 2.0 ** -4, 2.0 ** (shared - 10))
