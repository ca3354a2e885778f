"""Pins for the oracle's bf16 and OCP E4M3FN codecs.

The oracle's codecs are written from the format definitions.  They are
checked here against torch's CPU casts (library routines) and against the
closed-form structure of the formats.  torch's float32 -> float8_e4m3fn cast
does not saturate (magnitudes past the rounding range become NaN), so the
library comparison covers |v| <= 464 and saturation is pinned separately.
"""
import numpy as np
import pytest
import torch

import oracle


def torch_fp8_decode(codes):
    t = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return t.to(torch.float32).numpy()


def torch_fp8_encode(vals):
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_all_256_codes():
    ref = torch_fp8_decode(list(range(256)))
    for c in range(256):
        v = oracle.e4m3fn_decode(c)
        if c & 0x7F == 0x7F:
            assert np.isnan(v) and np.isnan(ref[c])
        else:
            assert v == float(ref[c]), c
    assert oracle.e4m3fn_decode(0x7E) == 448.0
    assert oracle.e4m3fn_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3fn_decode(0x08) == 2.0 ** -6


def test_encode_roundtrips_every_finite_code():
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        v = oracle.e4m3fn_decode(c)
        assert oracle.e4m3fn_encode(v) == c, hex(c)


def _adversarial_values():
    vals = []
    finite = sorted({oracle.e4m3fn_decode(c) for c in range(0x7F)})
    for a, b in zip(finite[:-1], finite[1:]):
        mid = (a + b) / 2
        for v in (mid, np.nextafter(np.float32(mid), np.float32(0)),
                  np.nextafter(np.float32(mid), np.float32(1e9)), a, b):
            vals.append(float(np.float32(v)))
    vals += [0.0, -0.0, 2.0 ** -10, 2.0 ** -11, 1e-30, 1.4e-45, 448.0, 456.0, 464.0,
             np.nextafter(np.float32(464.0), np.float32(0))]
    vals += [-v for v in vals]
    return np.array(vals, np.float32)


def test_encode_matches_torch_cast():
    rng = np.random.default_rng(0)
    rand = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 100,
        (rng.random(20000) * 464).astype(np.float32) * rng.choice([-1, 1], 20000),
        np.ldexp(rng.random(20000), rng.integers(-20, 9, 20000)).astype(np.float32),
    ])
    vals = np.concatenate([rand[np.abs(rand) <= 464], _adversarial_values()])
    ref = torch_fp8_encode(vals)
    got = np.array([oracle.e4m3fn_encode(float(v)) for v in vals], np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_encode_saturates():
    for v in (464.0001, 480.0, 500.0, 1e6, 3.0e38, float("inf")):
        assert oracle.e4m3fn_encode(v) == 0x7E
        assert oracle.e4m3fn_encode(-v) == 0xFE
    assert oracle.e4m3fn_encode(float("nan")) & 0x7F == 0x7F


def test_encode_rne_ties():
    # 1 + 1/16 lies halfway between 1 (mantissa 000) and 1.125 (001): even wins
    assert oracle.e4m3fn_encode(1.0625) == 0x38
    # 1.1875 lies between 1.125 (001) and 1.25 (010): even (010) wins
    assert oracle.e4m3fn_encode(1.1875) == 0x3A
    # halfway between 0 and the smallest subnormal rounds to +0
    assert oracle.e4m3fn_encode(2.0 ** -10) == 0x00
    assert oracle.e4m3fn_encode(3 * 2.0 ** -10) == 0x02


def test_bf16_codec_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 32, 50000, dtype=np.uint64).astype(np.uint32)
    # keep finite values, add halfway cases (low 16 bits == 0x8000)
    bits = bits[((bits >> 23) & 0xFF) != 0xFF]
    ties = (bits & 0xFFFF0000) | 0x8000
    allbits = np.concatenate([bits, ties, np.array([0, 0x80000000, 0x7F7FFFFF, 0x7F7F8000], np.uint32)])
    f = allbits.view(np.float32)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16_rne(float(v)) for v in f], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(hex(allbits[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


@pytest.mark.parametrize("b", [0x0000, 0x3F80, 0xBF80, 0x0001, 0x7F7F, 0xFF7F, 0x8001, 0x4049])
def test_bf16_decode(b):
    ref = torch.tensor([b], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float()[0]
    assert oracle.bf16_to_f32(b) == float(ref)
