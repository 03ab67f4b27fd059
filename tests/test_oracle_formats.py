"""Pins of the oracle's number formats and scale-atom addressing.

Each check compares the oracle against something other than itself: torch's
own float8 dtypes (an independent implementation of E4M3fn and E8M0), the
OCP MX specification's E2M1 table (tests/golden/e2m1_values.txt), exact
rational arithmetic, closed forms, and the page's own description of the
scale-factor tensor as a permutation of a physical buffer
("GEMM + Amax (SM100)", Using JAX arrays / Input tensor SFA).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_decode_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double()
    for c in range(256):
        got = O.dec_e4m3(c)
        want = float(ref[c])
        if math.isnan(want):
            assert math.isnan(got), c
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), c
    assert O.dec_e4m3(0x7E) == 448.0 and O.dec_e4m3(0x01) == 2.0 ** -9


def test_e5m2_decode_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e5m2).double()
    for c in range(256):
        got = O.dec_e5m2(c)
        want = float(ref[c])
        if math.isnan(want):
            assert math.isnan(got), c
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), c
    assert O.dec_e5m2(0x7B) == 57344.0 and O.dec_e5m2(0x01) == 2.0 ** -16
    assert O.dec_e5m2(0x7C) == math.inf and O.dec_e5m2(0xFC) == -math.inf


def test_e8m0_decode_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).double()
    for b in range(256):
        got, want = O.dec_e8m0(b), float(ref[b])
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want, b


def test_e2m1_decode_matches_ocp_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        got = O.dec_e2m1(int(code))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_bf16_decode_matches_torch():
    bits = torch.arange(0, 65536, 7, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).double()
    for h, v in zip(bits.tolist(), ref.tolist()):
        got = O.dec_bf16(h & 0xFFFF)
        assert (math.isnan(v) and math.isnan(got)) or got == v


def test_e4m3_encode_roundtrip_every_finite_code():
    for c in range(256):
        v = O.dec_e4m3(c)
        if math.isnan(v):
            continue
        assert O.enc_e4m3(v) == c, hex(c)


def test_e4m3_encode_rne_matches_torch_in_range():
    # torch's float32 -> float8_e4m3fn conversion rounds to nearest even; in
    # range (|x| < 448 + half step) it must agree with the oracle exactly.
    g = torch.Generator().manual_seed(1)
    x = torch.cat([torch.randn(20000, generator=g) * s for s in (1e-3, 0.05, 1, 30, 150)])
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float()
    finite = codes[~torch.isnan(codes)].unique()
    mids = ((finite[1:] + finite[:-1]) / 2).double()
    x = torch.cat([x.double(), mids, -mids]).clamp(-447.9, 447.9)
    ref = x.float().to(torch.float8_e4m3fn).view(torch.uint8)
    for v, r in zip(x.tolist(), ref.tolist()):
        got = O.enc_e4m3(v)
        if r in (0x00, 0x80) and got in (0x00, 0x80):
            continue
        assert got == r, (v, hex(got), hex(r))


def test_e4m3_encode_ties_to_even_and_saturates():
    # 1.0 = 0x38, next is 1.125 = 0x39; midpoint 1.0625 -> even mantissa (0x38);
    # midpoint between 1.125 and 1.25 -> 1.25 (0x3A).
    assert O.enc_e4m3(1.0625) == 0x38
    assert O.enc_e4m3(1.1875) == 0x3A
    assert O.enc_e4m3(448.0) == 0x7E and O.enc_e4m3(464.0) == 0x7E and O.enc_e4m3(1e9) == 0x7E
    assert O.enc_e4m3(-1e9) == 0xFE
    # smallest subnormal 2^-9; half of it ties to zero (even)
    assert O.enc_e4m3(2.0 ** -9) == 0x01 and O.enc_e4m3(2.0 ** -10) in (0x00,)
    assert O.enc_e4m3(3 * 2.0 ** -10) == 0x02


def _nearest_bf16_bits(x: float) -> int:
    """Exact nearest-even bf16 of a double by enumeration of neighbours (Fraction)."""
    f32 = np.float32(x)
    base = int(np.array([f32], dtype=np.float32).view(np.uint32)[0]) >> 16
    cands = []
    for h in range(max(0, (base & 0x7FFF) - 2), min(0x7F80, (base & 0x7FFF) + 3)):
        h |= base & 0x8000
        v = float(np.array([h << 16], dtype=np.uint32).view(np.float32)[0])
        cands.append((abs(Fraction(v) - Fraction(x)), h & 1, h))
    cands.sort()
    return cands[0][2]


def test_bf16_rounding_single_step_from_fp64():
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000)])
    for x in xs:
        assert O.rne_bf16(float(x)) == _nearest_bf16_bits(float(x)), x
    # torch agrees on values that are already binary32 (one rounding either way)
    t = torch.from_numpy(xs.astype(np.float32))
    ref = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, r in zip(t.double().tolist(), ref.tolist()):
        assert O.rne_bf16(x) == r


def test_e8m0_ceil_closed_forms():
    for j in range(-127, 128):
        assert O.e8m0_ceil(2.0 ** j) == min(254, max(0, 127 + j))
    for j in range(-100, 100):
        assert O.e8m0_ceil(2.0 ** j * (1 + 2.0 ** -52)) == 128 + j
        assert O.e8m0_ceil(2.0 ** j * (1 - 2.0 ** -53)) == 127 + j
        assert O.e8m0_ceil(2.0 ** j * 1.5) == 128 + j
    assert O.e8m0_ceil(0.0) == 0 and O.e8m0_ceil(2.0 ** 200) == 254


@pytest.mark.parametrize("mn,k,l", [(128, 128, 1), (300, 96, 2), (256, 512, 3), (7, 32, 1)])
def test_sf_offset_is_the_pages_permutation(mn, k, l):
    """The page: logical (32,4,MN',4,K',L) == physical (L,MN',K',32,4,4).permute(3,4,1,5,2,0).

    numpy builds the physical buffer of byte indices, permutes it as the page
    says, and the logical coordinate of row r / k-block kb (row mode read
    first-mode-fastest: r = 32*r4 + r32 + 128*mt; kb = k4 + 4*kt) must hold
    the oracle's offset."""
    mnt, kbl = -(-mn // 128), -(-k // 32)
    kt = -(-kbl // 4)
    phys = np.arange(l * mnt * kt * 32 * 4 * 4).reshape(l, mnt, kt, 32, 4, 4)
    logical = phys.transpose(3, 4, 1, 5, 2, 0)
    assert logical.shape == (32, 4, mnt, 4, kt, l)
    for li in range(l):
        for r in range(0, mnt * 128, 5):
            for kb in range(kt * 4):
                want = logical[r % 32, (r % 128) // 32, r // 128, kb % 4, kb // 4, li]
                assert O.sf_offset(r, kb, li, mn, kbl) == want


def test_sf_offset_bijective_and_row_words_contiguous():
    mn, k, l = 256, 256, 2
    kbl = k // 32
    seen = set()
    for li in range(l):
        for r in range(mn):
            offs = [O.sf_offset(r, kb, li, mn, kbl) for kb in range(kbl)]
            seen.update(offs)
            # the four scales of one row within a 128-wide K step share one 32-bit word
            for kt in range(kbl // 4):
                w = offs[4 * kt:4 * kt + 4]
                assert w == list(range(w[0], w[0] + 4)) and w[0] % 4 == 0
    assert seen == set(range(l * 2 * 2 * 512))


def test_e5m2_encode_roundtrip_every_finite_code():
    for c in range(256):
        v = O.dec_e5m2(c)
        if math.isnan(v) or math.isinf(v):
            continue
        assert O.enc_e5m2(v) == c, hex(c)


def test_e5m2_encode_rne_matches_torch_in_range():
    # In range (|x| <= 57344) torch's float32 -> float8_e5m2 conversion rounds
    # to nearest even, so the oracle must agree with it exactly.
    g = torch.Generator().manual_seed(2)
    x = torch.cat([torch.randn(20000, generator=g) * s for s in (1e-5, 1e-2, 1, 300, 9000)])
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e5m2).float()
    finite = codes[torch.isfinite(codes)].unique()
    mids = ((finite[1:] + finite[:-1]) / 2).double()
    x = torch.cat([x.double(), mids, -mids]).clamp(-57344.0, 57344.0)
    ref = x.float().to(torch.float8_e5m2).view(torch.uint8)
    for v, r in zip(x.tolist(), ref.tolist()):
        got = O.enc_e5m2(v)
        if r in (0x00, 0x80) and got in (0x00, 0x80):
            continue
        assert got == r, (v, hex(got), hex(r))


def test_e5m2_encode_ties_saturation_and_subnormals():
    # 1.0 = 0x3C, next 1.25 = 0x3D; midpoint 1.125 ties to the even mantissa (0x3C),
    # midpoint 1.375 rounds up to 1.5 (0x3E).
    assert O.enc_e5m2(1.125) == 0x3C and O.enc_e5m2(1.375) == 0x3E
    # the largest finite value 57344 = 0x7B; anything larger saturates to it, never Inf
    assert O.enc_e5m2(57344.0) == 0x7B and O.enc_e5m2(61440.0) == 0x7B
    assert O.enc_e5m2(1e30) == 0x7B and O.enc_e5m2(-1e30) == 0xFB
    # smallest subnormal 2^-16; half of it ties to zero (even), 3/2 of it to 2^-15
    assert O.enc_e5m2(2.0 ** -16) == 0x01 and O.enc_e5m2(2.0 ** -17) == 0x00
    assert O.enc_e5m2(3 * 2.0 ** -17) == 0x02


def test_e2m1_encode_roundtrip_ties_and_saturation():
    # every code round-trips (the negative zero code 0x8 decodes to -0.0)
    for c in range(16):
        assert O.enc_e2m1(O.dec_e2m1(c)) == c, hex(c)
    # midpoints tie to the even mantissa: 0.25->0, 0.75->1.0, 1.25->1.0,
    # 1.75->2, 2.5->2, 3.5->4, 5->4; just past a midpoint rounds up
    for v, c in [(0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4), (3.5, 0x6), (5.0, 0x6),
                 (0.2500001, 0x1), (1.2500001, 0x3), (2.5000001, 0x5), (5.0000001, 0x7)]:
        assert O.enc_e2m1(v) == c, (v, c)
        assert O.enc_e2m1(-v) == c | 0x8, (-v, c)
    # saturation at 6, never past it
    assert O.enc_e2m1(6.0) == 0x7 and O.enc_e2m1(7.9) == 0x7 and O.enc_e2m1(1e30) == 0x7
    assert O.enc_e2m1(-1e30) == 0xF


def test_e2m1_encode_is_nearest_by_brute_force():
    # against the decode table: the encoded magnitude is never farther from x
    # than any other code's
    mags = [O.dec_e2m1(c) for c in range(8)]
    rng = np.random.default_rng(11)
    for x in np.concatenate([rng.uniform(-7, 7, 4000), rng.uniform(-0.6, 0.6, 1000)]):
        got = O.dec_e2m1(O.enc_e2m1(float(x)))
        best = min(abs(m - min(abs(x), 6.0)) for m in mags)
        assert abs(abs(got) - min(abs(x), 6.0)) == best, x
        assert got == 0.0 or math.copysign(1, got) == math.copysign(1, x)
