"""Pins of the oracle's number-format decoding (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import formats
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_e4m3_matches_torch_cast_all_codes():
    # Library routine: torch's float8_e4m3fn -> float64 conversion (OCP E4M3FN).
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = ~np.isnan(lib)
    assert set(np.nonzero(~finite)[0].tolist()) == {0x7F, 0xFF}
    np.testing.assert_array_equal(formats.e4m3_to_f64(codes[finite]), lib[finite])
    assert np.signbit(formats.e4m3_to_f64(np.array([0x80], np.uint8)))[0]


def test_e4m3_golden_and_nan_rejected():
    g = _gold("e3_fp8.json")
    for c in g["cases"]:
        assert formats.e4m3_to_f64(np.array([c["code"]], np.uint8))[0] == c["value"]
    for n in g["nan_codes"]:
        with pytest.raises(formats.FormatError):
            formats.e4m3_to_f64(np.array([n], np.uint8))


def test_e8m0_matches_torch_cast():
    codes = np.arange(255, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(formats.e8m0_to_f64(codes), lib)
    with pytest.raises(formats.FormatError):
        formats.e8m0_to_f64(np.array([255], np.uint8))


def test_e2m1_matches_ocp_value_listing():
    # OCP MX v1.0 lists the E2M1 magnitudes for codes 0..7 as below; codes
    # 8..15 are their negatives.
    listing = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = formats.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    np.testing.assert_array_equal(got[:8], listing)
    np.testing.assert_array_equal(got[8:], [-v for v in listing])


def test_mxfp4_golden_bytes():
    for c in _gold("e2_mxfp4.json")["cases"]:
        b = np.zeros(16, np.uint8)
        b[0] = c["byte"]
        sc = np.full(1, c["scale_code"], np.uint8)
        v = formats.mxfp4_to_f64(b, sc)
        np.testing.assert_array_equal(v[:2], c["elements"])
        assert np.signbit(v[0]) == np.signbit(c["elements"][0])


def test_mxfp4_scale_applies_per_32_elements():
    b = np.full(256, 0x22, np.uint8)            # every element 1.0
    sc = np.arange(120, 136, dtype=np.uint8)    # 16 different scales
    v = formats.mxfp4_to_f64(b, sc)
    for g in range(16):
        np.testing.assert_array_equal(v[32 * g:32 * g + 32], 2.0 ** (int(sc[g]) - 127))


def test_mxfp4_roundtrip_error_bound():
    # Decoding the independent encoder's bytes must give each input back to
    # within half a grid step of its binade (OCP MX rounding), or the
    # saturation error for |x / 2^X| > 6.
    x = torch.randn(64, 512, generator=torch.Generator().manual_seed(7), dtype=torch.float32)
    p, s = synth.to_mxfp4(x)
    dec = formats.mxfp4_to_f64(p.numpy(), s.numpy())
    xd = x.double().numpy()
    scale = np.repeat(formats.e8m0_to_f64(s.numpy()), 32, axis=-1)
    a = np.abs(xd) / scale
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    bound = np.where(a <= 6, step / 2, a - 6) * scale
    assert np.all(np.abs(dec - xd) <= bound + 1e-12)
    # The block maximum lands in the top binade [4, 8) before saturation.
    amax = np.abs(xd).reshape(64, 16, 32).max(-1)
    r = amax / formats.e8m0_to_f64(s.numpy())
    assert np.all((r >= 4) & (r < 8))


def test_bf16_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = formats.bf16_to_f64(bits)
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(got[ok], lib[ok])
    assert np.all(np.isnan(got[~ok]))


# ---------------------------------------------------------------- encoding
def test_e4m3_encode_round_trips_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(formats.f64_to_e4m3(formats.e4m3_to_f64(codes)), codes)


def test_e4m3_encode_matches_torch_cast():
    # Library routine: torch's float32 -> float8_e4m3fn cast rounds to nearest
    # even; it does not saturate, so inputs are clamped to +-448 first.  The
    # inputs are fp32 values (the path encodes bf16), so that no double
    # rounding through fp32 enters the library's result.
    rng = np.random.default_rng(5)
    vals = formats.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)          # exact ties
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.exp2(rng.integers(-12, 10, 20000)),
        mids, -mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
        np.array([0.0, -0.0, 448.0, 460.0, 1e6, -1e6]),
    ]).astype(np.float32).astype(np.float64)
    lib = torch.from_numpy(np.clip(x, -448.0, 448.0).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(formats.f64_to_e4m3(x), lib)


def test_mxfp4_encode_round_trips():
    # Codes whose block holds a magnitude 4 or 6 element encode back to
    # themselves (that element fixes the shared exponent).  -0 is excluded:
    # a zero is stored as +0.
    rng = np.random.default_rng(6)
    nib = rng.integers(0, 16, size=(40, 512)).astype(np.uint8)
    nib[nib == 8] = 0
    nib[:, ::32] = rng.choice(np.array([6, 7, 14, 15], np.uint8), size=(40, 16))
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(1, 255, size=(40, 16)).astype(np.uint8)
    p, s = formats.f64_to_mxfp4(formats.mxfp4_to_f64(packed, scales))
    np.testing.assert_array_equal(p, packed)
    np.testing.assert_array_equal(s, scales)


def test_mxfp4_encode_worked_block():
    # amax 6.5 -> shared exponent floor(log2 6.5) - 2 = 0 (code 127); every
    # E2M1 tie goes to the even code; 6.5 saturates at 6; -0.2 -> +0.
    x = np.zeros(32)
    x[:12] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, -0.2, -0.3, -6.0, 0.26]
    p, s = formats.f64_to_mxfp4(x)
    nib = np.empty(32, np.uint8)
    nib[0::2], nib[1::2] = p & 0xF, p >> 4
    assert s.tolist() == [127]
    assert nib[:12].tolist() == [0, 2, 2, 4, 4, 6, 6, 7, 0, 9, 15, 1]
    assert not nib[12:].any()
    # All-zero block: code 0, all nibbles +0.
    p, s = formats.f64_to_mxfp4(np.zeros(32))
    assert s.tolist() == [0] and not p.any()
    # Power-of-two amax: 2^k -> exponent k - 2.
    for k in (-100, -3, 0, 5, 100):
        _, s = formats.f64_to_mxfp4(np.full(32, np.ldexp(1.0, k)))
        assert s.tolist() == [k - 2 + 127]


def test_mxfp4_encode_matches_the_input_recipe():
    # The input generator quantises with threshold comparisons in torch, a
    # separate implementation of the same OCP rule.
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 512)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))
    x[3, 64:96] = 0.0
    x[5, :32] = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75], 32) * 4.0
    xb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32)
    p_ref, s_ref = synth.to_mxfp4(xb)
    p, s = formats.f64_to_mxfp4(xb.numpy().astype(np.float64))
    np.testing.assert_array_equal(p, p_ref.numpy())
    np.testing.assert_array_equal(s, s_ref.numpy())


# --------------------------------------------------------------------------- FP4 / E4M3 per 16
def test_fp4e4_golden_bytes():
    for c in _gold("e5_fp4_e4m3.json")["decode"]:
        b = np.zeros(8, np.uint8)
        b[0] = c["byte"]
        sc = np.full(1, c["scale_code"], np.uint8)
        np.testing.assert_array_equal(formats.fp4e4_to_f64(b, sc)[:2], c["elements"])


def test_fp4e4_decode_matches_torch_scale_cast():
    # Every finite E4M3 scale code, decoded by torch's float8_e4m3fn cast,
    # times the OCP E2M1 value listing, one scale per 16 elements.
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    sv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    table = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    rng = np.random.default_rng(15)
    nib = rng.integers(0, 16, size=(len(codes), 512)).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    sc = np.stack([np.roll(codes, i)[:32] for i in range(len(codes))])
    scv = np.stack([np.roll(sv, i)[:32] for i in range(len(codes))])
    want = table[nib] * np.repeat(scv, 16, axis=-1)
    np.testing.assert_array_equal(formats.fp4e4_to_f64(packed, sc), want)
    with pytest.raises(formats.FormatError):
        formats.fp4e4_to_f64(packed[:1], np.full((1, 32), 0x7F, np.uint8))


def test_fp4e4_encode_worked_block():
    g = _gold("e5_fp4_e4m3.json")["encode"]
    p, s = formats.f64_to_fp4e4(np.array(g["block"], np.float64))
    nib = np.empty(16, np.uint8)
    nib[0::2], nib[1::2] = p & 0xF, p >> 4
    assert s.tolist() == [g["scale_code"]] and nib.tolist() == g["nibbles"]
    # All-zero block and a block too small for any scale: everything +0.
    for x in (np.zeros(16), np.full(16, 1e-6)):
        p, s = formats.f64_to_fp4e4(x)
        assert not p.any() and s.tolist() == [0]


def test_fp4e4_encode_matches_the_input_recipe():
    # The input generator quantises with torch's float8 cast and threshold
    # comparisons, a separate implementation of the same rule.
    rng = np.random.default_rng(16)
    x = rng.standard_normal((64, 512)) * np.exp2(rng.integers(-14, 10, size=(64, 1)))
    x[2, 32:48] = 0.0
    x[4, :16] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 2) * 1.125
    xb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32)
    p_ref, s_ref = synth.to_fp4_e4m3(xb)
    p, s = formats.f64_to_fp4e4(xb.numpy().astype(np.float64))
    np.testing.assert_array_equal(p, p_ref.numpy())
    np.testing.assert_array_equal(s, s_ref.numpy())


def test_fp4e4_encode_error_bound():
    # Decoding gives each input back within half an E2M1 step of its block's
    # grid (times the scale), or the saturation error above 6 s.
    x = torch.randn(64, 512, generator=torch.Generator().manual_seed(17), dtype=torch.float64).numpy()
    p, s = formats.f64_to_fp4e4(x)
    dec = formats.fp4e4_to_f64(p, s)
    scale = np.repeat(formats.e4m3_to_f64(s), 16, axis=-1)
    a = np.abs(x) / scale
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    bound = np.where(a <= 6, step / 2, a - 6) * scale
    assert np.all(np.abs(dec - x) <= bound + 1e-12)


# ---------------------------------------------------------------- bf16 rounding

def _bf16_rne_exact(x):
    """Nearest bf16 value of a Python float by integer arithmetic on its
    significand (ties to the even significand), as a float; independent of
    the oracle's encoder."""
    import math
    if x == 0.0 or math.isinf(x):
        return x
    m, e = math.frexp(abs(x))                # |x| = m 2^e, 0.5 <= m < 1
    mant = int(m * (1 << 53))                # exact 53-bit integer
    # bf16 keeps 8 bits in the binade; subnormal below 2^-126 (e - 1 < -126).
    keep = 8 - max(0, -126 - (e - 1))
    drop = 53 - keep
    if drop <= 0:
        return x
    q, rem = divmod(mant, 1 << drop)
    half = 1 << (drop - 1)
    if rem > half or (rem == half and (q & 1)):
        q += 1
    v = math.ldexp(q, e - 53 + drop)
    if v > (2.0 - 2.0 ** -7) * 2.0 ** 127:
        v = math.inf
    return math.copysign(v, x)


def pin_bf16_encode(encode):
    """Worked values (ties, subnormals, overflow, a case where rounding
    through binary32 first would differ), agreement with torch's binary32 ->
    bf16 cast, and with the integer-arithmetic rounding on fp64 inputs."""
    cases = [(1.0, 0x3F80), (1.0 + 2.0 ** -8, 0x3F80), (1.0 + 3 * 2.0 ** -8, 0x3F82),
             (-(1.0 + 2.0 ** -8), 0xBF80), (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),
             (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81), (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000),
             (3 * 2.0 ** -134, 0x0002), (2.0 ** 128, 0x7F80), ((2.0 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),
             (-0.0, 0x8000), (0.0, 0x0000), (-3.0, 0xC040)]
    for x, bits in cases:
        if int(encode(np.array([x]))[0]) != bits:
            return False
    rng = np.random.default_rng(12)
    f32 = (rng.standard_normal(4096) * np.exp2(rng.integers(-140, 120, 4096))).astype(np.float32)
    lib = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if not np.array_equal(encode(f32.astype(np.float64)), lib):
        return False
    f64 = rng.standard_normal(4096) * np.exp2(rng.integers(-130, 100, 4096).astype(np.float64))
    got = formats.bf16_to_f64(encode(f64))
    want = np.array([_bf16_rne_exact(float(v)) for v in f64])
    return np.array_equal(got, want)


def test_bf16_encode():
    assert pin_bf16_encode(formats.f64_to_bf16)


def test_bf16_encode_round_trips_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    assert np.array_equal(formats.f64_to_bf16(formats.bf16_to_f64(bits[finite])), bits[finite])
