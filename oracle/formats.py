"""Decoding of the stored number formats to fp64, and the encoding of new
entries into them (test infrastructure only).

[架构详解 §4]: main KV is stored as MXFP4 (E2M1 elements with block scales)
and is dequantised before attention; SWA KV is FP8.  [架构详解 §1 config
table]: indexer K is 128-dim.  Two scale layouts of the E2M1 elements are
decoded: one E8M0 scale per 32 elements (OCP MX v1.0, the layout of the
benchmark workloads), and the page's own: one E4M3 scale per 16 channels and
no global scale ([架构详解 §4]; [4sapi, "FP4 and Bounded Replay"]).

Closed forms (OCP):
  bf16     : the upper 16 bits of an IEEE binary32.
  E4M3FN   : s=b>>7, e=(b>>3)&15, m=b&7; e==0 -> (-1)^s (m/8) 2^-6,
             else (-1)^s (1+m/8) 2^(e-7); S.1111.111 is NaN; no infinity.
  E2M1     : s=n>>3, e=(n>>1)&3, m=n&1; e==0 -> (-1)^s 0.5 m,
             else (-1)^s (1+m/2) 2^(e-1).
  E8M0     : 2^(x-127); x == 255 is NaN.
  MXFP4    : v[i] = E2M1(nib_i) * E8M0(scale[i // 32]); byte j holds
             element 2j in its low nibble and element 2j+1 in its high nibble.
  FP4/E4M3 : v[i] = E2M1(nib_i) * E4M3FN(scale[i // 16]), same nibble packing.
"""
import numpy as np


class FormatError(ValueError):
    """A NaN code appeared where the method stores only finite values."""


def bf16_to_f64(u16):
    """bf16 bit patterns (uint16 array) -> fp64, exactly."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


# bf16 keeps 8 significant bits (1 implicit + 7 stored) and binary32's
# exponent range: normal magnitudes 2^-126 .. (2 - 2^-7) 2^127, subnormal
# steps of 2^-133.
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def f64_to_bf16(x):
    """fp64 -> bf16 bit patterns, rounded once to the nearest bf16 value (a
    tie goes to the even significand); magnitudes past the largest finite
    value after rounding become infinities.  Inputs must not be NaN."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise FormatError("NaN to encode")
    mag = np.abs(x)
    # Quantum of the binade of |x| (the spacing of bf16 values there): 2^(e - 7)
    # with e = floor(log2 |x|), never below the subnormal step 2^-133.
    _, e = np.frexp(np.where(mag > 0, mag, 1.0))      # mag = f 2^e, 0.5 <= f < 1
    quantum = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    r = np.round(mag / quantum) * quantum              # np.round: ties to even
    r = np.where(r > _BF16_MAX, np.inf, r)
    r = np.where(np.signbit(x), -r, r)
    with np.errstate(over="ignore"):
        bits = r.astype(np.float32).view(np.uint32)    # exact: <= 8 significant bits
    return (bits >> 16).astype(np.uint16)


def _e4m3_value(b):
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        v = (m / 8.0) * 2.0 ** -6
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def _e2m1_value(n):
    s, e, m = n >> 3, (n >> 1) & 3, n & 1
    if e == 0:
        v = 0.5 * m
    else:
        v = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -v if s else v


# Per-code values computed once from the closed forms above.
E4M3_VALUES = np.array([_e4m3_value(b) for b in range(256)], dtype=np.float64)
E2M1_VALUES = np.array([_e2m1_value(n) for n in range(16)], dtype=np.float64)


def e4m3_to_f64(u8):
    """FP8 E4M3FN codes -> fp64; a NaN code raises FormatError."""
    u8 = np.asarray(u8, dtype=np.uint8)
    if np.any((u8 & 0x7F) == 0x7F):
        raise FormatError("FP8 E4M3FN NaN code in input")
    return E4M3_VALUES[u8]


def e2m1_to_f64(nib):
    """E2M1 nibbles (0..15) -> fp64."""
    return E2M1_VALUES[np.asarray(nib, dtype=np.uint8) & 0xF]


def e8m0_to_f64(u8):
    """E8M0 scale codes -> 2^(x-127); code 255 (NaN) raises FormatError."""
    u8 = np.asarray(u8, dtype=np.uint8)
    if np.any(u8 == 255):
        raise FormatError("E8M0 NaN code in input")
    return np.ldexp(1.0, u8.astype(np.int64) - 127)


def mxfp4_to_f64(fp4_bytes, scales):
    """MXFP4 entries -> fp64 vectors.

    fp4_bytes: uint8 [..., D/2]; scales: uint8 [..., D/32].  Returns [..., D].
    """
    b = np.asarray(fp4_bytes, dtype=np.uint8)
    sc = np.asarray(scales, dtype=np.uint8)
    d = b.shape[-1] * 2
    if sc.shape[-1] * 32 != d:
        raise ValueError("MXFP4: need one scale per 32 elements")
    nib = np.empty(b.shape[:-1] + (d,), dtype=np.uint8)
    nib[..., 0::2] = b & 0xF
    nib[..., 1::2] = b >> 4
    vals = e2m1_to_f64(nib)
    scale = np.repeat(e8m0_to_f64(sc), 32, axis=-1)
    return vals * scale


def fp4e4_to_f64(fp4_bytes, scales):
    """E2M1 entries with one E4M3FN scale per 16 elements -> fp64 vectors.

    fp4_bytes: uint8 [..., D/2]; scales: uint8 [..., D/16].  Returns [..., D].
    A NaN scale code raises FormatError.
    """
    b = np.asarray(fp4_bytes, dtype=np.uint8)
    sc = np.asarray(scales, dtype=np.uint8)
    d = b.shape[-1] * 2
    if sc.shape[-1] * 16 != d:
        raise ValueError("FP4/E4M3: need one scale per 16 elements")
    nib = np.empty(b.shape[:-1] + (d,), dtype=np.uint8)
    nib[..., 0::2] = b & 0xF
    nib[..., 1::2] = b >> 4
    return e2m1_to_f64(nib) * np.repeat(e4m3_to_f64(sc), 16, axis=-1)


# ---------------------------------------------------------------------------
# Encoding (the KV append step: [架构详解 §4] stores each new main-KV entry as
# MXFP4 and each SWA entry as FP8).  Plain nearest-value rounding on the code
# tables above, written from the OCP definitions:
#   E4M3FN : saturate to +-448 (the largest finite value), then the nearest
#            finite value, a tie going to the even code; the sign bit is kept
#            for values that round to zero (as an IEEE conversion does).
#   MXFP4  : per 32 elements the shared exponent X = floor(log2(amax)) - 2
#            (2 = the largest E2M1 exponent), clamped to [-127, 127], with
#            X = -127 for an all-zero block; the E8M0 code is X + 127.  Each
#            element v / 2^X goes to the nearest E2M1 magnitude, a tie going
#            to the even code, saturating at 6; a value that rounds to zero
#            is stored as +0.  Element 2j goes to the low nibble of byte j.
# Inputs must be finite.

def _nearest_code(mag, table):
    """Index of the nearest entry of an ascending table; ties to the even index."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.clip(np.searchsorted(table, mag, side="left"), 1, len(table) - 1)
    lo = hi - 1
    d_lo = mag - table[lo]
    d_hi = table[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


# Non-negative finite E4M3FN values (codes 0x00 .. 0x7E) ascend with the code.
_E4M3_POS = E4M3_VALUES[:0x7F]
_E2M1_POS = E2M1_VALUES[:8]


def f64_to_e4m3(x):
    """fp64 -> FP8 E4M3FN codes (saturating, round to nearest even)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise FormatError("non-finite value to encode")
    mag = np.minimum(np.abs(x), _E4M3_POS[-1])
    code = _nearest_code(mag, _E4M3_POS).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def f64_to_mxfp4(x):
    """fp64 [..., D] (D a multiple of 32) -> (uint8 [..., D/2] packed E2M1,
    uint8 [..., D/32] E8M0 codes)."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise FormatError("non-finite value to encode")
    d = x.shape[-1]
    if d % 32:
        raise ValueError("MXFP4: the last dimension must be a multiple of 32")
    blocks = x.reshape(x.shape[:-1] + (d // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    _, e = np.frexp(amax)                    # amax = m 2^e with m in [0.5, 1)
    xexp = np.clip(e - 1 - 2, -127, 127)
    xexp = np.where(amax > 0, xexp, -127)
    scaled = np.abs(blocks) / np.ldexp(1.0, xexp)[..., None]
    mag = _nearest_code(np.minimum(scaled, 6.0), _E2M1_POS).astype(np.uint8)
    nib = np.where((blocks < 0) & (mag > 0), mag | 8, mag).astype(np.uint8)
    nib = nib.reshape(x.shape)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, (xexp + 127).astype(np.uint8)


def f64_to_fp4e4(x):
    """fp64 [..., D] (D a multiple of 16) -> (uint8 [..., D/2] packed E2M1,
    uint8 [..., D/16] E4M3FN scale codes): the page's layout.

    Per 16 elements the scale is the E4M3FN value nearest to amax / 6 (6 =
    the largest E2M1 magnitude; ties to the even code, saturating at 448), so
    the block's largest element lands at the top of the E2M1 range.  Each
    element v goes to the E2M1 magnitude nearest to |v| / s (ties to the even
    code, saturating at 6), sign kept, a zero stored as +0; a block whose
    scale is 0 stores +0 everywhere.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise FormatError("non-finite value to encode")
    d = x.shape[-1]
    if d % 16:
        raise ValueError("FP4/E4M3: the last dimension must be a multiple of 16")
    blocks = x.reshape(x.shape[:-1] + (d // 16, 16))
    amax = np.abs(blocks).max(axis=-1)
    code = f64_to_e4m3(amax / 6.0)
    s = E4M3_VALUES[code]
    with np.errstate(divide="ignore", invalid="ignore"):
        scaled = np.where(s[..., None] > 0, np.abs(blocks) / s[..., None], 0.0)
    mag = _nearest_code(np.minimum(scaled, 6.0), _E2M1_POS).astype(np.uint8)
    nib = np.where((blocks < 0) & (mag > 0), mag | 8, mag).astype(np.uint8).reshape(x.shape)
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, code.astype(np.uint8)
