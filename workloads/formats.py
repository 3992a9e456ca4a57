"""Storage formats of the inputs: bf16 (round to nearest even), OCP fp8 e4m3,
OCP MXFP4 (32-element blocks of FP4 E2M1 sharing an E8M0 scale) and OCP
MXFP8 (32-element blocks of FP8 E4M3 sharing an E8M0 scale).

These are input-preparation encoders only.  The oracle and the GPU library
each decode the stored bytes with their own code.

Dtype codes match the C-ABI enum: 0 = fp32, 1 = bf16, 2 = fp8 e4m3 (OCP
"e4m3fn": bias 7, no infinities, max finite 448).
"""
import numpy as np

DT_F32, DT_BF16, DT_E4M3 = 0, 1, 2
_NAMES = {DT_F32: "f32", DT_BF16: "bf16", DT_E4M3: "e4m3"}


def dtype_name(dt):
    return _NAMES[dt]


def bf16_bits(a):
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def _e4m3_positive_table():
    """All non-negative finite e4m3 values, indexed by code 0..126."""
    vals = np.empty(127, dtype=np.float64)
    for code in range(127):
        e, mnt = code >> 3, code & 7
        vals[code] = (mnt / 8.0) * 2.0 ** -6 if e == 0 else (1 + mnt / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3_positive_table()
E4M3_MAX = 448.0


def e4m3_scale(a):
    """Per-tensor scale so that max|a| maps to the largest finite e4m3 (448)."""
    amax = float(np.max(np.abs(np.asarray(a, dtype=np.float64))))
    return amax / E4M3_MAX if amax > 0 else 1.0


def e4m3_encode(a, scale):
    """Encode a/scale to e4m3 codes (uint8): nearest value, ties to the even
    code, saturating at +-448 (never produces the NaN code)."""
    v = np.asarray(a, dtype=np.float64) / float(scale)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, mag, side="left")        # first value >= mag
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(v < 0, code | np.uint8(0x80), code).astype(np.uint8)
    # -0 is stored as +0 so that equal values have equal codes
    code = np.where(code == 0x80, np.uint8(0), code).astype(np.uint8)
    return code


# Non-negative FP4 E2M1 values by code 0..7 (exponent bias 1, one mantissa
# bit, code 1 subnormal).
_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def mxfp4_encode(a):
    """Quantise rows of C values (C a multiple of 32) to MXFP4: codes uint8
    [..., C/2] (element 2j in the low nibble of byte j) and E8M0 scales uint8
    [..., C/32], one per 32-element block.  The scale exponent is floor(log2(amax)) - 2 (the
    largest E2M1 exponent), so the block's largest value lands in [4, 8)
    before rounding; elements round to the nearest E2M1 value, ties to the
    even code, saturating at 6.  All-zero blocks get scale 2^0."""
    v = np.asarray(a, dtype=np.float64)
    C = v.shape[-1]
    if C % 32:
        raise ValueError("mxfp4 rows are whole 32-element blocks")
    lead = v.shape[:-1]
    blk = v.reshape(lead + (C // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0)
    ex = np.clip(ex, -127, 127).astype(np.int64)
    scales = (ex + 127).astype(np.uint8)
    mag = np.minimum(np.abs(blk) / np.ldexp(1.0, ex)[..., None], 6.0)
    hi = np.minimum(np.searchsorted(_E2M1_POS, mag, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = mag - _E2M1_POS[lo], _E2M1_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where((blk < 0) & (code != 0), code | np.uint8(8), code).astype(np.uint8)
    code = code.reshape(lead + (C,))
    packed = (code[..., 0::2] | (code[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(scales)


def mxfp8_encode(a):
    """Quantise rows of C values (C a multiple of 32) to MXFP8 with E4M3
    elements: codes uint8 [..., C] (one byte an element) and E8M0 scales
    uint8 [..., C/32], one per 32-element block.  The scale exponent is
    floor(log2(amax)) - 8 (the largest E4M3 exponent), so the block's largest
    value lands in [256, 512) before rounding; elements round to the nearest
    E4M3 value, ties to the even code, saturating at 448.  All-zero blocks
    get scale 2^0."""
    v = np.asarray(a, dtype=np.float64)
    C = v.shape[-1]
    if C % 32:
        raise ValueError("mxfp8 rows are whole 32-element blocks")
    lead = v.shape[:-1]
    blk = v.reshape(lead + (C // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, 0)
    ex = np.clip(ex, -127, 127).astype(np.int64)
    scales = (ex + 127).astype(np.uint8)
    codes = e4m3_encode(blk / np.ldexp(1.0, ex)[..., None], 1.0).reshape(lead + (C,))
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales)
