"""Number formats used by the layer, decoded from their bit-level definitions (fp64).

Test infrastructure only (see the package docstring).

* bf16: 1 sign, 8 exponent (bias 127), 7 mantissa bits.  ``bf16_round`` rounds a
  real value to the nearest bf16, ties to the even mantissa, with gradual
  underflow and overflow to infinity.  The layer rounds to bf16 wherever it
  stores a bf16 operand.
* E2M1 (the 4-bit element of NVFP4; orcarouter.ai English post, "Where the
  kernel boundary sits": experts stored in 4-bit NVFP4): bit 3 sign, bits 2:1
  exponent with bias 1, bit 0 mantissa; exponent 0 is subnormal (value m/2).
* E4M3 (OCP "FN" variant, the per-16-element NVFP4 block scale): bit 7 sign,
  bits 6:3 exponent with bias 7, bits 2:0 mantissa; exponent 0 is subnormal
  (m/8 * 2^-6); 0x7F/0xFF are NaN and there is no infinity.
* NVFP4 matrix [N, K]: codes [N, K/2] (even k in the low nibble), block scales
  [N, K/16] E4M3 (block = 16 consecutive k of one row), one fp32 tensor scale.
  Element value = E2M1(code) * E4M3(scale) * ts.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even), returned as fp64."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)                       # xf = m * 2**e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: quantum = 2**(floor(log2|x|) - 7) = 2**(e - 8);
    # below the smallest normal (2**-126) the quantum stays 2**-133
    q_exp = np.maximum(e - 8, -133)
    scaled = np.ldexp(xf, -q_exp)             # exact (power-of-two scaling)
    r = np.ldexp(np.round(scaled), q_exp)     # np.round: half to even
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, xf), r)
    out[finite] = r[finite]
    out[~finite] = x[~finite]
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e2m1_value(code) -> np.ndarray:
    code = np.asarray(code).astype(np.int64)
    sign = np.where(code & 0x8, -1.0, 1.0)
    e = (code >> 1) & 0x3
    m = code & 0x1
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, e - 1))
    return sign * mag


def e4m3_value(byte) -> np.ndarray:
    b = np.asarray(byte).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


_E2M1_TABLE = e2m1_value(np.arange(16))
_E4M3_TABLE = e4m3_value(np.arange(256))


def nvfp4_dequant(codes: np.ndarray, scales: np.ndarray, ts: float) -> np.ndarray:
    """codes uint8 [N, K/2], scales uint8 [N, K/16], ts -> fp64 [N, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    N, half = codes.shape
    K = 2 * half
    assert scales.shape == (N, K // 16), (scales.shape, N, K)
    vals = np.empty((N, K), dtype=np.float64)
    vals[:, 0::2] = _E2M1_TABLE[codes & 0x0F]
    vals[:, 1::2] = _E2M1_TABLE[codes >> 4]
    s = _E4M3_TABLE[scales]
    if np.isnan(s).any():
        raise ValueError("NaN E4M3 block scale")
    vals *= np.repeat(s, 16, axis=1)
    vals *= float(ts)
    return vals


# --------------------------------------------------------------------------------------------
# NVFP4 encoding of an activation (the down projection's input when it is gathered as fp4)
# --------------------------------------------------------------------------------------------
E4M3_MAX = 448.0
_E2M1_POS = _E2M1_TABLE[:8]          # codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6 (increasing)
_E4M3_POS = _E4M3_TABLE[:0x7F]       # codes 0..126: every finite non-negative value (increasing)


def nearest_code(mag, grid: np.ndarray) -> np.ndarray:
    """Code of the grid value nearest to each non-negative `mag` (codes are grid indices, the
    grid increasing); equal distances go to the even code.  Beyond the largest value the
    nearest is the largest: the rounding saturates."""
    mag = np.asarray(mag, dtype=np.float64)
    dist = np.abs(mag[..., None] - grid)
    cand = dist == dist.min(axis=-1, keepdims=True)
    n = grid.shape[0]
    first = np.argmax(cand, axis=-1)
    last = n - 1 - np.argmax(cand[..., ::-1], axis=-1)
    return np.where(first % 2 == 0, first, last)


def nvfp4_quantize(v, ts: float):
    """fp32 rows v [N, K] (K % 16 == 0) with fp32 tensor scale ts > 0 -> (codes uint8 [N, K]
    with the sign in bit 3, block scales uint8 [N, K/16]).

    Same format as the stored expert weights (E2M1 element, E4M3 scale per 16 consecutive
    elements, one fp32 tensor scale), encoded with the weights' own rule: the block scale is
    the E4M3 value nearest to amax_block / (6 ts), and each element the E2M1 value nearest to
    v / (scale ts), both ties to even and saturating (448, 6); a zero scale gives zero codes.
    Every step that decides a code is taken in fp32 (product, then quotient, each rounded),
    the precision the kernel computes them in.
    """
    v = np.asarray(v, dtype=np.float32)
    N, K = v.shape
    assert K % 16 == 0
    t32 = np.float32(ts)
    assert t32 > 0
    blk = v.reshape(N, K // 16, 16)
    amax = np.abs(blk).max(axis=-1)
    sd = amax / (np.float32(6.0) * t32)
    sd = np.minimum(sd, np.float32(E4M3_MAX))
    s_code = nearest_code(sd, _E4M3_POS)
    den = _E4M3_POS[s_code].astype(np.float32) * t32
    ok = den > 0
    x = np.where(ok[..., None], blk / np.where(ok, den, np.float32(1.0))[..., None], np.float32(0.0))
    m_code = nearest_code(np.minimum(np.abs(x), np.float32(6.0)), _E2M1_POS)
    codes = np.where((x < 0) & (m_code > 0), m_code | 8, m_code).astype(np.uint8)
    return codes.reshape(N, K), s_code.astype(np.uint8)


def nvfp4_values(codes, scales) -> np.ndarray:
    """E2M1(code) * E4M3(block scale), codes uint8 [N, K] (one per element), scales [N, K/16]
    -> fp64 [N, K] (exact; the tensor scale is not applied)."""
    codes = np.asarray(codes, dtype=np.uint8)
    s = _E4M3_TABLE[np.asarray(scales, dtype=np.uint8)]
    return _E2M1_TABLE[codes & 0x0F] * np.repeat(s, 16, axis=1)
