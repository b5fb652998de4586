"""Pins of the oracle's number formats (CPU only).

Each check compares the oracle against something other than itself: an exact
closed form written with Python fractions, hand-decoded fixtures under
tests/golden/, or a library rounding routine (torch's fp32 -> bf16 cast).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats
from moe_layer_persistent_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _exact_minifloat(bits: int, ebits: int, mbits: int, bias: int) -> Fraction:
    """sign * 2^(E - bias) * (1 + M / 2^mbits), subnormal 2^(1 - bias) * M / 2^mbits."""
    sign = -1 if (bits >> (ebits + mbits)) & 1 else 1
    E = (bits >> mbits) & ((1 << ebits) - 1)
    M = bits & ((1 << mbits) - 1)
    if E == 0:
        return sign * Fraction(2) ** (1 - bias) * Fraction(M, 1 << mbits)
    return sign * Fraction(2) ** (E - bias) * (1 + Fraction(M, 1 << mbits))


def test_e2m1_exhaustive_closed_form():
    got = formats.e2m1_value(np.arange(16))
    for c in range(16):
        assert Fraction(got[c]) == _exact_minifloat(c, 2, 1, 1), c
    assert sorted(set(np.abs(got))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e4m3_exhaustive_closed_form():
    got = formats.e4m3_value(np.arange(256))
    for b in range(256):
        if b & 0x7F == 0x7F:
            assert np.isnan(got[b])
            continue
        assert Fraction(got[b]) == _exact_minifloat(b, 4, 3, 7), hex(b)
    finite = got[~np.isnan(got)]
    assert finite.max() == 448.0 and np.min(np.abs(finite[finite != 0])) == 2.0 ** -9


def _read_kv(path):
    out = {}
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = vals
    return out


def test_e4m3_golden_points():
    for line in open(os.path.join(GOLDEN, "e4m3_points.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        b, v = line.split()
        got = formats.e4m3_value(int(b, 16))
        assert got == float(v) and np.signbit(got) == v.startswith("-"), (b, got, v)


def test_nvfp4_golden_row():
    g = _read_kv(os.path.join(GOLDEN, "nvfp4_row.txt"))
    codes = np.array([[int(v, 16) for v in g["codes"]]], dtype=np.uint8)
    scales = np.array([[int(v, 16) for v in g["scales"]]], dtype=np.uint8)
    want = np.array([float(v) for v in g["values"]])
    got = formats.nvfp4_dequant(codes, scales, float(g["ts"][0]))[0]
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(np.signbit(got), [v.startswith("-") for v in g["values"]])


def test_nvfp4_dequant_blockwise_route():
    """Dequantise-then-dot equals sum over blocks of scale * (codes . x), times ts."""
    rng = np.random.default_rng(3)
    N, K = 7, 96
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7E, size=(N, K // 16), dtype=np.uint8)
    ts = 0.0123
    x = rng.standard_normal(K)
    full = formats.nvfp4_dequant(codes, scales, ts) @ x
    e2m1 = [float(_exact_minifloat(c, 2, 1, 1)) for c in range(16)]
    e4m3 = [float(_exact_minifloat(b, 4, 3, 7)) for b in range(256)]
    for n in range(N):
        acc = 0.0
        for blk in range(K // 16):
            part = 0.0
            for j in range(16):
                k = blk * 16 + j
                byte = int(codes[n, k // 2])
                c = byte & 15 if k % 2 == 0 else byte >> 4
                part += e2m1[c] * x[k]
            acc += e4m3[int(scales[n, blk])] * part
        assert abs(acc * ts - full[n]) <= 1e-12 * (1 + abs(full[n]))


def test_nvfp4_roundtrip_encoder_decoder():
    """encode(decode(c)) == c for every non-negative-zero code and in-range scale."""
    rng = np.random.default_rng(11)
    N, K = 64, 256
    ts = 2.0 ** -12
    codes = rng.integers(0, 16, size=(N, K))
    codes[codes == 8] = 0                    # -0 encodes as +0; compare values for it
    codes[:, ::16] = 7                       # every block holds a +6 so its amax fixes the scale
    scale_bytes = rng.integers(0x08, 0x7E, size=(N, K // 16))
    scale_bytes[0, 0] = 0x7E                 # global amax -> ts = amax / (6 * 448)
    vals = (formats.e2m1_value(codes) * np.repeat(formats.e4m3_value(scale_bytes), 16, axis=1) * ts)
    packed, s8, ts_enc = synth.encode_nvfp4(torch.tensor(vals, dtype=torch.float32))
    assert float(ts_enc) == ts
    np.testing.assert_array_equal(s8.numpy(), scale_bytes)
    want = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    np.testing.assert_array_equal(packed.numpy(), want)
    back = formats.nvfp4_dequant(packed.numpy(), s8.numpy(), float(ts_enc))
    np.testing.assert_array_equal(back, vals)


def test_bf16_round_matches_library_cast():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x3F808000, 0x3F818000, 0x3F80FFFF, 0x00008000, 0x00018000, 0x007FFFFF,
                        0x7F7FFFFF, 0x7F7F8000, 0xFF7F8000, 0x80000001, 0x00000000, 0x80000000,
                        0x3F7F8000, 0x3F7FC000], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = formats.bf16_round(f.astype(np.float64))
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all(), (f[~same][:5], got[~same][:5], want[~same][:5])
    np.testing.assert_array_equal(np.signbit(got), np.signbit(want))


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even mantissa (1.0)
    assert formats.bf16_round(1.0 + 2.0 ** -8) == 1.0
    assert formats.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # just above the tie rounds up
    assert formats.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    # a value only fp64 holds: the tie at 1 + 2^-8 exactly vs 1 + 2^-8 - 2^-40
    assert formats.bf16_round(1.0 + 2.0 ** -8 - 2.0 ** -40) == 1.0


# ---------------------------------------------------------------- NVFP4 encoding (fp4 gather)
def _grid_codes(table_fn, n):
    return [(c, _exact_minifloat(c, *table_fn)) for c in range(n)]


@pytest.mark.parametrize("fmt", ["e2m1", "e4m3"])
def test_nearest_code_exact_nearest_with_even_ties(fmt):
    """Every grid point, every midpoint (-> the even code), the fp32 neighbours of every
    midpoint (-> the nearer side) and values past the top (-> the top code), against the
    nearest point found with exact rational distances."""
    if fmt == "e2m1":
        grid, n = formats._E2M1_POS, 8
        exact = [_exact_minifloat(c, 2, 1, 1) for c in range(n)]
    else:
        grid, n = formats._E4M3_POS, 0x7F
        exact = [_exact_minifloat(c, 4, 3, 7) for c in range(n)]
    probes = []
    for c in range(n):
        probes.append(float(exact[c]))
        if c + 1 < n:
            mid = (exact[c] + exact[c + 1]) / 2
            m32 = np.float32(float(mid))
            assert Fraction(float(m32)) == mid        # every midpoint is an fp32 value
            probes += [float(m32), float(np.nextafter(m32, np.float32(0))),
                       float(np.nextafter(m32, np.float32(np.inf)))]
    top = float(exact[-1])
    probes += [top * 1.01, top * 4, 0.0]
    got = formats.nearest_code(np.array(probes), grid)
    for v, c in zip(probes, got):
        d = [abs(Fraction(v) - g) for g in exact]
        best = min(d)
        cands = [i for i in range(n) if d[i] == best]
        want = cands[0] if len(cands) == 1 else [i for i in cands if i % 2 == 0][0]
        assert c == want, (fmt, v, c, want)


def test_nvfp4_quantize_representable_blocks_are_unchanged():
    """Blocks built from E2M1 codes and an E4M3 scale, with one element at 6 * scale, encode to
    those codes and that scale (the scale rule amax / (6 ts) and the element rule v / (s ts))."""
    rng = np.random.default_rng(21)
    N, K = 24, 128
    ts = 2.0 ** -7                               # a power of two keeps every product exact in fp32
    codes = rng.integers(0, 16, size=(N, K))
    codes[codes == 8] = 0                        # -0 encodes as +0
    codes[:, ::16] = np.where(rng.random((N, K // 16)) < 0.5, 7, 15)   # +-6 fixes each block's amax
    scale_bytes = rng.integers(0x01, 0x7F, size=(N, K // 16))
    vals = formats.e2m1_value(codes) * np.repeat(formats.e4m3_value(scale_bytes), 16, axis=1) * ts
    v32 = vals.astype(np.float32)
    assert np.array_equal(v32.astype(np.float64), vals)
    c, s = formats.nvfp4_quantize(v32, ts)
    np.testing.assert_array_equal(s, scale_bytes)
    np.testing.assert_array_equal(c, codes)
    np.testing.assert_array_equal(formats.nvfp4_values(c, s) * ts, vals)


def test_nvfp4_quantize_matches_weight_encoder():
    """With the weights' own tensor scale (amax / (6 * 448)) the encoding is the one the
    synthetic weights are stored in, whose E4M3 rounding is torch's float8_e4m3fn cast."""
    rng = np.random.default_rng(8)
    for trial in range(4):
        w = (rng.standard_normal((48, 256)) * 10.0 ** rng.uniform(-3, 1)).astype(np.float32)
        w[3, 16:32] = 0.0                        # a zero block
        w[5, 40] = -w[5, 40]
        packed, s8, ts = synth.encode_nvfp4(torch.from_numpy(w))
        c, s = formats.nvfp4_quantize(w, float(ts))
        np.testing.assert_array_equal(s, s8.numpy())
        want = np.empty_like(c)
        want[:, 0::2] = packed.numpy() & 0x0F
        want[:, 1::2] = packed.numpy() >> 4
        np.testing.assert_array_equal(c, want)


def test_nvfp4_quantize_saturation_zero_and_sign():
    ts = 1.0
    v = np.zeros((1, 48), dtype=np.float32)
    v[0, 0:16] = np.linspace(-1.0, 1.0, 16)
    v[0, 5] = 1e6                                # block 0: amax / 6 far above 448 -> scale 448
    v[0, 16:32] = 0.0                            # block 1: zero -> scale 0, codes 0
    v[0, 32:48] = -np.float32(0.75)              # block 2: amax 0.75 -> scale 0.125, codes -6
    c, s = formats.nvfp4_quantize(v, ts)
    assert s[0, 0] == 0x7E and formats.e4m3_value(s[0, 0]) == 448.0
    assert c[0, 5] == 7                          # 1e6 / 448 saturates at +6
    assert np.all(c[0, [i for i in range(16) if i != 5]] == 0)   # |v| <= 1 is below 0.25 * 448
    assert s[0, 1] == 0 and np.all(c[0, 16:32] == 0)
    assert formats.e4m3_value(s[0, 2]) == 0.125 and np.all(c[0, 32:48] == 15)
    np.testing.assert_array_equal(formats.nvfp4_values(c, s)[0, 32:48], -0.75)
