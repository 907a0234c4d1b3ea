"""Pins for the oracle's element formats and block quantizers (CPU only).

Each check ties the oracle to something other than itself: values printed on
the pages (tests/golden), torch's own float8/bfloat16 conversions (an
independent library), closed forms of the scale rule, and brute-force nearest
searches over the decode tables.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- E2M1
def test_e2m1_decode_matches_printed_table():
    g = gold("e2m1_magnitudes.json")
    vals = [oracle.e2m1_value(c) for c in range(16)]
    assert sorted(set(abs(v) for v in vals)) == g["magnitudes"]
    assert vals[:8] == g["magnitudes"]                      # codes 0..7 ascend
    assert vals[8:] == [-m for m in g["magnitudes"]]        # sign bit is bit 3
    distinct = set(vals)
    assert len(distinct) == g["distinct_values_with_sign"]  # +0 and -0 coincide
    assert max(abs(v) for v in vals) == g["max_magnitude"]
    assert math.copysign(1.0, vals[8]) == -1.0              # code 8 is -0


def _nearest_even_bruteforce(a, table):
    """Nearest table entry; on a tie the entry with even index (mantissa bit 0)."""
    d = [abs(t - a) for t in table]
    best = min(d)
    cands = [i for i, x in enumerate(d) if x == best]
    if len(cands) > 1:
        cands = [i for i in cands if i % 2 == 0]
    return cands[0]


def test_e2m1_encode_bruteforce_and_midpoints():
    table = gold("e2m1_magnitudes.json")["magnitudes"]
    rng = np.random.default_rng(5)
    xs = list(rng.uniform(-8, 8, 4000)) + [m for m in table]
    mids = [(a + b) / 2 for a, b in zip(table[:-1], table[1:])]
    xs += mids + [-m for m in mids] + [6.5, 7.0, 100.0, -100.0, 1e-30, -1e-30, 0.0]
    for x in xs:
        code = oracle.e2m1_encode(x)
        mag = _nearest_even_bruteforce(abs(x), table)
        assert code == ((8 if math.copysign(1.0, x) < 0 else 0) | mag), x
    # documented midpoint outcomes (round half to even code)
    expect = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for x, v in expect.items():
        assert oracle.e2m1_value(oracle.e2m1_encode(x)) == v
    # every code round-trips (except -0 which re-encodes to itself too)
    for c in range(16):
        assert oracle.e2m1_encode(oracle.e2m1_value(c)) == c
    assert oracle.e2m1_encode(-0.1) == 8  # sign of zero kept


def test_e2m1_saturates_at_every_magnitude():
    """Every magnitude above the largest E2M1 value 6 encodes to 6 (code 7,
    sign in bit 3), up to the largest binary64 values and infinity."""
    for k in range(3, 1024):
        for m in (1.0, 1.5, 1.9999999):
            assert oracle.e2m1_encode(m * 2.0 ** k) == 7, (m, k)
            assert oracle.e2m1_encode(-m * 2.0 ** k) == 15, (m, k)
    assert oracle.e2m1_encode(math.inf) == 7 and oracle.e2m1_encode(-math.inf) == 15
    assert oracle.e2m1_encode(6.000001) == 7 and oracle.e2m1_encode(5.0) == 6  # 5 is the tie 4|6 -> even (4)


def test_e2m1_monotone():
    xs = np.linspace(-7, 7, 20001)
    vals = [oracle.e2m1_value(oracle.e2m1_encode(x)) for x in xs]
    assert all(a <= b for a, b in zip(vals, vals[1:]))


# --------------------------------------------------------------------------- E4M3
def test_e4m3_decode_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(mine) == nan).all()
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert (mine[~nan] == ref[~nan]).all()
    assert oracle.e4m3_value(0x7E) == 448.0


def test_e4m3_encode_matches_torch_below_overflow():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.uniform(-463, 463, 200000),
        np.exp2(rng.uniform(-14, 8.85, 200000)) * rng.choice([-1, 1], 200000),
        np.array([0.0, -0.0, 2.0**-10, 3 * 2.0**-11, 2.0**-9, 2.0**-6, 1.0625, 1.1875, 240.0, 248.0, 264.0]),
    ]).astype(np.float32)
    # all representable midpoints (exact ties)
    vals = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    x = np.concatenate([x, ((vals[:-1] + vals[1:]) / 2).astype(np.float32)])
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = oracle.e4m3_encode_array(x.astype(np.float64))
    assert (mine == ref).all(), np.nonzero(mine != ref)[0][:10]


def test_e4m3_saturates_and_roundtrips():
    for x in (448.0, 464.0, 480.0, 1e6, float("inf")):
        assert oracle.e4m3_encode(x) == 0x7E
        assert oracle.e4m3_encode(-x) == 0xFE
    assert oracle.e4m3_encode(float("nan")) == 0x7F
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c


# --------------------------------------------------------------------------- bf16
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(100000), rng.standard_normal(1000) * 1e-39,
                        np.exp2(rng.uniform(-120, 120, 10000))]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = oracle.bf16_from_double_array(x.astype(np.float64))
    assert (mine == ref).all()
    bits = np.array([0x3F80, 0xBF80, 0x0001, 0x7F7F, 0x4049], np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert [oracle.bf16_value(int(b)) for b in bits] == list(ref)
    # infinities and overflow: the largest finite bf16 is 0x7F7F = (2 - 2^-7) 2^127;
    # from the midpoint (2 - 2^-8) 2^127 on, values round to infinity (ties to even)
    big = np.array([np.inf, -np.inf, 3.3895e38, 3.3961776e38, 3.3961775e38, -3.4e38,
                    np.finfo(np.float32).max], np.float32)
    ref = torch.from_numpy(big).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = oracle.bf16_from_double_array(big.astype(np.float64))
    assert (mine == ref).all(), (mine, ref)
    assert oracle.bf16_from_double(1e300) == 0x7F80 and oracle.bf16_from_double(-1e300) == 0xFF80
    assert oracle.bf16_from_double(float("nan")) == 0x7FC0


# --------------------------------------------------------------------------- E8M0 / scale rule
def test_scale_rule_closed_forms():
    for k in range(-100, 100, 7):
        assert oracle.mx_exponent(2.0**k, 2) == k - 2          # amax = 2^k -> element 4
        assert oracle.mx_exponent(2.0**k * 1.01, 2) == k - 1   # just above -> next power
        assert oracle.mx_exponent(2.0**k * 0.99, 2) == k - 2
        assert oracle.mx_exponent(2.0**k, 8) == k - 8          # E4M3 block: amax -> 256
    assert oracle.mx_exponent(0.0, 2) == -127
    assert oracle.mx_exponent(2.0**-140, 2) == -127            # clamped
    assert oracle.mx_exponent(2.0**-149, 8) == -127
    assert oracle.e8m0_value(127) == 1.0 and oracle.e8m0_value(0) == 2.0**-127
    assert math.isnan(oracle.e8m0_value(255))


def _block_scale_numpy(block, k):
    amax = np.max(np.abs(block))
    if amax == 0:
        return -127
    return int(min(127, max(-127, math.ceil(np.log2(amax)) - k)))


def test_mxfp4_quantizer_bruteforce():
    table = gold("e2m1_magnitudes.json")["magnitudes"]
    rng = np.random.default_rng(11)
    B, H, S, D = 1, 2, 37, 64
    x = rng.standard_normal((B, H, S, D)).astype(np.float32)
    x[0, 0, 3, 5] *= 300.0              # outlier in one block
    x[0, 1, 4, :32] = 0.0               # all-zero block
    x[0, 1, 5, 32:] *= 1e-30            # tiny block
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales, _ = oracle.quantize_qk4(bits)
    assert codes.shape == (B, H, S, D // 2) and scales.shape == (B, H, S, D // 32)
    xv = oracle.bf16_to_f64(bits)
    for h in range(H):
        for s in range(S):
            for blk in range(D // 32):
                v = xv[0, h, s, blk * 32:(blk + 1) * 32]
                e = _block_scale_numpy(v, 2)
                assert scales[0, h, s, blk] == e + 127
                for i in range(32):
                    a = v[i] * 2.0**-e
                    want = (8 if math.copysign(1.0, a) < 0 else 0) | _nearest_even_bruteforce(abs(a), table)
                    byte = codes[0, h, s, (blk * 32 + i) // 2]
                    got = (byte >> 4) if i % 2 else (byte & 15)
                    assert got == want, (h, s, blk, i, a)
    # the block maximum lands in (2, 4] after scaling
    deq = oracle.dequant_qk4(codes, scales)
    blocks = np.abs(deq.reshape(-1, 32)).max(axis=1) / np.array([oracle.e8m0_value(c) for c in scales.ravel()])
    nz = blocks > 0
    assert ((blocks[nz] > 1.5) & (blocks[nz] <= 4.0)).all()


def test_mxfp4_prescaled_quantizer_bruteforce():
    """Q is quantised as fl32(q * c2): the binary32 product (numpy float32
    multiply) is brute-forced through the block rule and the printed E2M1
    table; a power-of-two prescale only moves the scale byte."""
    table = gold("e2m1_magnitudes.json")["magnitudes"]
    rng = np.random.default_rng(13)
    B, H, S, D = 1, 1, 23, 64
    x = rng.standard_normal((B, H, S, D)).astype(np.float32) * 3.0
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    c2 = oracle.exp2_scale(1.0 / math.sqrt(128))
    assert c2 == float(np.float32(np.float32(1.0 / math.sqrt(128)) * np.float32(math.log2(math.e))))
    codes, scales, _ = oracle.quantize_qk4(bits, prescale=c2)
    xv = oracle.bf16_to_f64(bits).astype(np.float32) * np.float32(c2)  # binary32 products
    for s_ in range(S):
        for blk in range(D // 32):
            v = xv[0, 0, s_, blk * 32:(blk + 1) * 32].astype(np.float64)
            e = _block_scale_numpy(v, 2)
            assert scales[0, 0, s_, blk] == e + 127
            for i in range(32):
                a = v[i] * 2.0**-e
                want = (8 if math.copysign(1.0, a) < 0 else 0) | _nearest_even_bruteforce(abs(a), table)
                byte = codes[0, 0, s_, (blk * 32 + i) // 2]
                got = (byte >> 4) if i % 2 else (byte & 15)
                assert got == want, (s_, blk, i, a)
    c1, s1, _ = oracle.quantize_qk4(bits)
    c8, s8, _ = oracle.quantize_qk4(bits, prescale=8.0)
    assert np.array_equal(c1, c8) and np.array_equal(s8.astype(int), s1.astype(int) + 3)


def test_mxfp4_bits_per_element_and_nonfinite():
    g = gold("mx_bits_per_element.json")
    D = 128
    bits = 8 * (D // 2 + D // 32) / D
    assert bits == g["mxfp4_block32_bits"]
    assert round(16 / bits, 2) == g["compression_vs_fp16_block32"]
    assert round(16 / (4 + 8 / 16), 2) == g["compression_vs_fp16_block16"]
    assert round((4 + 4 + 8) / 3, 2) == g["qk4v8_average_element_bits"]
    x = np.zeros((1, 1, 2, 64), np.float32)
    x[0, 0, 0, 3] = np.nan
    x[0, 0, 1, 40] = np.inf
    bits_ = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales, _ = oracle.quantize_qk4(bits_)
    assert scales[0, 0, 0, 0] == 0xFF and scales[0, 0, 0, 1] == 0  # zero block: code 0
    assert scales[0, 0, 1, 1] == 0xFF
    assert (codes[0, 0, 0, :16] == 0).all() and (codes[0, 0, 1, 16:] == 0).all()


def test_v8_quantizer_bruteforce_vs_torch():
    rng = np.random.default_rng(13)
    B, H, S, D = 1, 2, 75, 64   # ragged: last block holds 11 tokens
    v = rng.standard_normal((B, H, S, D)).astype(np.float32)
    v[0, 1, 40, 7] = 50.0
    bits = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales = oracle.quantize_v8(bits)
    nb = (S + 31) // 32
    assert codes.shape == (B, H, nb, D, 32) and scales.shape == (B, H, nb, D)
    vv = oracle.bf16_to_f64(bits)
    for h in range(H):
        for blk in range(nb):
            j0, j1 = blk * 32, min(S, blk * 32 + 32)
            for c in range(D):
                col = vv[0, h, j0:j1, c]
                e = _block_scale_numpy(col, 8)
                assert scales[0, h, blk, c] == e + 127
                want = torch.from_numpy((col * 2.0**-e).astype(np.float32)).to(torch.float8_e4m3fn)
                want = want.view(torch.uint8).numpy()
                got = codes[0, h, blk, c, :j1 - j0]
                assert (got == want).all()
                assert (codes[0, h, blk, c, j1 - j0:] == 0).all()   # absent tokens
                m = np.abs(np.array([oracle.e4m3_value(x) for x in got])).max()
                assert m == 0 or 128 <= m <= 256


def test_kbar_is_nearest_bf16_of_exact_mean():
    rng = np.random.default_rng(17)
    S, D = 300, 64  # blocks of 128, 128, 44
    k = (rng.standard_normal((1, 1, S, D)) + rng.normal(0, 3, (1, 1, 1, D))).astype(np.float32)
    bits = torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales, kbar = oracle.quantize_qk4(bits, smooth=True)
    assert kbar.shape == (1, 1, 3, D)
    kv = oracle.bf16_to_f64(bits)[0, 0]
    for t in range(3):
        blk = kv[t * 128:min(S, t * 128 + 128)]
        from fractions import Fraction
        for c in range(D):
            mean = sum(Fraction(float(x)) for x in blk[:, c]) / len(blk)
            b = int(kbar[0, 0, t, c])
            got = Fraction(oracle.bf16_value(b))
            for nb in (b - 1, b + 1):   # neighbouring bf16 values are no nearer
                other = Fraction(oracle.bf16_value(nb & 0xFFFF))
                assert abs(got - mean) <= abs(other - mean)
    # smoothed tensor: constant tokens in a block give K - Kbar = 0 -> zero codes, scale code 0
    k2 = np.tile(rng.standard_normal((1, 1, 1, D)).astype(np.float32), (1, 1, 128, 1))
    b2 = torch.from_numpy(k2).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    c2, s2, kb2 = oracle.quantize_qk4(b2, smooth=True)
    assert (kb2[0, 0, 0] == b2[0, 0, 0]).all()
    assert (s2 == 0).all() and ((c2 & 0x77) == 0).all()


def test_kbar_nonfinite_and_order():
    """Kbar of blocks holding infinities or NaN is the IEEE mean (inf, -inf or
    NaN), and the smoothed blocks of that channel are non-finite (scale 0xFF,
    zero codes).  The sum runs in token order: a channel whose values span
    more than binary64 adds exactly keeps the token-order rounding."""
    D = 64
    k = np.ones((1, 1, 128, D), np.float32)
    k[0, 0, 3, 0] = np.inf                        # -> +inf
    k[0, 0, 4, 1] = -np.inf                       # -> -inf
    k[0, 0, 5, 2], k[0, 0, 6, 2] = np.inf, -np.inf  # -> NaN
    k[0, 0, 7, 3] = np.nan                        # -> NaN
    k[0, 0, 0, 32], k[0, 0, 64, 32] = 2.0**60, -(2.0**60)   # token order: 2^60 + 1 = 2^60
    bits = torch.from_numpy(k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales, kbar = oracle.quantize_qk4(bits, smooth=True)
    kb = kbar[0, 0, 0]
    assert kb[0] == 0x7F80 and kb[1] == 0xFF80
    assert (kb[2] & 0x7FFF) > 0x7F80 and (kb[3] & 0x7FFF) > 0x7F80
    assert (kb[4:32] == 0x3F80).all()                  # mean of ones
    # rows 1..63 add 1 to 2^60 and are lost; from row 64 on the sum restarts at 0
    assert oracle.bf16_value(int(kb[32])) == 63.0 / 128.0
    assert (scales[0, 0, :, 0] == 0xFF).all() and (codes[0, 0, :, :16] == 0).all()
    assert (scales[0, 0, :, 1] != 0xFF).all()
    nv_codes, nv_scales, nv_kbar = oracle.quantize_nvfp4(bits, 1.0, smooth=True)
    assert (nv_kbar == kbar).all()


def test_v4_quantizer_bruteforce_vs_printed_table():
    """MXFP4 V (the full-FP4 contrast case): each block of 32 consecutive
    tokens of one channel gets e = ceil(log2 amax) - 2 and E2M1 codes by the
    nearest-even rule over the printed magnitudes; token 2k in the low nibble
    of byte k; tokens past S count as 0."""
    table = gold("e2m1_magnitudes.json")["magnitudes"]
    rng = np.random.default_rng(17)
    B, H, S, D = 1, 2, 75, 32   # ragged: last block holds 11 tokens
    v = rng.standard_normal((B, H, S, D)).astype(np.float32)
    v[0, 1, 40, 7] = 50.0       # outlier
    v[0, 0, 32:64, 3] = 0.0     # all-zero block
    bits = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales = oracle.quantize_v4(bits)
    nb = (S + 31) // 32
    assert codes.shape == (B, H, nb, D, 16) and scales.shape == (B, H, nb, D)
    vv = oracle.bf16_to_f64(bits)
    for h in range(H):
        for blk in range(nb):
            j0, j1 = blk * 32, min(S, blk * 32 + 32)
            for c in range(D):
                col = vv[0, h, j0:j1, c]
                e = _block_scale_numpy(col, 2)
                assert scales[0, h, blk, c] == e + 127
                for t in range(32):
                    a = col[t] * 2.0**-e if t < j1 - j0 else 0.0
                    want = (8 if math.copysign(1.0, a) < 0 else 0) | _nearest_even_bruteforce(abs(a), table)
                    byte = codes[0, h, blk, c, t // 2]
                    got = (byte >> 4) if t % 2 else (byte & 15)
                    assert got == want, (h, blk, c, t)
        dq = oracle.dequant_v4(codes[0, h], scales[0, h], S)
        assert dq.shape == (S, D)
        # decoding the brute-forced codes by the printed table gives the same values
        for j in (0, 17, 40, 74):
            for c in (0, 3, 7):
                blk = j // 32
                byte = codes[0, h, blk, c, (j % 32) // 2]
                code = (byte >> 4) if j % 2 else (byte & 15)
                mag = table[code & 7] * 2.0 ** (int(scales[0, h, blk, c]) - 127)
                assert dq[j, c] == (-mag if code & 8 else mag)


def test_nvfp4_tensor_scale_closed_forms():
    """The per-tensor scale is the smallest power of two g with amax / (6 g) <= 448."""
    assert oracle.nvfp4_tensor_scale(6 * 448.0) == 1.0
    assert oracle.nvfp4_tensor_scale(6 * 448.0 * 1.0001) == 2.0
    assert oracle.nvfp4_tensor_scale(6 * 448.0 / 2) == 0.5
    assert oracle.nvfp4_tensor_scale(0.0) == 1.0
    for amax in (1e-3, 0.37, 5.0, 1234.5, 1e6):
        g = oracle.nvfp4_tensor_scale(amax)
        assert amax / (6 * g) <= 448.0 < amax / (6 * g / 2)
        assert math.frexp(g)[0] == 0.5


def test_nvfp4_quantizer_bruteforce():
    """NVFP4 blocks of 16: the E4M3 scale (torch float8 of the binary32 quotient
    fl32(fl32(amax / g) / 6)) and the E2M1 elements (nearest-even over the
    printed magnitudes of the binary32 quotient x / (s g)), brute-forced; and
    the format's 4.5 bits per element."""
    table = gold("e2m1_magnitudes.json")["magnitudes"]
    g_bits = gold("mx_bits_per_element.json")
    assert 4 + 8 / 16 == g_bits["nvfp4_block16_bits"]
    rng = np.random.default_rng(19)
    B, H, S, D = 1, 2, 23, 64
    x = rng.standard_normal((B, H, S, D)).astype(np.float32)
    x[0, 0, 3, 5] *= 300.0              # outlier: sets the tensor scale
    x[0, 1, 4, :16] = 0.0               # all-zero block
    x[0, 1, 5, 16:32] *= 1e-4           # small block, small scale
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    xv = oracle.bf16_to_f64(bits).astype(np.float32)
    for prescale in (1.0, oracle.exp2_scale(0.125)):
        xp = xv * np.float32(prescale) if prescale != 1.0 else xv
        g = oracle.nvfp4_tensor_scale(float(np.abs(xp).max()))
        codes, scales, _ = oracle.quantize_nvfp4(bits, g, prescale=prescale)
        assert codes.shape == (B, H, S, D // 2) and scales.shape == (B, H, S, D // 16)
        for h in range(H):
            for s in range(S):
                for blk in range(D // 16):
                    v = xp[0, h, s, blk * 16:(blk + 1) * 16]
                    q = np.float32(np.float32(np.abs(v).max()) / np.float32(g)) / np.float32(6.0)
                    want_sc = torch.tensor([float(q)], dtype=torch.float32).to(torch.float8_e4m3fn)
                    want_sc = int(want_sc.view(torch.uint8).item())
                    assert scales[0, h, s, blk] == want_sc, (prescale, h, s, blk)
                    t = np.float32(oracle.e4m3_value(want_sc)) * np.float32(g)
                    for i in range(16):
                        if t == 0:
                            want = 0
                        else:
                            a = float(np.float32(v[i]) / t)
                            want = (8 if math.copysign(1.0, a) < 0 else 0) | _nearest_even_bruteforce(abs(a), table)
                        byte = codes[0, h, s, (blk * 16 + i) // 2]
                        got = (byte >> 4) if i % 2 else (byte & 15)
                        assert got == want, (prescale, h, s, blk, i)
        assert (scales[0, 1, 4, 0] == 0) and (codes[0, 1, 4, :8] == 0).all()
        deq = oracle.dequant_nvfp4(codes, scales, g)
        # decoding is code value x block scale x tensor scale
        c0 = codes[0, 0, 0, 0] & 15
        assert deq[0, 0, 0, 0] == (-1 if c0 & 8 else 1) * table[c0 & 7] * oracle.e4m3_value(scales[0, 0, 0, 0]) * g


def test_nvfp4_nonfinite_block():
    x = np.ones((1, 1, 1, 32), np.float32)
    x[0, 0, 0, 20] = np.nan
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales, _ = oracle.quantize_nvfp4(bits, 1.0)
    assert scales[0, 0, 0, 1] == 0x7F and (codes[0, 0, 0, 8:] == 0).all()
    assert scales[0, 0, 0, 0] != 0x7F
