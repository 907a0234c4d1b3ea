"""Pin of the oracle's binary32 exponent argument, and of its dequantiser layouts
(CPU only).

Exponent argument.  Where floating point decides an integer (here: the E4M3
code of each probability and the integer running max), the oracle and the
kernels decide in binary32: the argument of P is
    y = fl32( fl32(S') + fl32( c2 * fl32(delta) ) ),   c2 = fl32(scale * fl32(log2 e)),
the running max m' = max(m, ceil(max_j y_j)) per 128-key tile, and
P = E4M3(256 * fl32(2^(y - m'))), the exponential also rounded to binary32
(the online softmax of the FP4 tutorial's section "注意力慢在哪儿", with the
rank-one compensation term of the MpFA abstract).  The brute force below
rebuilds that row computation with numpy float32 arithmetic (each operation
rounds to binary32) and a nearest-value E4M3 rounding over torch's float8
decode table (ties to the even code), independent of the oracle's C code.
The inputs are built so that the binary32 and binary64 arguments give
different P codes, so that a plausible mistake in the rounding order --
rounding c2 * delta in binary64 first, or adding delta before rounding S' --
gives different codes too, and so that a binary64 exponential of the binary32
argument does as well: the test tells all of these apart.

Dequantisers.  Known codes at known positions are decoded with the E2M1
magnitudes printed in the tutorial's section "FP4 只有约 15 个可表示的数"
(tests/golden) and torch's float8 decode, and compared with the oracle's
dequantisers element by element: nibble order (even element in the low
nibble), the V record layout [S/32][D][32] and its scale per (32 tokens,
channel).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

LOG2E_F32 = np.float32(1.44269502162933349609375)
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _e4m3_table():
    codes = torch.arange(0, 0x7F, dtype=torch.uint8)  # 0x00 .. 0x7E: every finite non-negative code
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


E4M3_POS = _e4m3_table()


def e4m3_nearest(x):
    """E4M3 rounding of non-negative x by nearest-value search over torch's
    decode table; an exact tie goes to the even code (the table index is the
    code)."""
    x = np.asarray(x, np.float64)
    d = np.abs(x[..., None] - E4M3_POS)
    i = np.argmin(d, axis=-1)               # the lower of two tied codes
    srt = np.sort(d, axis=-1)
    tie = (srt[..., 1] == srt[..., 0]) & (x != 0)
    i = np.where(tie & (i % 2 == 1), i + 1, i)
    return E4M3_POS[i]


def p_codes(y, mnew, mode):
    """E4M3(256 * 2^(y - m')): the exponential rounded to binary32, except in
    the all-binary64 mode and the binary64-exponential mistake."""
    e = np.exp2(y - mnew)
    if mode not in ("fp64", "exp64"):
        e = e.astype(np.float32).astype(np.float64)
    return e4m3_nearest(256.0 * e)


def argument(Sp, delta, scale, mode):
    """Exponent argument of one tile's keys.  Sp: exact S' (binary64 values
    that are binary32-representable or not); delta: the tile's exact
    compensation sum."""
    c2f = np.float32(np.float32(scale) * LOG2E_F32)
    if mode == "fp32":            # the reading: fl32(fl32(S') + fl32(c2 * fl32(delta)))
        d32 = np.float32(c2f * np.float32(delta))
        return (Sp.astype(np.float32) + d32).astype(np.float64)
    if mode == "fp64":            # everything in binary64
        return Sp + float(np.float32(scale)) * math.log2(math.e) * delta
    if mode == "c2_in_fp64":      # mistake: fl32(c2 * delta) formed from the binary64 product
        d32 = np.float32(float(c2f) * delta)
        return (Sp.astype(np.float32) + d32).astype(np.float64)
    if mode == "add_first":       # mistake: S' + c2 delta added before any rounding
        return (Sp + float(c2f) * float(np.float32(delta))).astype(np.float32).astype(np.float64)
    if mode == "exp64":           # mistake: the binary32 argument, but a binary64 exponential
        return argument(Sp, delta, scale, "fp32")
    raise ValueError(mode)


def bruteforce_row(Sp, deltas, V, scale, mode, tile=128):
    """The online schedule of one row in binary64 around the argument above:
    per tile m' = max(m, ceil(max y)), P = E4M3(256 * 2^(y - m')),
    l = 2^(m - m') l + sum P, o = 2^(m - m') o + P V."""
    L, D = V.shape
    m, l, o = -math.inf, 0.0, np.zeros(D)
    codes = []
    for t in range((L + tile - 1) // tile):
        j0, j1 = t * tile, min(L, (t + 1) * tile)
        y = argument(Sp[j0:j1], deltas[t], scale, mode)
        mnew = max(m, math.ceil(float(y.max())))
        alpha = 0.0 if m == -math.inf else 2.0 ** (m - mnew)
        P = p_codes(y, mnew, mode)
        codes.append(P * 2.0 ** (mnew - 0.0))
        l = alpha * l + P.sum()
        o = alpha * o + P @ V[j0:j1]
        m = mnew
    return o / l, math.log(2.0) * (m + math.log2(l / 256.0)), np.concatenate(codes)


MODES = ("fp32", "fp64", "c2_in_fp64", "add_first", "exp64")


def _case(seed, scale):
    """One row, 300 keys in three tiles.  Q = e0 and K[:, 0] = S' so that
    S'_j = K[j, 0] exactly; Qc = e0 and Kbar[t, 0] = delta_t so that the
    compensation sum of tile t is delta_t exactly.  The keys of tile 1 sit
    next to E4M3 rounding boundaries of 256 * 2^(y - m'), and delta_1 is
    searched until the binary32 and binary64 arguments (and the two mistaken
    rounding orders) put at least one key on different sides."""
    rng = np.random.default_rng(seed)
    D, L = 4, 300
    c2d = float(np.float32(scale)) * math.log2(math.e)
    V = rng.standard_normal((L, D))
    Sp = rng.uniform(-6.0, 0.0, L)
    deltas = rng.uniform(-2.0, 2.0, 3)
    # E4M3 midpoints between consecutive normal codes in [32, 256): 256 * 2^(y - m') = mid
    mids = np.array([(E4M3_POS[k] + E4M3_POS[k + 1]) / 2 for k in range(len(E4M3_POS) - 1)])
    mids = mids[(mids > 32) & (mids < 256)]
    for _ in range(20000):
        d1 = rng.uniform(-3.0, 3.0)
        deltas[1] = d1
        # tile 1: key 128 carries the tile max (y ~ 0.4, so m' = 1); the others aim at midpoints
        tgt = np.empty(128)
        tgt[0] = 0.4
        tgt[1:] = 1.0 + np.log2(rng.choice(mids, 127) / 256.0)
        Sp[128:256] = tgt - c2d * d1
        Sp[128:256] = Sp[128:256].astype(np.float32).astype(np.float64) + rng.uniform(-1, 1, 128) * 2.0**-40
        ys = {m: argument(Sp[128:256], d1, scale, m) for m in MODES}
        if any(math.ceil(y.max()) != 1 for y in ys.values()):
            continue
        pc = {m: p_codes(y, 1.0, m) for m, y in ys.items()}
        if all(np.any(pc["fp32"] != pc[m]) for m in MODES[1:]):
            break
    else:
        raise AssertionError("no discriminating input found")
    Q = np.zeros((1, D))
    Q[0, 0] = 1.0
    K = np.zeros((L, D))
    K[:, 0] = Sp
    Kbar = np.zeros((3, D))
    Kbar[:, 0] = deltas
    return Q, K, V, Kbar, Sp, deltas


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_binary32_argument_matches_float32_bruteforce(seed):
    scale = 1.0 / math.sqrt(128.0)
    Q, K, V, Kbar, Sp, deltas = _case(seed, scale)
    Oa, la = oracle.attn_quant_rows(Q, np.zeros(1, np.int64), K, V, 1, False, scale, Qc=Q, Kbar=Kbar,
                                    fp32_arg=True)
    Ob, lb = oracle.attn_quant_rows(Q, np.zeros(1, np.int64), K, V, 1, False, scale, Qc=Q, Kbar=Kbar,
                                    fp32_arg=False)
    res = {m: bruteforce_row(Sp, deltas, V, scale, m) for m in MODES}
    # the oracle's binary32 path is the float32 brute force, to rounding of the binary64 sums
    assert np.abs(Oa[0] - res["fp32"][0]).max() < 1e-12
    assert abs(la[0] - res["fp32"][1]) < 1e-12
    # its binary64 path is the binary64 brute force
    assert np.abs(Ob[0] - res["fp64"][0]).max() < 1e-12
    assert abs(lb[0] - res["fp64"][1]) < 1e-12
    # and the inputs discriminate: every other rounding order gives other codes and another O
    for m in MODES[1:]:
        assert np.any(res[m][2] != res["fp32"][2]), m
        assert np.abs(res[m][0] - Oa[0]).max() > 1e-9, m


def test_running_max_decided_in_binary32():
    """m' = ceil(max y) is taken on the binary32 argument: a key whose binary64
    argument lies just above an integer while its binary32 argument rounds onto
    it moves m' by one.  With a second key in E4M3's subnormal range (where
    the power-of-two invariance of the codes breaks) that is visible in O."""
    scale = 1.0 / math.sqrt(128.0)
    c2f = np.float32(np.float32(scale) * LOG2E_F32)
    D = 4
    rng = np.random.default_rng(7)
    for _ in range(100000):
        delta = rng.uniform(1.0, 2.0)
        d32 = np.float32(c2f * np.float32(delta))
        # y32 = fl32(S' + d32) == 3 exactly while y64 = S' + c2 delta > 3
        s = np.float32(3.0) - d32
        y64 = float(s) + float(np.float32(scale)) * math.log2(math.e) * delta
        if np.float32(s + d32) == np.float32(3.0) and y64 > 3.0:
            break
    else:
        raise AssertionError("no input found")
    Sp = np.array([float(s), float(s) - 15.3, float(s) - 2.0])
    V = rng.standard_normal((3, D))
    Q = np.zeros((1, D))
    Q[0, 0] = 1.0
    K = np.zeros((3, D))
    K[:, 0] = Sp
    Kbar = np.zeros((1, D))
    Kbar[0, 0] = delta
    Oa, la = oracle.attn_quant_rows(Q, np.zeros(1, np.int64), K, V, 1, False, scale, Qc=Q, Kbar=Kbar,
                                    fp32_arg=True)
    Ob, _ = oracle.attn_quant_rows(Q, np.zeros(1, np.int64), K, V, 1, False, scale, Qc=Q, Kbar=Kbar,
                                   fp32_arg=False)
    r32 = bruteforce_row(Sp, [delta], V, scale, "fp32")
    r64 = bruteforce_row(Sp, [delta], V, scale, "fp64")
    assert np.abs(Oa[0] - r32[0]).max() < 1e-12 and abs(la[0] - r32[1]) < 1e-12
    assert np.abs(Ob[0] - r64[0]).max() < 1e-12
    assert np.abs(r32[0] - r64[0]).max() > 1e-9  # m' = 3 against m' = 4 changes the subnormal code


# ----------------------------------------------------------------------------- dequantiser layouts
def _e2m1_values():
    with open(os.path.join(GOLD, "e2m1_magnitudes.json")) as f:
        mag = json.load(f)["magnitudes"]
    return np.array(mag + [-m for m in mag])  # codes 0..7 non-negative, bit 3 the sign


def _e4m3_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("D", [64, 128])
def test_dequant_qk4_layout(D):
    rng = np.random.default_rng(D)
    rows = 5
    codes = rng.integers(0, 256, (rows, D // 2), dtype=np.uint8)
    scales = rng.integers(110, 145, (rows, D // 32), dtype=np.uint8)
    got = oracle.dequant_qk4(codes, scales)
    tab = _e2m1_values()
    want = np.empty((rows, D))
    for r in range(rows):
        for c in range(D):
            nib = (int(codes[r, c // 2]) >> (4 * (c % 2))) & 15   # element 2k in the low nibble of byte k
            want[r, c] = tab[nib] * 2.0 ** (int(scales[r, c // 32]) - 127)
    assert np.array_equal(got, want)
    # the swapped nibble order would be caught
    swapped = want.reshape(rows, D // 2, 2)[:, :, ::-1].reshape(rows, D)
    assert not np.array_equal(got, swapped)


def test_dequant_v8_layout():
    rng = np.random.default_rng(11)
    S, D = 77, 64
    nb = (S + 31) // 32
    codes = rng.integers(0, 256, (nb, D, 32), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10     # no NaN codes
    scales = rng.integers(110, 145, (nb, D), dtype=np.uint8)
    got = oracle.dequant_v8(codes, scales, S)
    dec = _e4m3_decode(codes)
    want = np.empty((S, D))
    for j in range(S):
        for c in range(D):
            # record (block j // 32, channel c) holds its 32 tokens contiguously
            want[j, c] = dec[j // 32, c, j % 32] * 2.0 ** (int(scales[j // 32, c]) - 127)
    assert np.array_equal(got, want)
    # a token-major reading [S/32][32][D] of the same bytes would be caught
    tm = np.empty((S, D))
    flat = dec.reshape(nb, 32, D)
    for j in range(S):
        tm[j] = flat[j // 32, j % 32] * 2.0 ** (scales[j // 32].astype(np.float64) - 127)
    assert not np.array_equal(got, tm)


def test_dequant_v4_layout():
    rng = np.random.default_rng(13)
    S, D = 70, 64
    nb = (S + 31) // 32
    codes = rng.integers(0, 256, (nb, D, 16), dtype=np.uint8)
    scales = rng.integers(110, 145, (nb, D), dtype=np.uint8)
    got = oracle.dequant_v4(codes, scales, S)
    tab = _e2m1_values()
    want = np.empty((S, D))
    for j in range(S):
        for c in range(D):
            t = j % 32
            nib = (int(codes[j // 32, c, t // 2]) >> (4 * (t % 2))) & 15
            want[j, c] = tab[nib] * 2.0 ** (int(scales[j // 32, c]) - 127)
    assert np.array_equal(got, want)


def test_dequant_nvfp4_layout():
    rng = np.random.default_rng(17)
    rows, D, g = 4, 64, 2.0 ** -3
    codes = rng.integers(0, 256, (rows, D // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (rows, D // 16), dtype=np.uint8)  # non-negative finite E4M3
    got = oracle.dequant_nvfp4(codes, scales, g)
    tab = _e2m1_values()
    sdec = _e4m3_decode(scales)
    want = np.empty((rows, D))
    for r in range(rows):
        for c in range(D):
            nib = (int(codes[r, c // 2]) >> (4 * (c % 2))) & 15
            want[r, c] = tab[nib] * sdec[r, c // 16] * g
    assert np.array_equal(got, want)
