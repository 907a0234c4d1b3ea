"""GPU-side pins: the hardware conversions and the FP4 product the kernels rely
on, checked against the CPU oracle in isolation (through the test-only probe
library tests/hip/libqfa_probe.so), and a regression check that the decode
kernel reads no LDS byte it did not write.

Converters.  Every binary32 mantissa of every binade of each format's exponent
window, both signs, plus zeros, binary32 subnormals and the saturation range,
is converted by the instruction the kernels use and compared with the oracle's
encoder of the same value (round to nearest, ties to even: the MXFP4 notes,
section 5.2; the E2M1 values of the FP4 tutorial, section
"FP4 只有约 15 个可表示的数"; OCP E4M3 with maximum 448).  The scaled forms are
driven with the power-of-two scale operands the kernels pass (2^(m - 8) for
E4M3 P with m in [-100, 100]; 2^(e - 2) for E2M1 P), so x / scale is exact.

Row sums.  The E4M3-P denominator (one 16x16x128 MFMA per 64 keys against an
E2M1 selector, then one FMA per tile) must give every lane the sum of its own
query's P codes; checked on edge patterns that must match to the bit and on
random codes against exact sums.

Delta.  The rank-one compensation term (K-bar . q_bf16 for 32 tiles x 32
rows) on the FP64 MFMA must equal fl32 of the exact sum bit for bit, with
zeros past the valid tiles and rows.

S tile.  One 128-key tile of S' = Q'4 K4^T from the block-scaled FP4 MFMA,
through the kernels' own tile DMA and operand layout, is compared bit for bit
with the oracle's exact Q' . K (binary64) on workload-shaped inputs: the
products of E2M1 codes scaled by E8M0 are exact and their sums stay exact in
binary32 for these inputs.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from gpu_util import compare_o, say, to_np

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip"))
import build_probe  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    return build_probe.load()


def _binade(b, sign):
    """Every binary32 value of binade [2^b, 2^(b+1)) with the given sign."""
    m = np.arange(1 << 23, dtype=np.uint32)
    bits = ((b + 127) << 23) | m
    if sign < 0:
        bits |= np.uint32(0x80000000)
    return bits.view(np.float32)


def _run_cvt(probe, kind, x32, scale):
    dev = torch.device("cuda:0")
    xt = torch.from_numpy(np.ascontiguousarray(x32)).to(dev)
    n = xt.numel()
    out = torch.empty(n // 2 if kind == 0 else n, dtype=torch.uint8, device=dev)
    rc = probe.probe_cvt(kind, xt.data_ptr(), n, float(scale), out.data_ptr())
    assert rc == 0, rc
    torch.cuda.synchronize()
    o = to_np(out)
    if kind == 0:
        o = np.stack([o & 15, o >> 4], axis=1).reshape(-1)
    return o


def _check(probe, kind, v64, scale, encode, label, limit=math.inf):
    """Convert x = v * scale on the GPU and compare with encode(v) for every
    |v| < limit.  Beyond the limit (values the kernels never feed a
    converter) mismatches are reported, not asserted."""
    if v64.size % 2:
        v64 = np.concatenate([v64, [0.0]])
    x32 = (v64 * scale).astype(np.float32)
    assert np.array_equal(x32.astype(np.float64) / scale, v64), "x / scale must be exact"
    got = _run_cvt(probe, kind, x32, scale)
    want = encode(v64)
    inside = np.abs(v64) < limit
    bad = np.nonzero((got != want) & inside)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError("%s: %d mismatches, first v=%r got 0x%02x want 0x%02x"
                             % (label, bad.size, v64[i], got[i], want[i]))
    out = np.nonzero((got != want) & ~inside)[0]
    if out.size:
        i = out[0]
        say("%s: beyond |v| < %g (never fed by the kernels) %d of %d differ, e.g. v=%r got 0x%02x oracle 0x%02x"
            % (label, limit, out.size, int((~inside).sum()), v64[i], got[i], want[i]))
    return int(inside.sum())


def _extras(hi, subnormals=True):
    """Zeros, binary32 subnormals, and values past the top of the window."""
    sub = np.array([1, 2, 3, 0x400000, 0x7FFFFF], dtype=np.uint32).view(np.float32).astype(np.float64)
    big = np.array([2.0 ** hi, 2.0 ** hi * 1.5, 2.0 ** (hi + 5), 2.0 ** 100], dtype=np.float64)
    parts = [[0.0, -0.0], big, -big] + ([sub, -sub] if subnormals else [])
    return np.concatenate(parts)


E2M1_BINADES = range(-4, 3)     # [1/16, 8): below the half of 1/2 up to past the maximum 6
E4M3_BINADES = range(-11, 9)    # [2^-11, 2^9): below the half of the smallest subnormal 2^-9 up to past 448
E2M1_LIMIT = math.inf           # E2M1: the hardware saturates at 6 like the oracle, asserted everywhere
E4M3_LIMIT = 464.0              # E4M3: the conversions as the kernels call them return NaN above 464
                                # where the oracle saturates to 448; the kernels feed them |x / scale| <= 448
                                # (P <= 256, V <= 256 by the scale rule, the NVFP4 scale clamped to 448)


@pytest.mark.parametrize("scale_exp", [0, -102, -2, 98])
def test_converter_e2m1_every_mantissa(probe, scale_exp):
    scale = 2.0 ** scale_exp
    n = 0
    for b in E2M1_BINADES:
        for sgn in (1, -1):
            n += _check(probe, 0, _binade(b, sgn).astype(np.float64), scale, oracle.e2m1_encode_array,
                        "E2M1 scale 2^%d binade %d sign %d" % (scale_exp, b, sgn), E2M1_LIMIT)
    # past the maximum: saturation to 6
    for b in (3, 4, 5):
        n += _check(probe, 0, _binade(b, 1).astype(np.float64)[::97], scale, oracle.e2m1_encode_array,
                    "E2M1 saturation binade %d" % b, E2M1_LIMIT)
    ex = _extras(3, subnormals=scale_exp == 0)
    n += _check(probe, 0, ex[np.abs(ex) * scale < 1e38], scale, oracle.e2m1_encode_array,
                "E2M1 zeros/subnormals/large", E2M1_LIMIT)
    say("E2M1 scale 2^%d: %d values bit-exact" % (scale_exp, n))


@pytest.mark.parametrize("scale_exp", [-8, -108, 92])
def test_converter_e4m3_scaled_every_mantissa(probe, scale_exp):
    scale = 2.0 ** scale_exp
    n = 0
    for b in E4M3_BINADES:
        for sgn in (1, -1):
            v = _binade(b, sgn).astype(np.float64)
            if scale_exp != -8:
                v = v[::61]  # the other scales: every 61st mantissa
            n += _check(probe, 1, v, scale, oracle.e4m3_encode_array,
                        "E4M3 scale 2^%d binade %d sign %d" % (scale_exp, b, sgn), E4M3_LIMIT)
    ex = _extras(9, subnormals=False)
    ex = ex[np.abs(ex) * scale < 1e38]
    n += _check(probe, 1, ex, scale, oracle.e4m3_encode_array, "E4M3 zeros/large", E4M3_LIMIT)
    say("E4M3 scale 2^%d: %d values bit-exact" % (scale_exp, n))


def test_converter_e4m3_unscaled_every_mantissa(probe):
    n = 0
    for b in E4M3_BINADES:
        for sgn in (1, -1):
            n += _check(probe, 2, _binade(b, sgn).astype(np.float64), 1.0, oracle.e4m3_encode_array,
                        "E4M3 unscaled binade %d sign %d" % (b, sgn), E4M3_LIMIT)
    n += _check(probe, 2, _extras(9), 1.0, oracle.e4m3_encode_array, "E4M3 unscaled zeros/subnormals/large",
                E4M3_LIMIT)
    say("E4M3 unscaled: %d values bit-exact" % n)


def _workload_qk(kind, D, L, seed):
    """Q (32 rows) and K [L] bf16 bits shaped like the workloads: outlier
    channels x20 (Llama-shaped), a per-channel K offset with smoothing
    (Qwen-shaped), or 1% of K rows x8 (long-context)."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((1, 1, 32, D), generator=g)
    k = torch.randn((1, 1, L, D), generator=g)
    smooth = False
    if kind == "outlier":
        q[..., [3, 70 % D]] *= 20.0
        k[..., [5, 17, 40, 99 % D]] *= 20.0
    elif kind == "offset":
        k += torch.randn((1, 1, 1, D), generator=g) * 3.0
        smooth = True
    elif kind == "rows":
        idx = torch.randperm(L, generator=g)[: max(1, L // 100)]
        k[..., idx, :] *= 8.0
    bits = lambda t: t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bits(q), bits(k), smooth


@pytest.mark.parametrize("kind,D,L", [("outlier", 128, 384), ("offset", 128, 300), ("rows", 128, 256),
                                      ("plain", 64, 200), ("outlier", 64, 130)])
def test_s_tile_bit_exact(probe, kind, D, L):
    dev = torch.device("cuda:0")
    scale = 1.0 / math.sqrt(D)
    q, k, smooth = _workload_qk(kind, D, L, seed=D + L)
    qc, qs, _ = oracle.quantize_qk4(q, prescale=oracle.exp2_scale(scale))
    kc, ks, _ = oracle.quantize_qk4(k, smooth=smooth)
    Qd = oracle.dequant_qk4(qc, qs)[0, 0]
    Kd = oracle.dequant_qk4(kc, ks)[0, 0]
    args = [torch.from_numpy(np.ascontiguousarray(a[0, 0])).to(dev) for a in (qc, qs, kc, ks)]
    for t in range((L + 127) // 128):
        nk = min(128, L - 128 * t)
        S = torch.full((32, 128), float("nan"), dtype=torch.float32, device=dev)
        say("S tile %s D%d L%d tile %d" % (kind, D, L, t))
        rc = probe.probe_s_tile(*[a.data_ptr() for a in args], D, L, t, S.data_ptr())
        assert rc == 0, rc
        torch.cuda.synchronize()
        got = to_np(S)[:, :nk].astype(np.float64)
        exact = Qd @ Kd[128 * t:128 * t + nk].T          # exact in binary64 (E2M1 x E8M0 products)
        assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact), "S' not binary32-exact"
        assert np.array_equal(got, exact), np.abs(got - exact).max()


@pytest.mark.parametrize("kind,D,L", [("offset", 128, 300), ("outlier", 128, 256), ("offset", 64, 200)])
def test_s_tile_seeded_accumulator_error_bound(probe, kind, D, L):
    """The compensated kernels start the S accumulator at the row's offset
    d = fl32(c2 fl32(delta)), so the exponent argument y comes out of the
    FP4 MFMAs instead of an add per score.  Measured on MI355X: the
    instruction adds each 32-channel block's product to the accumulator with
    its own binary32 rounding, in MFMA order (blocks 0, 2, 1, 3 for D = 128),
    which reproduces y bit for bit on smooth data; with outlier channels a
    block's internal sum is not always exact.  Pinned here as the recursive-
    summation bound |y - (d + S')| <= n_blocks 2^-24 (|d| + sum_b |S'_b|) for
    the n_blocks = D/32 roundings, S'_b the exact product of channel block b.
    The number of scores where y differs from the oracle's
    fl32(fl32(S') + d) is reported."""
    dev = torch.device("cuda:0")
    scale = 1.0 / math.sqrt(D)
    q, k, smooth = _workload_qk(kind, D, L, seed=3 * D + L)
    qc, qs, _ = oracle.quantize_qk4(q, prescale=oracle.exp2_scale(scale))
    kc, ks, _ = oracle.quantize_qk4(k, smooth=smooth)
    Qd = oracle.dequant_qk4(qc, qs)[0, 0]
    Kd = oracle.dequant_qk4(kc, ks)[0, 0]
    rng = np.random.default_rng(D + L)
    # offsets with full binary32 mantissas, of the size the compensation gives
    d32 = (rng.standard_normal(32) * 4.0).astype(np.float32)
    args = [torch.from_numpy(np.ascontiguousarray(a[0, 0])).to(dev) for a in (qc, qs, kc, ks)]
    dt = torch.from_numpy(d32).to(dev)
    nb = D // 32
    differs = total = 0
    worst = 0.0
    for t in range((L + 127) // 128):
        nk = min(128, L - 128 * t)
        S = torch.full((32, 128), float("nan"), dtype=torch.float32, device=dev)
        say("seeded S tile %s D%d L%d tile %d" % (kind, D, L, t))
        rc = probe.probe_s_tile_seeded(*[a.data_ptr() for a in args], dt.data_ptr(), D, L, t, S.data_ptr())
        assert rc == 0, rc
        torch.cuda.synchronize()
        got = to_np(S)[:, :nk].astype(np.float64)
        Kt = Kd[128 * t:128 * t + nk]
        exact = d32[:, None].astype(np.float64) + Qd @ Kt.T
        mag = np.abs(d32[:, None]).astype(np.float64)
        for b in range(nb):
            ch = slice(32 * b, 32 * b + 32)
            mag = mag + np.abs(Qd[:, ch] @ Kt[:, ch].T)
        rel = np.abs(got - exact) / (mag * 2.0 ** -24)
        worst = max(worst, float(rel.max()))
        assert rel.max() <= nb, (rel.max(), nb)
        reading = ((Qd @ Kt.T).astype(np.float32) + d32[:, None]).astype(np.float64)
        differs += int(np.sum(got != reading))
        total += got.size
    say("seeded S %s D%d: error <= %.2f x 2^-24 of the summed magnitudes (bound %d); %d of %d scores differ "
        "from fl32(fl32(S') + d)" % (kind, D, worst, nb, differs, total))


def _rowsum_inputs(case, rng):
    """P codes per (lane, tile, half, byte) in the 32x32x64 B layout of the
    P V product (lane l holds 32 keys of query l % 32), and per-query scale
    codes 2^(m - m_ref) (the same for lanes l and l + 32, as the kernels pass)."""
    codes = np.zeros((64, 2, 2, 32), dtype=np.uint8)
    query = np.arange(64) % 32
    if case == "random":
        codes[:] = rng.integers(0, 0x7F, size=codes.shape)          # every finite E4M3 code >= 0
        codes[rng.random(codes.shape) < 0.3] = 0
    elif case == "ones":
        codes[:] = 0x38
    elif case == "query_halves":                                      # queries 0..15 only, then 16..31 only
        codes[query < 16, 0] = 0x38
        codes[query >= 16, 1] = 0x38
    elif case == "lane_groups":                                       # only lanes 32..63 (second key half)
        codes[32:] = 0x38
    elif case == "extremes":                                          # 448 beside subnormals
        codes[:] = rng.choice(np.array([0x7E, 0x01, 0x07, 0x08, 0x00], dtype=np.uint8), size=codes.shape)
    qs = rng.integers(0, 65, size=(32, 2))
    ps = (127 + qs[query]).astype(np.int32)                         # (64, 2)
    return codes, ps


@pytest.mark.parametrize("case", ["ones", "query_halves", "lane_groups", "random", "extremes"])
def test_tile_rowsum_sums_each_lanes_own_query(probe, case):
    """The E4M3-P denominator: per 64-key half one 16x16x128 MFMA (E2M1
    selector x the P operand, unit scales), then lsum += 2^(m - m_ref) x the
    tile's row sum.  Every element of lane l must carry the row sum of query
    l % 32.  Sums of E4M3 1.0 codes are exact, so the selection cases must
    match to the bit; on random codes the matrix unit's FP8 accumulation is
    not exact (measured up to 1.0e-4 relative, with 448 beside subnormals),
    so the bound there is 2^-12,
    far below the error of a wrong selection (a whole query's sum)."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(len(case))
    codes, ps = _rowsum_inputs(case, rng)
    pb = torch.from_numpy(np.ascontiguousarray(codes).view(np.int32).reshape(64, 32)).to(dev)
    pst = torch.from_numpy(np.ascontiguousarray(ps)).to(dev)
    ts = torch.full((2, 64, 4), float("nan"), dtype=torch.float32, device=dev)
    lsum = torch.full((64,), float("nan"), dtype=torch.float32, device=dev)
    say("tile row sums: %s" % case)
    rc = probe.probe_tile_rowsum(pb.data_ptr(), pst.data_ptr(), ts.data_ptr(), lsum.data_ptr())
    assert rc == 0, rc
    torch.cuda.synchronize()
    ts, lsum = to_np(ts).astype(np.float64), to_np(lsum).astype(np.float64)
    val = np.array([oracle.e4m3_value(c) for c in range(256)])
    per_lane = val[codes].sum(axis=(2, 3))                           # (64, 2): tile sums of a lane's keys
    exact = np.zeros((32, 2))
    np.add.at(exact, np.arange(64) % 32, per_lane)
    want = exact[np.arange(64) % 32]                                 # (64, 2)
    assert np.array_equal(ts, np.repeat(ts[..., :1], 4, axis=-1)), "a lane's four elements differ"
    got = ts[..., 0].T                                               # (64, 2)
    want_l = (want * 2.0 ** (ps - 127)).sum(axis=1)
    if case in ("ones", "query_halves", "lane_groups"):
        assert np.array_equal(got, want), (got, want)
        # two FMAs: the first term is exact, the second rounds the exact sum once
        assert np.array_equal(lsum, want_l.astype(np.float32).astype(np.float64)), (lsum, want_l)
    else:
        rel = np.abs(got - want) / np.maximum(want, 1e-30)
        rl = np.abs(lsum - want_l) / np.maximum(want_l, 1e-30)
        say("tile row sums %s: worst relative error %.3g (tile), %.3g (denominator)" % (case, rel.max(), rl.max()))
        assert rel.max() <= 2.0 ** -12 and rl.max() <= 2.0 ** -12, (rel.max(), rl.max())


@pytest.mark.parametrize("kind,D,ntiles,tau0,tlim,nrows", [
    ("offset", 128, 32, 0, 32, 32), ("outlier", 128, 32, 0, 32, 32), ("offset", 64, 32, 0, 32, 32),
    ("offset", 128, 45, 32, 45, 32), ("outlier", 128, 64, 32, 50, 7), ("offset", 64, 40, 32, 33, 1)])
def test_delta_exactly_rounded(probe, kind, D, ntiles, tau0, tlim, nrows):
    """The rank-one term delta[tile][row] = Kbar_tile . q_row of 32 tiles at
    once, on the FP64 MFMA: the bf16 products are exact in binary64 and so is
    their sum for these inputs, so every entry must be fl32 of the exact
    binary64 sum, bit for bit (the offset decides P codes, and the oracle
    rounds the exact value).  Tiles from tlim on and rows from nrows on give
    exactly 0, except that a 16-tile half starting at or past tlim is not
    computed at all (no wave reads it)."""
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(D + 7 * ntiles + tau0 + nrows)
    off = rng.standard_normal(D) * 3.0                              # per-channel K offset (the smoothed part)
    kbar = off[None, :] + 0.3 * rng.standard_normal((ntiles, D))
    q = rng.standard_normal((32, D)) * 2.0
    if kind == "outlier":
        q[:, [3, 70 % D]] *= 20.0
    kb_bits = oracle.bf16_from_double_array(kbar).reshape(kbar.shape)
    q_bits = oracle.bf16_from_double_array(q).reshape(q.shape)
    kb_v, q_v = oracle.bf16_to_f64(kb_bits), oracle.bf16_to_f64(q_bits)
    kt = torch.from_numpy(np.ascontiguousarray(kb_bits).view(np.int16)).to(dev)
    qt = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).to(dev)
    out = torch.full((32, 32), float("nan"), dtype=torch.float32, device=dev)
    say("delta %s D%d tiles %d tau0 %d tlim %d rows %d" % (kind, D, ntiles, tau0, tlim, nrows))
    rc = probe.probe_delta(kt.data_ptr(), tlim, tau0, qt.data_ptr(), D, nrows, D, out.data_ptr())
    assert rc == 0, rc
    torch.cuda.synchronize()
    got = to_np(out).astype(np.float64)                             # [tile][row]
    nt, nr = min(32, tlim - tau0), nrows
    exact = kb_v[tau0:tau0 + nt] @ q_v[:nr].T                       # bf16 products: exact in binary64
    written = 16 if nt <= 16 else 32                                # tile halves the call computes
    assert np.all(got[nt:written, :] == 0.0) and np.all(got[:written, nr:] == 0.0), "past tlim / nrows: not 0"
    want = exact.astype(np.float32).astype(np.float64)
    bad = int(np.sum(got[:nt, :nr] != want))
    say("delta %s D%d: %d of %d entries differ from fl32(exact)" % (kind, D, bad, want.size))
    assert bad == 0, np.abs(got[:nt, :nr] - want).max()


@pytest.mark.parametrize("D,lens", [(64, [5, 517, 129, 1]), (128, [517, 5, 255, 130])])
def test_decode_after_lds_filled_with_nan_codes(probe, D, lens):
    """Fill every compute unit's LDS with 0x7F (the E4M3 NaN code), then decode
    ragged caches whose last tiles are partial: a kernel that read LDS bytes
    its own DMA did not write would turn O into NaN."""
    import bit_quantized_attention_qk4pv8_amd as qfa
    from bit_quantized_attention_qk4pv8_amd.workloads import bf16_bits
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(D)
    B, Hq, Hkv, Smax = len(lens), 8, 2, max(lens)
    scale = 1.0 / math.sqrt(D)
    q = torch.randn((B, Hq, 1, D), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((B, Hkv, Smax, D), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((B, Hkv, Smax, D), generator=g, device=dev).to(torch.bfloat16)
    k4, k4s, _ = qfa.quantize_qk4(k)
    kv_lens = torch.tensor(lens, dtype=torch.int32, device=dev)
    # each sequence's cache holds its own tokens quantised (what the cache writer stores)
    v8 = torch.zeros((B, Hkv, (Smax + 31) // 32, D, 32), dtype=torch.uint8, device=dev)
    v8s = torch.zeros((B, Hkv, (Smax + 31) // 32, D), dtype=torch.uint8, device=dev)
    for b, L in enumerate(lens):
        vb, vbs = qfa.quantize_v8(v[b:b + 1, :, :L].contiguous())
        v8[b, :, :vb.shape[2]] = vb[0]
        v8s[b, :, :vbs.shape[2]] = vbs[0]
        kb, kbs, _ = qfa.quantize_qk4(k[b:b + 1, :, :L].contiguous())
        k4[b, :, :L] = kb[0]
        k4s[b, :, :L] = kbs[0]
    say("LDS fill 0x7F then decode D%d lens %s" % (D, lens))
    assert probe.probe_lds_fill(0x7F7F7F7F, 4096, 160 * 1024) == 0
    torch.cuda.synchronize()
    O, lse, used = qfa.fwd_decode(None, None, k4, k4s, v8, v8s, Smax, scale, q_bf16=q, num_splits=3,
                                  kv_lens=kv_lens)
    torch.cuda.synchronize()
    Og = to_np(O)
    assert np.isfinite(Og).all()
    rows = np.array([(b, h, 0) for b in range(B) for h in range(Hq)], dtype=np.int64)
    res = oracle.decode_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, scale, used, kv_lens=lens,
                             exact=False)
    compare_o(Og[rows[:, 0], rows[:, 1]], res["O_q"], to_np(lse)[rows[:, 0], rows[:, 1]], res["lse_q"],
              label="decode-after-lds-fill-D%d" % D)


@pytest.mark.parametrize("lo,hi", [(-1.0, 1.0), (-30.0, 30.0), (-120.0, 120.0)])
def test_exp2_within_one_ulp_of_correctly_rounded(probe, lo, hi):
    """The kernels' exponential (v_exp_f32) against the correctly rounded
    binary32 2^x, over the arguments the softmax sees: at most one ulp off.
    The oracle decides P codes from the correctly rounded binary32 value, so
    the two decisions can differ only where 256 * 2^(y - m') lies within that
    ulp of an E4M3 rounding midpoint."""
    rng = np.random.default_rng(int(hi))
    n = 1 << 20
    x = rng.uniform(lo, hi, n).astype(np.float32)
    xt = torch.from_numpy(x).cuda()
    out = torch.empty_like(xt)
    say("exp2 probe [%g, %g], %d arguments" % (lo, hi, n))
    assert probe.probe_exp2(xt.data_ptr(), n, out.data_ptr()) == 0
    torch.cuda.synchronize()
    g = to_np(out)
    cr = np.exp2(x.astype(np.float64)).astype(np.float32)
    ok = np.isfinite(cr) & (cr >= np.float32(2.0 ** -126))          # normal results
    ulp = g[ok].view(np.int32).astype(np.int64) - cr[ok].view(np.int32).astype(np.int64)
    say("exp2 probe: %.2f%% one ulp off, max %d" % (100.0 * np.mean(ulp != 0), int(np.abs(ulp).max())))
    assert int(np.abs(ulp).max()) <= 1
