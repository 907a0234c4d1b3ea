"""Pins for the oracle's attention parts (CPU only).

(a) exact attention and the online-softmax machinery of (c) are checked against
torch's float64 softmax (an independent library) with bottom-right causal masks
and GQA; (c)'s quantised path is checked with closed-form special cases,
invariants, and a brute-force recomputation of tiny inputs that uses torch's
float8 rounding instead of the oracle's encoder.

(c) takes pre-scaled query rows q' = c2 q (c2 = softmax_scale * log2 e), so
q' . k is the logit in log2 units; the exact references below multiply by c2
in binary64 before calling it.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def c2d(scale):
    """softmax_scale * log2 e in binary64, with the scale rounded to binary32 as
    the oracle receives it."""
    return float(np.float32(scale)) * math.log2(math.e)


def torch_attention(Q, K, V, Sq, causal, scale, qpos):
    """Library reference: softmax(scale * Q K^T) V in float64 with masks."""
    q = torch.from_numpy(Q)
    k = torch.from_numpy(K)
    v = torch.from_numpy(V)
    L = K.shape[0]
    s = (q @ k.T) * scale
    if causal:
        j = torch.arange(L)[None, :]
        i = torch.from_numpy(np.asarray(qpos))[:, None]
        s = s.masked_fill(j > i + (L - Sq), float("-inf"))
    lse = torch.logsumexp(s, dim=1)
    p = torch.softmax(s, dim=1)
    return (p @ v).numpy(), lse.numpy()


@pytest.mark.parametrize("L,Sq,causal", [(200, 200, True), (300, 40, True), (129, 129, False),
                                         (700, 700, True), (64, 1, False)])
def test_exact_attention_matches_torch(L, Sq, causal):
    rng = np.random.default_rng(L + Sq)
    D = 64
    Q = rng.standard_normal((Sq, D))
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    qpos = np.arange(Sq)
    O, lse = oracle.attn_exact_rows(Q, qpos, K, V, Sq, causal, 0.125)
    Or, lr = torch_attention(Q, K, V, Sq, causal, 0.125, qpos)
    assert np.abs(O - Or).max() < 1e-12
    assert np.abs(lse - lr).max() < 1e-12


@pytest.mark.parametrize("L,Sq,causal,split", [(300, 300, True, 0), (700, 50, True, 0), (1000, 1, False, 1),
                                               (1000, 1, False, 3), (1000, 1, False, 7), (128, 128, False, 0),
                                               (257, 1, False, 2)])
def test_online_schedule_identity_quantizer_equals_softmax(L, Sq, causal, split):
    """With identity quantizers the tiled online softmax (and the split merge)
    must reproduce full softmax attention: the exactness claim of FlashAttention
    tiling in the tutorial's section '注意力慢在哪儿'."""
    rng = np.random.default_rng(L * 7 + Sq)
    D = 64
    Q = rng.standard_normal((Sq, D)) * 2
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    qpos = np.arange(Sq)
    O, lse = oracle.attn_quant_rows(Q * c2d(0.125), qpos, K, V, Sq, causal, 0.125, split_tiles=split,
                                    quantize_p=False, fp32_arg=False)
    Or, lr = torch_attention(Q, K, V, Sq, causal, float(np.float32(0.125)), qpos)
    assert np.abs(O - Or).max() < 1e-12
    assert np.abs(lse - lr).max() < 1e-11


def test_compensation_identity_restores_logits():
    """Smoothing K by per-block means and adding back q.Kbar per (row, tile) is an
    algebraic identity: with identity quantizers it equals plain attention.  A
    dropped or sign-flipped compensation term fails this."""
    rng = np.random.default_rng(21)
    L, Sq, D = 400, 400, 64
    Q = rng.standard_normal((Sq, D))
    K = rng.standard_normal((L, D)) + rng.normal(0, 3, (1, D))
    V = rng.standard_normal((L, D))
    nt = (L + 127) // 128
    Kbar = np.stack([K[t * 128:(t + 1) * 128].mean(axis=0) for t in range(nt)])
    Ks = K - np.repeat(Kbar, 128, axis=0)[:L]
    qpos = np.arange(Sq)
    O, lse = oracle.attn_quant_rows(Q * c2d(0.125), qpos, Ks, V, Sq, True, 0.125, Qc=Q, Kbar=Kbar,
                                    quantize_p=False, fp32_arg=False)
    Or, lr = torch_attention(Q, K, V, Sq, True, float(np.float32(0.125)), qpos)
    assert np.abs(O - Or).max() < 1e-10
    assert np.abs(lse - lr).max() < 1e-10
    # without the compensation term the result is different (the term matters)
    O2, _ = oracle.attn_quant_rows(Q * c2d(0.125), qpos, Ks, V, Sq, True, 0.125, quantize_p=False,
                                   fp32_arg=False)
    assert np.abs(O2 - Or).max() > 1e-3


def _quantized_inputs(rng, Sq, L, D, scale_q=1.0, softmax_scale=0.125):
    """Decoded Q' (quantised as fl32(q * c2)), K and V of random bf16 inputs."""
    def bf(x):
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q = bf(rng.standard_normal((1, 1, Sq, D)) * scale_q)
    k = bf(rng.standard_normal((1, 1, L, D)))
    v = bf(rng.standard_normal((1, 1, L, D)))
    qc, qs, _ = oracle.quantize_qk4(q, prescale=oracle.exp2_scale(softmax_scale))
    kc, ks, _ = oracle.quantize_qk4(k)
    vc, vs = oracle.quantize_v8(v)
    return (oracle.dequant_qk4(qc, qs)[0, 0], oracle.dequant_qk4(kc, ks)[0, 0],
            oracle.dequant_v8(vc[0, 0], vs[0, 0], L))


def _e4m3_torch(x):
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_single_tile_equals_two_pass_definition():
    """S_kv <= 128: one tile, so m = ceil(row max) (log2 units, integer grid)
    and P8 = E4M3(256 * 2^(s - m)).  Brute force with numpy exp2 and torch's
    float8 rounding."""
    rng = np.random.default_rng(23)
    Sq, L, D = 20, 100, 64
    Qd, Kd, Vd = _quantized_inputs(rng, Sq, L, D, scale_q=3.0)
    scale = float(np.float32(0.125))
    O, lse = oracle.attn_quant_rows(Qd, np.arange(Sq), Kd, Vd, Sq, False, scale, fp32_arg=False)
    s = Qd @ Kd.T  # log2 units (Q' carries the scale)
    m = np.ceil(s.max(axis=1, keepdims=True))
    p = _e4m3_torch(256.0 * np.exp2(s - m))
    Oref = (p @ Vd) / p.sum(axis=1, keepdims=True)
    lref = math.log(2) * (m[:, 0] + np.log2(p.sum(axis=1) / 256.0))
    assert np.abs(O - Oref).max() < 1e-12
    assert np.abs(lse - lref).max() < 1e-12


def test_two_tiles_online_schedule_bruteforce():
    """Two 128-token tiles: codes of tile 1 are taken against m1 = ceil(max of
    tile 1), codes of tile 2 against m2 = max(m1, ceil(max of tile 2)); l and O
    are rescaled by 2^(m1 - m2).  Recomputed by brute force (numpy + torch
    float8)."""
    rng = np.random.default_rng(29)
    Sq, L, D = 8, 200, 64
    Qd, Kd, Vd = _quantized_inputs(rng, Sq, L, D, scale_q=3.0)
    scale = float(np.float32(0.125))
    O, _ = oracle.attn_quant_rows(Qd, np.arange(Sq), Kd, Vd, Sq, False, scale, fp32_arg=False)
    s = Qd @ Kd.T  # log2 units
    s1, s2 = s[:, :128], s[:, 128:]
    m1 = np.ceil(s1.max(axis=1, keepdims=True))
    m2 = np.maximum(m1, np.ceil(s2.max(axis=1, keepdims=True)))
    p1 = _e4m3_torch(256.0 * np.exp2(s1 - m1))
    p2 = _e4m3_torch(256.0 * np.exp2(s2 - m2))
    a = np.exp2(m1 - m2)
    num = a * (p1 @ Vd[:128]) + p2 @ Vd[128:]
    den = a * p1.sum(axis=1, keepdims=True) + p2.sum(axis=1, keepdims=True)
    assert np.abs(O - num / den).max() < 1e-12
    # on the integer grid the schedule barely matters: codes against the final
    # max give the same O except where a code crosses into E4M3's subnormal
    # range (measured ~1e-5) ...
    pf = _e4m3_torch(256.0 * np.exp2(s - m2))
    Of = (pf @ Vd) / pf.sum(axis=1, keepdims=True)
    assert np.abs(Of - O).max() < 1e-4
    # ... whereas a reference point off the grid changes many codes (~3e-2)
    pr = _e4m3_torch(256.0 * np.exp2(s - s.max(axis=1, keepdims=True)))
    Or = (pr @ Vd) / pr.sum(axis=1, keepdims=True)
    assert np.abs(Or - O).max() > 1e-3


def test_special_cases_quantized():
    rng = np.random.default_rng(31)
    Sq, L, D = 300, 300, 64
    Qd, Kd, Vd = _quantized_inputs(rng, Sq, L, D)
    qpos = np.arange(Sq)
    # causal row 0 sees only key 0: O = decoded v8[0]
    O, lse = oracle.attn_quant_rows(Qd, qpos, Kd, Vd, Sq, True, 0.125)
    assert np.array_equal(O[0], Vd[0])
    # Q = 0: every visible logit is 0 -> all P codes equal -> O = mean of visible V rows
    O0, _ = oracle.attn_quant_rows(np.zeros_like(Qd), qpos, Kd, Vd, Sq, True, 0.125)
    for i in (0, 5, 127, 128, 299):
        assert np.abs(O0[i] - Vd[:i + 1].mean(axis=0)).max() < 1e-13
    # constant V rows: O is exactly that row (convex combination of equal rows)
    Vc = np.tile(Vd[7:8], (L, 1))
    Oc, _ = oracle.attn_quant_rows(Qd, qpos, Kd, Vc, Sq, True, 0.125)
    assert np.abs(Oc - Vd[7]).max() < 1e-13


def test_integer_log2_shift_invariance():
    """Adding an integer k (log2 units) to every logit of a row scales every
    P code by 2^k exactly (E4M3 rounding commutes with powers of two), so O is
    bit-identical and LSE moves by k ln 2.  The shift is injected through the
    rank-one term (Kbar constant across tiles)."""
    rng = np.random.default_rng(37)
    Sq, L, D = 16, 400, 64
    Qd, Kd, Vd = _quantized_inputs(rng, Sq, L, D, scale_q=2.0)
    scale = 0.125
    c2 = float(np.float32(scale)) * math.log2(math.e)
    nt = (L + 127) // 128
    Qc = np.zeros((Sq, D))
    Qc[:, 0] = 1.0
    k = 3
    Kbar = np.zeros((nt, D))
    Kbar[:, 0] = k / c2
    O1, l1 = oracle.attn_quant_rows(Qd, np.arange(Sq), Kd, Vd, Sq, False, scale, fp32_arg=False)
    O2, l2 = oracle.attn_quant_rows(Qd, np.arange(Sq), Kd, Vd, Sq, False, scale, Qc=Qc, Kbar=Kbar,
                                    fp32_arg=False)
    assert np.abs(O1 - O2).max() < 1e-14
    assert np.abs((l2 - l1) - k * math.log(2)).max() < 1e-12


def test_no_visible_key_and_empty_splits():
    rng = np.random.default_rng(41)
    D = 64
    # S_q > S_kv causal: the first rows see nothing
    Q = rng.standard_normal((10, D))
    K = rng.standard_normal((4, D))
    V = rng.standard_normal((4, D))
    O, lse = oracle.attn_quant_rows(Q, np.arange(10), K, V, 10, True, 0.125)
    assert (O[:6] == 0).all() and np.isneginf(lse[:6]).all()
    assert np.isfinite(lse[6:]).all()
    Ox, lx = oracle.attn_exact_rows(Q, np.arange(10), K, V, 10, True, 0.125)
    assert (Ox[:6] == 0).all() and np.isneginf(lx[:6]).all()
    # decode: 300 keys, 4 tiles per split of 3 tiles -> split 1 holds tiles 3 (partial)
    Q1 = rng.standard_normal((1, D))
    K1 = rng.standard_normal((300, D))
    V1 = rng.standard_normal((300, D))
    Oa, la = oracle.attn_quant_rows(Q1 * c2d(0.125), np.zeros(1, np.int64), K1, V1, 1, False, 0.125,
                                    split_tiles=2, quantize_p=False, fp32_arg=False)
    Or, lr = torch_attention(Q1, K1, V1, 1, False, float(np.float32(0.125)), [0])
    assert np.abs(Oa - Or).max() < 1e-12 and abs(la[0] - lr[0]) < 1e-12


def test_fp32_argument_close_to_fp64_argument():
    """Forming the exponent argument in binary32 only moves rare P codes across a
    rounding boundary; O stays within 1e-5 of the binary64-argument result."""
    rng = np.random.default_rng(43)
    Sq, L, D = 64, 700, 128
    scale = 1 / math.sqrt(128)
    Qd, Kd, Vd = _quantized_inputs(rng, Sq, L, D, scale_q=2.0, softmax_scale=scale)
    Oa, la = oracle.attn_quant_rows(Qd, np.arange(Sq), Kd, Vd, Sq, True, scale, fp32_arg=True)
    Ob, lb = oracle.attn_quant_rows(Qd, np.arange(Sq), Kd, Vd, Sq, True, scale, fp32_arg=False)
    assert np.abs(Oa - Ob).max() < 1e-5
    assert np.abs(la - lb).max() < 1e-5


def test_gqa_mapping_and_causal_alignment_in_driver():
    """The row driver maps query head h to kv head h // (Hq/Hkv); checked on the
    exact path against torch with repeat_interleave (library)."""
    rng = np.random.default_rng(47)
    B, Hq, Hkv, Sq, L, D = 1, 4, 2, 40, 150, 64

    def bf(x):
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q = bf(rng.standard_normal((B, Hq, Sq, D)))
    k = bf(rng.standard_normal((B, Hkv, L, D)) + np.arange(Hkv)[None, :, None, None] * 2)
    v = bf(rng.standard_normal((B, Hkv, L, D)) + np.arange(Hkv)[None, :, None, None] * 5)
    rows = [(0, h, i) for h in range(Hq) for i in (0, 7, 39)]
    res = oracle.prefill_rows(q, k, v, rows, True, 0.125)
    qf, kf, vf = oracle.bf16_to_f64(q), oracle.bf16_to_f64(k), oracle.bf16_to_f64(v)
    kr = np.repeat(kf, Hq // Hkv, axis=1)
    vr = np.repeat(vf, Hq // Hkv, axis=1)
    for n, (b, h, i) in enumerate(rows):
        Or, lr = torch_attention(qf[b, h], kr[b, h], vr[b, h], Sq, True, 0.125, np.arange(Sq))
        assert np.abs(res["O_x"][n] - Or[i]).max() < 1e-12
        assert abs(res["lse_x"][n] - lr[i]) < 1e-12
    # the quantised result is close to exact (sanity only; accuracy is unpinned)
    err = np.linalg.norm(res["O_q"] - res["O_x"]) / np.linalg.norm(res["O_x"])
    assert err < 0.2


@pytest.mark.parametrize("fp32_arg", [False, True])
def test_split_schedule_invariance_on_integer_grid(fp32_arg):
    """Split-KV decode (log-sum-exp merge of independent splits) matches the
    single-split result: each split's P codes are power-of-two rescalings of
    the single-split codes except in E4M3's subnormal range (~1e-5 effect)."""
    rng = np.random.default_rng(53)
    L, D = 2000, 128
    scale = 1 / math.sqrt(128)
    Qd, Kd, Vd = _quantized_inputs(rng, 4, L, D, scale_q=2.0, softmax_scale=scale)
    O1, l1 = oracle.attn_quant_rows(Qd, np.zeros(4, np.int64), Kd, Vd, 1, False, scale, split_tiles=0,
                                    fp32_arg=fp32_arg)
    for per in (1, 3, 7):
        Os, ls = oracle.attn_quant_rows(Qd, np.zeros(4, np.int64), Kd, Vd, 1, False, scale, split_tiles=per,
                                        fp32_arg=fp32_arg)
        assert np.abs(Os - O1).max() < 1e-4
        assert np.abs(ls - l1).max() < 1e-4


def test_fp32_argument_with_compensation_close_to_fp64():
    """With the compensation the binary32 argument fl32(S + delta32) rounds;
    that only moves rare codes across a rounding boundary: O within 1e-5 of
    the binary64 path, and split schedules agree to 1e-4."""
    rng = np.random.default_rng(59)
    Sq, L, D = 32, 900, 128
    scale = 1 / math.sqrt(128)
    Qd, Kd, Vd = _quantized_inputs(rng, Sq, L, D, scale_q=2.0, softmax_scale=scale)
    nt = (L + 127) // 128
    Qc = rng.standard_normal((Sq, D))
    Kbar = rng.normal(0, 3, (nt, D))
    Oa, la = oracle.attn_quant_rows(Qd, np.arange(Sq), Kd, Vd, Sq, True, scale, Qc=Qc, Kbar=Kbar, fp32_arg=True)
    Ob, lb = oracle.attn_quant_rows(Qd, np.arange(Sq), Kd, Vd, Sq, True, scale, Qc=Qc, Kbar=Kbar, fp32_arg=False)
    assert np.abs(Oa - Ob).max() < 1e-5
    assert np.abs(la - lb).max() < 1e-5
    Q1 = Qd[:2]
    O1, l1 = oracle.attn_quant_rows(Q1, np.zeros(2, np.int64), Kd, Vd, 1, False, scale, Qc=Qc[:2], Kbar=Kbar)
    for per in (1, 3):
        Os, ls = oracle.attn_quant_rows(Q1, np.zeros(2, np.int64), Kd, Vd, 1, False, scale, Qc=Qc[:2], Kbar=Kbar,
                                        split_tiles=per)
        assert np.abs(Os - O1).max() < 1e-4
        assert np.abs(ls - l1).max() < 1e-4


# ----------------------------------------------------------------------------- P/V format variants
def _two_block_case(y_b, vA, vB, L=64, D=4):
    """One query row against 64 keys in two 32-key blocks: logit (log2 units)
    0 in block A, y_b in block B; V rows vA in A and vB in B.  Q and K are
    passed decoded, so the logits are exact."""
    Q = np.zeros((1, D))
    Q[0, 0] = 1.0
    K = np.zeros((L, D))
    K[32:, 0] = y_b
    V = np.zeros((L, D))
    V[:32] = vA
    V[32:] = vB
    return Q, K, V


@pytest.mark.parametrize("p_mode", [oracle.P_E4M3, oracle.P_E4M3_BLOCK, oracle.P_E2M1_BLOCK])
def test_block_p_scale_closed_form(p_mode):
    """Block A at logit 0 and block B at logit -20.  With one P scale per row
    (the method) block B's code 256 * 2^-20 = 2^-12 rounds to E4M3 zero, so
    O = vA.  With a scale per (row, 32 keys) block B is coded against its own
    max (code 256 or E2M1 4, exact) and weighted 2^-20, so
    O = (vA + 2^-20 vB) / (1 + 2^-20) and LSE = ln(32 (1 + 2^-20))."""
    vA = np.array([1.0, 0.5, -2.0, 0.0])
    vB = np.array([3.0, -2.0, 6.0, 1.0])
    Q, K, V = _two_block_case(-20.0, vA, vB)
    O, lse = oracle.attn_quant_rows(Q, np.zeros(1, np.int64), K, V, 1, False, 0.125, p_mode=p_mode)
    if p_mode == oracle.P_E4M3:
        assert np.array_equal(O[0], vA)
        assert abs(lse[0] - math.log(32.0)) < 1e-15
    else:
        w = 2.0**-20
        assert np.abs(O[0] - (vA + w * vB) / (1 + w)).max() < 1e-15
        assert abs(lse[0] - math.log(32.0 * (1 + w))) < 1e-14


def test_block_p_scale_floor():
    """A block more than 64 binades below the row is coded against m - 64:
    at logit -70 its MXFP4 code is E2M1(4 * 2^-6) = 0 (smallest non-zero 1/2),
    so it contributes nothing; its E4M3 code 256 * 2^-6 = 4 is exact, so there
    it still contributes 2^-70 of its weight."""
    vA = np.array([0.0, 1.0, 0.0, 0.0])
    vB = np.array([5.0, 1.0, 0.0, 0.0])
    Q, K, V = _two_block_case(-70.0, vA, vB)
    O4, _ = oracle.attn_quant_rows(Q, np.zeros(1, np.int64), K, V, 1, False, 0.125, p_mode=oracle.P_E2M1_BLOCK)
    assert O4[0, 0] == 0.0
    O8, _ = oracle.attn_quant_rows(Q, np.zeros(1, np.int64), K, V, 1, False, 0.125, p_mode=oracle.P_E4M3_BLOCK)
    w = 2.0**-70
    assert O8[0, 0] == 5.0 * w / (1 + w)
    # causal row 10 of 64 sees keys 0..10: block B has no visible key and
    # contributes nothing; block A holds the row max, so the codes are the method's
    Qr = np.tile(Q, (64, 1))
    rng = np.random.default_rng(3)
    Kr = K.copy()
    Kr[:, 1] = rng.standard_normal(64)
    Qr[:, 1] = 1.5
    qpos = np.arange(64)
    Ob, lb = oracle.attn_quant_rows(Qr, qpos, Kr, V, 64, True, 0.125, p_mode=oracle.P_E4M3_BLOCK)
    Om, lm = oracle.attn_quant_rows(Qr, qpos, Kr, V, 64, True, 0.125, p_mode=oracle.P_E4M3)
    assert np.array_equal(Ob[:32], Om[:32]) and np.array_equal(lb[:32], lm[:32])


def _blockwise_bruteforce(s, Vd, p_mode):
    """Brute force of the per-(row, 32 keys) P scale over 128-key tiles with
    numpy exp2 and torch float8 (E4M3) or the printed E2M1 table (E2M1)."""
    import json
    import os
    table = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e2m1_magnitudes.json")))["magnitudes"]

    def e2m1(a):
        out = np.empty_like(a)
        for idx, x in np.ndenumerate(a):
            d = [abs(t - x) for t in table]
            best = min(d)
            c = [i for i, z in enumerate(d) if z == best]
            if len(c) > 1:
                c = [i for i in c if i % 2 == 0]
            out[idx] = table[c[0]]
        return out

    n, L = s.shape
    m = np.full((n, 1), -np.inf)
    num = np.zeros((n, Vd.shape[1]))
    den = np.zeros((n, 1))
    for t0 in range(0, L, 128):
        st = s[:, t0:t0 + 128]
        mn = np.maximum(m, np.ceil(st.max(axis=1, keepdims=True)))
        a = np.where(np.isneginf(m), 0.0, np.exp2(m - mn))
        num *= a
        den *= a
        for b0 in range(0, st.shape[1], 32):
            sb = st[:, b0:b0 + 32]
            e = np.maximum(np.ceil(sb.max(axis=1, keepdims=True)), mn - 64)
            if p_mode == oracle.P_E4M3_BLOCK:
                p = _e4m3_torch(256.0 * np.exp2(sb - e))
            else:
                p = e2m1(4.0 * np.exp2(sb - e))
            p = p * np.exp2(e - mn)
            num += p @ Vd[t0 + b0:t0 + b0 + sb.shape[1]]
            den += p.sum(axis=1, keepdims=True)
        m = mn
    return num / den


@pytest.mark.parametrize("p_mode", [oracle.P_E4M3_BLOCK, oracle.P_E2M1_BLOCK])
def test_block_p_scale_bruteforce(p_mode):
    """Three tiles (the last one ragged) of random logits with a spread of
    block maxima, recomputed by brute force."""
    rng = np.random.default_rng(53)
    Sq, L, D = 6, 300, 32
    Qd, Kd, Vd = _quantized_inputs(rng, Sq, L, D, scale_q=3.0)
    Kd[64:96] *= 0.25    # a block with small logits
    Kd[200:232] -= 2.0   # and one shifted
    scale = float(np.float32(0.125))
    O, _ = oracle.attn_quant_rows(Qd, np.arange(Sq), Kd, Vd, Sq, False, scale, fp32_arg=False, p_mode=p_mode)
    ref = _blockwise_bruteforce(Qd @ Kd.T, Vd, p_mode)
    assert np.abs(O - ref).max() < 1e-12
    # the row scale of the method gives a different result
    O1, _ = oracle.attn_quant_rows(Qd, np.arange(Sq), Kd, Vd, Sq, False, scale, fp32_arg=False)
    assert np.abs(O1 - O).max() > 1e-6


def test_block_p_scale_equals_row_scale_when_every_block_reaches_the_max():
    """If every 32-key block holds a key at the tile's max, every block's
    exponent is the row's and the per-block E4M3 codes are the method's."""
    rng = np.random.default_rng(59)
    L, D = 256, 16
    Q = np.zeros((3, D))
    Q[:, 0] = 1.0
    K = np.zeros((L, D))
    K[:, 0] = -np.abs(rng.standard_normal(L)) * 3.0
    K[::32, 0] = 0.5   # the tile max, once per block
    V = rng.standard_normal((L, D))
    O1, l1 = oracle.attn_quant_rows(Q, np.zeros(3, np.int64), K, V, 1, False, 0.125)
    O2, l2 = oracle.attn_quant_rows(Q, np.zeros(3, np.int64), K, V, 1, False, 0.125, p_mode=oracle.P_E4M3_BLOCK)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("pv", [oracle.PV_FP8_BLOCKP, oracle.PV_FP4])
def test_pv_variants_close_to_exact_attention(pv):
    """The variants run end to end through the drivers.  On N(0,1) data every
    block's max lies within a few binades of its row's, so per-block FP8 P
    scales give the method's codes exactly; MXFP4 P and V add error on top of
    the method's (which MXFP4 Q and K dominate)."""
    rng = np.random.default_rng(61)
    B, Hq, Hkv, S, D = 1, 2, 1, 200, 64

    def bf(x):
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q = bf(rng.standard_normal((B, Hq, S, D)))
    k = bf(rng.standard_normal((B, Hkv, S, D)))
    v = bf(rng.standard_normal((B, Hkv, S, D)))
    rows = np.array([(0, h, i) for h in range(Hq) for i in range(0, S, 7)])

    def rel(r):
        return np.linalg.norm(r["O_q"] - r["O_x"]) / np.linalg.norm(r["O_x"])
    r0 = oracle.prefill_rows(q, k, v, rows, True, 0.125)
    r1 = oracle.prefill_rows(q, k, v, rows, True, 0.125, pv=pv)
    if pv == oracle.PV_FP8_BLOCKP:
        assert np.array_equal(r1["O_q"], r0["O_q"])
    else:
        assert rel(r0) < rel(r1) < 2.5 * rel(r0)
    d0 = oracle.decode_rows(q[:, :, :1], k, v, np.array([(0, 0, 0), (0, 1, 0)]), 0.125, 2)
    d1 = oracle.decode_rows(q[:, :, :1], k, v, np.array([(0, 0, 0), (0, 1, 0)]), 0.125, 2, pv=pv)
    assert rel(d1) < 2.5 * rel(d0) + 1e-12


def test_nvfp4_qk_more_accurate_than_mxfp4():
    """Q and K in NVFP4 (blocks of 16 with E4M3 scales) run through the same
    online-softmax schedule; with twice as many, finer scales the result is
    closer to exact attention than with MXFP4 ([FA4tut] "FP4 只有约 15 个可表示的数":
    NVFP4 matches local dynamic range more often)."""
    rng = np.random.default_rng(61)
    B, Hq, Hkv, S, D = 1, 2, 1, 200, 64

    def bf(x):
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q = bf(rng.standard_normal((B, Hq, S, D)))
    k = bf(rng.standard_normal((B, Hkv, S, D)))
    v = bf(rng.standard_normal((B, Hkv, S, D)))
    rows = np.array([(0, h, i) for h in range(Hq) for i in range(0, S, 7)])
    c2 = oracle.exp2_scale(0.125)
    gq = oracle.nvfp4_tensor_scale(float(np.abs(oracle.bf16_to_f64(q) * np.float32(c2)).max()))
    gk = oracle.nvfp4_tensor_scale(float(np.abs(oracle.bf16_to_f64(k)).max()))

    def rel(r):
        return np.linalg.norm(r["O_q"] - r["O_x"]) / np.linalg.norm(r["O_x"])
    r0 = oracle.prefill_rows(q, k, v, rows, True, 0.125)
    r1 = oracle.prefill_rows(q, k, v, rows, True, 0.125, nvfp4=(gq, gk))
    assert rel(r1) < 0.8 * rel(r0)
    # a doubled tensor scale halves every block scale: where the halved scale
    # stays an E4M3 normal the decoded values are the same, so O is (almost) too
    r2 = oracle.prefill_rows(q, k, v, rows, True, 0.125, nvfp4=(gq, gk * 2))
    assert np.abs(r2["O_q"] - r1["O_q"]).max() < 1e-3
