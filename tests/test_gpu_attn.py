"""GPU prefill and split-KV decode vs the oracle (c).

Small shapes compare every row (several tiles, ragged tails, GQA packing,
head chunks, bottom-right causal alignment, rows with no visible key, the
compensation term across a 32-tile boundary).  Full workload sizes run the
kernels exactly as the benchmark launches them and compare sampled rows.
Bar: O within 3e-3 max-abs and 1e-3 relative L2 of the oracle; LSE within
1e-3; error against exact FP64 attention is reported, not gated.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import bit_quantized_attention_qk4pv8_amd as qfa
import oracle
from bit_quantized_attention_qk4pv8_amd.workloads import WORKLOADS, Workload, bf16_bits, make_inputs
from gpu_util import compare_o, sample_rows, say, to_np

pytestmark = pytest.mark.gpu


def _rand_inputs(B, Hq, Hkv, Sq, Skv, D, seed, k_offset=0.0, q_scale=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn((B, Hq, Sq, D), generator=g, device="cuda") * q_scale
    k = torch.randn((B, Hkv, Skv, D), generator=g, device="cuda")
    if k_offset:
        k += torch.randn((B, Hkv, 1, D), generator=g, device="cuda") * k_offset
    v = torch.randn((B, Hkv, Skv, D), generator=g, device="cuda")
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def _quantize_v(v, pv):
    return qfa.quantize_v4(v) if pv == qfa.QFA_PV_FP4 else qfa.quantize_v8(v)


def _gpu_prefill(q, k, v, causal, scale, smooth, fused=False, pv=qfa.QFA_PV_FP8):
    """fused: Q goes in as bf16 and the prefill kernel quantises it (q4 = q4s = NULL).
    pv: the P/V format."""
    B, Hq, Sq, D = q.shape
    Skv = k.shape[2]
    if fused:
        q4 = q4s = None
    else:
        q4, q4s, _ = qfa.quantize_qk4(q, prescale=qfa.qfa_exp2_scale(scale))
    k4, k4s, kbar = qfa.quantize_qk4(k, smooth=smooth)
    v8, v8s = _quantize_v(v, pv)
    O, lse = qfa.fwd_prefill(q4, q4s, k4, k4s, v8, v8s, Skv, causal, scale, kbar=kbar,
                             q_bf16=q if (smooth or fused) else None, pv_format=pv)
    torch.cuda.synchronize()
    return O, lse


def _check_prefill(q, k, v, causal, scale, smooth, rows, label, fused=False, pv=qfa.QFA_PV_FP8):
    B, Hq, Sq, D = q.shape
    say("prefill", label, "q", tuple(q.shape), "k", tuple(k.shape), "causal", causal, "smooth", smooth,
        "fused Q" if fused else "", "pv", pv)
    O, lse = _gpu_prefill(q, k, v, causal, scale, smooth, fused, pv)
    res = oracle.prefill_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, causal, scale, smooth=smooth,
                              pv=pv)
    Og = to_np(O)[rows[:, 0], rows[:, 1], rows[:, 2]]
    lg = to_np(lse)[rows[:, 0], rows[:, 1], rows[:, 2]]
    compare_o(Og, res["O_q"], lg, res["lse_q"], label)
    ok = np.isfinite(res["lse_x"])
    if ok.any():
        ex = res["O_x"][ok]
        err = np.linalg.norm(Og[ok] - ex) / np.linalg.norm(ex)
        cos = float(np.sum(Og[ok] * ex) / (np.linalg.norm(Og[ok]) * np.linalg.norm(ex)))
        say("%s vs exact FP64: rel-L2 %.3e cosine %.6f (reported only)" % (label, err, cos))
    return O, lse


def _all_rows(B, H, S):
    return np.array([(b, h, i) for b in range(B) for h in range(H) for i in range(S)], dtype=np.int64)


CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, smooth, k_offset, label
    (1, 2, 2, 256, 256, 64, False, False, 0.0, "tiny-shape"),
    (1, 4, 2, 300, 300, 128, True, False, 0.0, "causal-ragged-D128"),
    (1, 5, 1, 70, 333, 64, True, False, 0.0, "bottom-right-G5-D64"),
    (1, 2, 2, 100, 64, 128, True, False, 0.0, "sq>skv-empty-rows"),
    (1, 4, 1, 700, 700, 128, True, True, 3.0, "compensation-causal"),
    (1, 16, 2, 45, 1000, 128, False, False, 0.0, "noncausal-G8"),
    (1, 12, 1, 200, 200, 128, True, False, 0.0, "G12-two-head-chunks"),
    (2, 4, 4, 130, 130, 64, True, True, 3.0, "batch2-comp-D64"),
    (1, 2, 1, 129, 1001, 64, True, False, 0.0, "odd-keys-D64-8tiles"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[-1] for c in CASES])
def test_prefill_small_all_rows(case):
    B, Hq, Hkv, Sq, Skv, D, causal, smooth, koff, label = case
    q, k, v = _rand_inputs(B, Hq, Hkv, Sq, Skv, D, seed=zlib.crc32(label.encode()) % 1000, k_offset=koff, q_scale=2.0)
    _check_prefill(q, k, v, causal, 1.0 / math.sqrt(D), smooth, _all_rows(B, Hq, Sq), label)


def test_prefill_tiny_workload():
    w = WORKLOADS["tiny"]
    inp = make_inputs(w, seed=0)
    _check_prefill(inp["q"], inp["k"], inp["v"], w.causal, w.scale, w.smooth, _all_rows(1, w.Hq, w.S_q), "tiny")


def test_prefill_compensation_beyond_32_tiles():
    """Delta is recomputed every 32 key tiles (4096 keys): 64 rows over 5000 keys."""
    q, k, v = _rand_inputs(1, 2, 1, 64, 5000, 128, seed=77, k_offset=3.0)
    _check_prefill(q, k, v, False, 1 / math.sqrt(128), True, _all_rows(1, 2, 64), "comp-5000keys")


@pytest.mark.parametrize("D,S,fused", [(64, 4500, False), (128, 4200, True)])
def test_prefill_compensation_causal_many_tiles(D, S, fused):
    """Causal rows whose delta chunks (32 tiles) end inside the wave's range,
    a chunk boundary at key 4096, a ragged last tile, and tile halves of a
    chunk that lie past a wave's last tile (skipped by the delta product)."""
    q, k, v = _rand_inputs(1, 4, 2, S, S, D, seed=D + S, k_offset=3.0, q_scale=2.0)
    must = (0, 31, 32, 2047, 2048, 2049, 4063, 4064, 4095, 4096, 4097, 4127, 4128)
    rows = sample_rows(1, 4, S, 360, seed=S, must=must)
    _check_prefill(q, k, v, True, 1.0 / math.sqrt(D), True, rows, "comp-causal-D%d-S%d" % (D, S), fused=fused)


FUSED_CASES = [
    (1, 4, 2, 300, 300, 128, True, False, 0.0, "fused-causal-ragged-D128"),
    (1, 5, 1, 70, 333, 64, True, False, 0.0, "fused-bottom-right-G5-D64"),
    (1, 4, 1, 700, 700, 128, True, True, 3.0, "fused-compensation-causal"),
    (2, 4, 4, 130, 130, 64, False, True, 3.0, "fused-batch2-comp-D64"),
    (1, 2, 2, 100, 64, 128, True, False, 0.0, "fused-sq>skv-empty-rows"),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[-1] for c in FUSED_CASES])
def test_prefill_fused_q_matches_two_pass(case):
    """Q quantised inside the prefill kernel gives the same bytes as the quantiser
    pass, so O and LSE are bit-identical to the two-pass path."""
    B, Hq, Hkv, Sq, Skv, D, causal, smooth, koff, label = case
    q, k, v = _rand_inputs(B, Hq, Hkv, Sq, Skv, D, seed=zlib.crc32(label.encode()) % 1000, k_offset=koff, q_scale=2.0)
    q[..., 0, :32] = 0.0                 # an all-zero Q block (scale code 0)
    q[..., 1, 5] = 300.0                 # an outlier channel
    say("prefill fused-vs-two-pass", label, tuple(q.shape), tuple(k.shape))
    O1, l1 = _gpu_prefill(q, k, v, causal, 1.0 / math.sqrt(D), smooth)
    O2, l2 = _gpu_prefill(q, k, v, causal, 1.0 / math.sqrt(D), smooth, fused=True)
    assert torch.equal(O1, O2), label
    assert torch.equal(l1, l2), label


def test_prefill_fused_q_workload_vs_oracle():
    w = WORKLOADS["llama16k"]
    inp = make_inputs(w, seed=0)
    rows = sample_rows(1, w.Hq, w.S_q, 256, seed=3, must=(0, 127, 128, 16383))
    _check_prefill(inp["q"], inp["k"], inp["v"], w.causal, w.scale, w.smooth, rows, "llama16k-fused-q", fused=True)


def test_prefill_deterministic():
    q, k, v = _rand_inputs(1, 4, 2, 300, 300, 128, seed=5)
    O1, l1 = _gpu_prefill(q, k, v, True, 0.088, False)
    O2, l2 = _gpu_prefill(q, k, v, True, 0.088, False)
    assert torch.equal(O1, O2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name,nrows,fused", [("llama16k", 384, False), ("qwen32k", 320, True),
                                              ("long128k", 192, True)])
def test_prefill_workload_sampled(name, nrows, fused):
    """Full-size workloads, sampled rows.  qwen32k and long128k run the launch
    the benchmark times (bf16 Q quantised inside the prefill kernel); llama16k
    runs the two-pass path here and the fused one in the test above."""
    w = WORKLOADS[name]
    inp = make_inputs(w, seed=0)
    rows = sample_rows(1, w.Hq, w.S_q, nrows, seed=1, must=(0, 127, 128, 4095))
    _check_prefill(inp["q"], inp["k"], inp["v"], w.causal, w.scale, w.smooth, rows,
                   name + ("-fused-q" if fused else ""), fused=fused)


# ----------------------------------------------------------------------------- decode
def _gpu_decode(q, k, v, num_splits, kv_lens=None, smooth=False, fused=False, pv=qfa.QFA_PV_FP8):
    B, Hq, _, D = q.shape
    Smax = k.shape[2]
    if fused:
        q4 = q4s = None
    else:
        q4, q4s, _ = qfa.quantize_qk4(q, prescale=qfa.qfa_exp2_scale(1 / math.sqrt(D)))
    k4, k4s, kbar = qfa.quantize_qk4(k, smooth=smooth)
    v8, v8s = _quantize_v(v, pv)
    if kv_lens is not None:
        # a cache holds what the writer quantised: each sequence's own L_b tokens
        # (its last K-mean tile and V block cover only those)
        for b, L in enumerate(kv_lens):
            if L == 0:
                continue
            kc, ksc, kb = qfa.quantize_qk4(k[b:b + 1, :, :L].contiguous(), smooth=smooth)
            vc, vsc = _quantize_v(v[b:b + 1, :, :L].contiguous(), pv)
            k4[b:b + 1, :, :L] = kc
            k4s[b:b + 1, :, :L] = ksc
            if smooth:
                kbar[b:b + 1, :, :kb.shape[2]] = kb
            v8[b:b + 1, :, :vc.shape[2]] = vc
            v8s[b:b + 1, :, :vsc.shape[2]] = vsc
    lens = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device="cuda")
    O, lse, used = qfa.fwd_decode(q4, q4s, k4, k4s, v8, v8s, Smax, 1 / math.sqrt(D), num_splits=num_splits,
                                  kv_lens=lens, kbar=kbar, q_bf16=q if (smooth or fused) else None, pv_format=pv)
    torch.cuda.synchronize()
    return O, lse, used


def _check_decode(q, k, v, num_splits, kv_lens=None, label="", seqs=None, smooth=False, pv=qfa.QFA_PV_FP8):
    B, Hq, _, D = q.shape
    say("decode", label, "q", tuple(q.shape), "k", tuple(k.shape), "splits", num_splits, "pv", pv)
    O, lse, used = _gpu_decode(q, k, v, num_splits, kv_lens, smooth, pv=pv)
    if num_splits:
        assert used == num_splits
    seqs = list(range(B)) if seqs is None else seqs
    rows = np.array([(b, h, 0) for b in seqs for h in range(Hq)], dtype=np.int64)
    if smooth:
        res = _decode_oracle_smooth(q, k, v, rows, used, kv_lens, pv)
    else:
        res = oracle.decode_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, 1 / math.sqrt(D), used,
                                 kv_lens=kv_lens, pv=pv)
    Og = to_np(O)[rows[:, 0], rows[:, 1]]
    lg = to_np(lse)[rows[:, 0], rows[:, 1]]
    compare_o(Og, res["O_q"], lg, res["lse_q"], label)
    return used


def _decode_oracle_smooth(q, k, v, rows, splits, kv_lens, pv=oracle.PV_FP8):
    """Oracle decode with K smoothing: quantise with the oracle, run the split schedule."""
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    B, Hq, _, D = qb.shape
    Hkv, Smax = kb.shape[1], kb.shape[2]
    G = Hq // Hkv
    out = {"O_q": np.zeros((len(rows), D)), "lse_q": np.zeros(len(rows))}
    for n, (b, h, _) in enumerate(rows):
        g = h // G
        L = Smax if kv_lens is None else kv_lens[b]
        nt = (L + 127) // 128
        per = max(1, -(-nt // splits))
        kc, ks, kbar = oracle.quantize_qk4(np.ascontiguousarray(kb[b:b + 1, g:g + 1, :L]), smooth=True)
        vsl = np.ascontiguousarray(vb[b:b + 1, g:g + 1, :L])
        if pv == oracle.PV_FP4:
            vc, vs = oracle.quantize_v4(vsl)
            Vd = oracle.dequant_v4(vc[0, 0], vs[0, 0], L)
        else:
            vc, vs = oracle.quantize_v8(vsl)
            Vd = oracle.dequant_v8(vc[0, 0], vs[0, 0], L)
        qc, qs, _ = oracle.quantize_qk4(np.ascontiguousarray(qb[b:b + 1, h:h + 1]),
                                        prescale=oracle.exp2_scale(1 / math.sqrt(D)))
        O, l = oracle.attn_quant_rows(oracle.dequant_qk4(qc, qs)[0, 0], np.zeros(1, np.int64),
                                      oracle.dequant_qk4(kc, ks)[0, 0], Vd,
                                      1, False, 1 / math.sqrt(D), Qc=oracle.bf16_to_f64(qb[b, h]),
                                      Kbar=oracle.bf16_to_f64(kbar[0, 0]), split_tiles=per,
                                      p_mode=oracle._P_MODE_OF_PV[pv])
        out["O_q"][n] = O[0]
        out["lse_q"][n] = l[0]
    return out


def _random_prefill_case(i):
    """Seeded random prefill shape: GQA ratio, odd lengths (Sq > Skv too), D,
    causal, compensation and fused Q drawn independently."""
    rng = np.random.default_rng(1000 + i)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 3]))
    G = int(rng.choice([1, 2, 4, 5, 8]))
    B = int(rng.choice([1, 2]))
    Skv = int(rng.integers(1, 900))
    Sq = int(rng.integers(1, min(Skv + 120, 600)))
    causal, smooth, fused = (bool(x) for x in rng.integers(0, 2, size=3))
    koff = 3.0 if smooth else float(rng.choice([0.0, 1.0]))
    qs = float(rng.choice([1.0, 2.0]))
    return B, Hkv * G, Hkv, Sq, Skv, D, causal, smooth, fused, koff, qs


@pytest.mark.parametrize("i", range(64))
def test_prefill_random_shapes(i):
    B, Hq, Hkv, Sq, Skv, D, causal, smooth, fused, koff, qs = _random_prefill_case(i)
    label = "rand%d B%d H%d/%d S%d/%d D%d causal%d comp%d fused%d" % (i, B, Hq, Hkv, Sq, Skv, D, causal, smooth,
                                                                    fused)
    q, k, v = _rand_inputs(B, Hq, Hkv, Sq, Skv, D, seed=2000 + i, k_offset=koff, q_scale=qs)
    _check_prefill(q, k, v, causal, 1.0 / math.sqrt(D), smooth, _all_rows(B, Hq, Sq), label, fused=fused)


@pytest.mark.parametrize("i", range(200, 216))
def test_prefill_random_compensated(i):
    """The random-shape recipe with the compensation forced on (K with a
    per-channel offset): the compensated exponent argument has a full binary32
    mantissa, so these rows are where P codes near E4M3 rounding boundaries
    are decided (both sides from a binary32 exponential)."""
    B, Hq, Hkv, Sq, Skv, D, causal, _, fused, _, qs = _random_prefill_case(i)
    label = "crand%d B%d H%d/%d S%d/%d D%d causal%d fused%d" % (i, B, Hq, Hkv, Sq, Skv, D, causal, fused)
    q, k, v = _rand_inputs(B, Hq, Hkv, Sq, Skv, D, seed=2000 + i, k_offset=3.0, q_scale=qs)
    _check_prefill(q, k, v, causal, 1.0 / math.sqrt(D), True, _all_rows(B, Hq, Sq), label, fused=fused)


@pytest.mark.parametrize("i", range(24))
def test_decode_random_shapes(i):
    """Seeded random decode shape: batch, GQA ratio (up to 40 query heads per KV
    head, i.e. two row chunks), ragged cache lengths including empty ones, split
    count (0 = the library's default), D and compensation."""
    rng = np.random.default_rng(3000 + i)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 4, 8, 40]))
    B = int(rng.integers(1, 5))
    Smax = int(rng.integers(1, 5000))
    lens = [int(x) for x in rng.integers(0, Smax + 1, size=B)]
    lens[0] = Smax
    splits = int(rng.choice([0, 1, 2, 5, 16]))
    smooth = bool(rng.integers(2))
    label = "drand%d B%d H%d/%d S%d D%d splits%d comp%d" % (i, B, Hkv * G, Hkv, Smax, D, splits, smooth)
    q, k, v = _rand_inputs(B, Hkv * G, Hkv, 1, Smax, D, seed=4000 + i, k_offset=3.0 if smooth else 0.0)
    _check_decode(q, k, v, splits, kv_lens=lens, label=label, smooth=smooth)


@pytest.mark.parametrize("pv", [qfa.QFA_PV_FP8_BLOCKP, qfa.QFA_PV_FP4], ids=["blockp", "fp4"])
@pytest.mark.parametrize("i", range(100, 116))
def test_decode_formats_random_shapes(i, pv):
    """The random decode recipe in the P/V contrast formats (block-scaled E4M3
    P with the compensation as drawn, MXFP4 P/V without it)."""
    rng = np.random.default_rng(3000 + i)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 4, 8, 40]))
    B = int(rng.integers(1, 5))
    Smax = int(rng.integers(1, 5000))
    lens = [int(x) for x in rng.integers(0, Smax + 1, size=B)]
    lens[0] = Smax
    splits = int(rng.choice([0, 1, 2, 5, 16]))
    smooth = bool(rng.integers(2)) and pv == qfa.QFA_PV_FP8_BLOCKP
    label = "drand%d-pv%d B%d H%d/%d S%d D%d splits%d comp%d" % (i, pv, B, Hkv * G, Hkv, Smax, D, splits, smooth)
    q, k, v = _rand_inputs(B, Hkv * G, Hkv, 1, Smax, D, seed=4000 + i, k_offset=3.0 if smooth else 0.0)
    _check_decode(q, k, v, splits, kv_lens=lens, label=label, smooth=smooth, pv=pv)


@pytest.mark.parametrize("splits", [3, 0, 1])
def test_decode_small_varlen(splits):
    q, k, v = _rand_inputs(3, 8, 2, 1, 1000, 128, seed=11, q_scale=2.0)
    _check_decode(q, k, v, splits, kv_lens=[1000, 517, 0], label="varlen-splits%d" % splits)


def test_decode_d64_and_more_splits_than_tiles():
    q, k, v = _rand_inputs(2, 4, 4, 1, 300, 64, seed=12)
    _check_decode(q, k, v, 7, label="d64-7splits")   # 3 tiles: splits 3..6 are empty


def test_decode_more_than_64_splits():
    """The LSE merge takes split weights 64 lanes at a time: 70 splits of 9000 keys
    (71 tiles) run a full chunk and a partial one."""
    q, k, v = _rand_inputs(1, 4, 1, 1, 9000, 128, seed=14)
    used = _check_decode(q, k, v, 70, label="decode-70splits")
    assert used == 70


def test_decode_compensation():
    q, k, v = _rand_inputs(2, 4, 1, 1, 5000, 128, seed=13, k_offset=3.0)
    _check_decode(q, k, v, 2, label="decode-comp", smooth=True)


def test_decode_workload_sampled_sequences():
    w = WORKLOADS["decode"]
    inp = make_inputs(w, seed=0)
    seqs = [0, 17, 42, 63]
    used = _check_decode(inp["q"], inp["k"], inp["v"], w.num_splits, label="decode-B64", seqs=seqs)
    assert used == 16
    # error of the method against exact FP64 attention on the same rows (reported, not gated)
    O, _, _ = _gpu_decode(inp["q"], inp["k"], inp["v"], w.num_splits)
    rows = np.array([(b, h, 0) for b in seqs for h in range(w.Hq)], dtype=np.int64)
    ex = oracle.prefill_rows(bf16_bits(inp["q"]), bf16_bits(inp["k"]), bf16_bits(inp["v"]), rows, False, w.scale)
    Og = to_np(O)[rows[:, 0], rows[:, 1]]
    err = np.linalg.norm(Og - ex["O_x"]) / np.linalg.norm(ex["O_x"])
    cos = float(np.sum(Og * ex["O_x"]) / (np.linalg.norm(Og) * np.linalg.norm(ex["O_x"])))
    say("decode-B64 vs exact FP64: rel-L2 %.3e cosine %.6f (reported only)" % (err, cos))


@pytest.mark.parametrize("smooth", [False, True])
def test_decode_fused_q_matches_two_pass(smooth):
    q, k, v = _rand_inputs(3, 8, 2, 1, 1000, 128, seed=21, q_scale=2.0, k_offset=3.0 if smooth else 0.0)
    say("decode fused-vs-two-pass smooth", smooth)
    O1, l1, u1 = _gpu_decode(q, k, v, 3, kv_lens=[1000, 517, 0], smooth=smooth)
    O2, l2, u2 = _gpu_decode(q, k, v, 3, kv_lens=[1000, 517, 0], smooth=smooth, fused=True)
    assert u1 == u2 == 3
    assert torch.equal(O1, O2) and torch.equal(l1, l2)


# ----------------------------------------------------------------------------- P/V formats and extreme logits
BLOCKP_CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, smooth, k_offset, label
    (1, 4, 1, 333, 333, 128, True, False, 0.0, "blockp-causal-ragged-G4"),
    (2, 5, 1, 70, 700, 64, False, False, 0.0, "blockp-d64-G5"),
    (1, 2, 1, 200, 600, 128, True, True, 3.0, "blockp-compensation"),
]


@pytest.mark.parametrize("pv", [qfa.QFA_PV_FP8_BLOCKP, qfa.QFA_PV_FP4], ids=["blockp", "fp4"])
@pytest.mark.parametrize("case", BLOCKP_CASES, ids=[c[-1] for c in BLOCKP_CASES])
def test_prefill_pv_formats_small_all_rows(case, pv):
    B, Hq, Hkv, Sq, Skv, D, causal, smooth, koff, label = case
    q, k, v = _rand_inputs(B, Hq, Hkv, Sq, Skv, D, seed=zlib.crc32(label.encode()) % 1000, k_offset=koff, q_scale=2.0)
    _check_prefill(q, k, v, causal, 1.0 / math.sqrt(D), smooth, _all_rows(B, Hq, Sq), label, fused=True, pv=pv)


def test_prefill_fp4_two_pass_q_and_sq_gt_skv():
    """QK4PV4 with Q quantised by the separate pass, and rows with no visible key."""
    q, k, v = _rand_inputs(1, 4, 2, 300, 200, 128, seed=31, q_scale=2.0)
    _check_prefill(q, k, v, True, 1.0 / math.sqrt(128), False, _all_rows(1, 4, 300), "fp4-sq>skv",
                   pv=qfa.QFA_PV_FP4)


def _spread_inputs(seed, Sq=128, Skv=1000, D=128):
    """Strongly peaked rows whose 32-key blocks sit many binades apart: Q and
    K scaled up, the keys of every other block scaled down."""
    q, k, v = _rand_inputs(1, 2, 1, Sq, Skv, D, seed=seed, q_scale=4.0)
    k = k.float()
    k *= 2.0
    blk = (torch.arange(Skv, device="cuda") // 32) % 2 == 1
    k[:, :, blk] *= 0.15
    return q, k.to(torch.bfloat16), v


def test_prefill_blockp_differs_where_blocks_spread():
    """Where block maxima lie far below the row's, per-block P scales keep
    codes that one scale per row rounds to zero: the two formats then give
    different O, each matching its own oracle."""
    q, k, v = _spread_inputs(seed=5)
    rows = _all_rows(1, 2, 128)
    O1, _ = _check_prefill(q, k, v, False, 1.0 / math.sqrt(128), False, rows, "spread-blockp", fused=True,
                           pv=qfa.QFA_PV_FP8_BLOCKP)
    O0, _ = _check_prefill(q, k, v, False, 1.0 / math.sqrt(128), False, rows, "spread-fp8", fused=True)
    d = (O1 - O0).abs().max().item()
    say("spread: max |O_blockp - O_fp8| = %.3e" % d)
    assert d > 0


@pytest.mark.parametrize("pv,D", [(qfa.QFA_PV_FP8, 128), (qfa.QFA_PV_FP8, 64), (qfa.QFA_PV_FP8_BLOCKP, 128),
                                  (qfa.QFA_PV_FP4, 128)])
def test_prefill_extreme_logits_far_and_rebase(pv, D):
    """Logits far beyond 100 in log2 units (the kernel's subtract-first path)
    and a row max that climbs by more than 64 binades across the key range
    (the frame rebase of O and l; for the method's format at both head
    dimensions, whose kernels keep O in fixed accumulation registers)."""
    Skv = 1200
    q, k, v = _rand_inputs(1, 2, 1, 64, Skv, D, seed=9, q_scale=30.0)
    k = (k.float() * (1.0 + torch.arange(Skv, device="cuda").float() / 200.0)[None, None, :, None]).to(torch.bfloat16)
    _check_prefill(q, k, v, False, 1.0 / math.sqrt(D), False, _all_rows(1, 2, 64), "extreme-logits", fused=True,
                   pv=pv)


@pytest.mark.parametrize("pv", [qfa.QFA_PV_FP8, qfa.QFA_PV_FP8_BLOCKP, qfa.QFA_PV_FP4])
def test_decode_extreme_logits(pv):
    Skv, D = 1200, 128
    q, k, v = _rand_inputs(2, 8, 2, 1, Skv, D, seed=10, q_scale=30.0)
    k = (k.float() * (1.0 + torch.arange(Skv, device="cuda").float() / 200.0)[None, None, :, None]).to(torch.bfloat16)
    _check_decode(q, k, v, 3, kv_lens=[1200, 700], label="decode-extreme", pv=pv)


@pytest.mark.parametrize("pv", [qfa.QFA_PV_FP8_BLOCKP, qfa.QFA_PV_FP4], ids=["blockp", "fp4"])
@pytest.mark.parametrize("smooth", [False, True])
def test_decode_pv_formats(smooth, pv):
    q, k, v = _rand_inputs(3, 8, 2, 1, 1000, 128, seed=23, q_scale=2.0, k_offset=3.0 if smooth else 0.0)
    _check_decode(q, k, v, 3, kv_lens=[1000, 517, 0], label="decode-pv%d" % pv, smooth=smooth, pv=pv)


def test_decode_fp4_d64():
    q, k, v = _rand_inputs(2, 4, 4, 1, 300, 64, seed=24)
    _check_decode(q, k, v, 7, label="decode-fp4-d64", pv=qfa.QFA_PV_FP4)


# ----------------------------------------------------------------------------- NVFP4 Q/K
def _nv_scales(q, k, scale):
    c2 = qfa.qfa_exp2_scale(scale)
    gq = qfa.nvfp4_tensor_scale(float((q.float() * c2).abs().max()))
    gk = qfa.nvfp4_tensor_scale(float(k.float().abs().max()))
    return c2, gq, gk


def _check_prefill_nv(q, k, v, causal, scale, smooth, rows, label):
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    say("prefill-nvfp4", label, "q", tuple(q.shape), "k", tuple(k.shape), "causal", causal, "smooth", smooth)
    c2, gq, gk = _nv_scales(q, k, scale)
    if smooth:  # the tensor scale of the smoothed K
        kb = bf16_bits(k)
        _, _, kbar_o = oracle.quantize_qk4(kb, smooth=True)
        ks = oracle.bf16_to_f64(kb) - np.repeat(oracle.bf16_to_f64(kbar_o), 128, axis=2)[:, :, :Skv]
        gk = qfa.nvfp4_tensor_scale(float(np.abs(ks).max()))
    q4, q4s, _ = qfa.quantize_nvfp4(q, gq, prescale=c2)
    k4, k4s, kbar = qfa.quantize_nvfp4(k, gk, smooth=smooth)
    v8, v8s = qfa.quantize_v8(v)
    O = torch.empty((B, Hq, Sq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    qfa.qfa_fwd_prefill_nvfp4(q4, q4s, k4, k4s, kbar, q if smooth else None, v8, v8s, B, Hq, Hkv, Sq, Skv, D,
                              causal, scale, gq, gk, O, lse)
    torch.cuda.synchronize()
    res = oracle.prefill_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, causal, scale, smooth=smooth,
                              nvfp4=(gq, gk))
    Og = to_np(O)[rows[:, 0], rows[:, 1], rows[:, 2]]
    lg = to_np(lse)[rows[:, 0], rows[:, 1], rows[:, 2]]
    compare_o(Og, res["O_q"], lg, res["lse_q"], label)
    ok = np.isfinite(res["lse_x"])
    if ok.any():
        ex = res["O_x"][ok]
        say("%s vs exact FP64: rel-L2 %.3e (reported only)" % (label, np.linalg.norm(Og[ok] - ex) / np.linalg.norm(ex)))


NV_CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, smooth, label
    (1, 4, 1, 333, 333, 128, True, False, "nv-causal-ragged-G4"),
    (2, 5, 1, 70, 700, 64, False, False, "nv-d64-G5"),
    (1, 4, 2, 300, 200, 128, True, False, "nv-sq>skv"),
    (1, 2, 1, 200, 600, 128, True, True, "nv-compensation"),
]


@pytest.mark.parametrize("case", NV_CASES, ids=[c[-1] for c in NV_CASES])
def test_prefill_nvfp4_small_all_rows(case):
    B, Hq, Hkv, Sq, Skv, D, causal, smooth, label = case
    q, k, v = _rand_inputs(B, Hq, Hkv, Sq, Skv, D, seed=zlib.crc32(label.encode()) % 1000,
                           k_offset=3.0 if smooth else 0.0, q_scale=2.0)
    _check_prefill_nv(q, k, v, causal, 1.0 / math.sqrt(D), smooth, _all_rows(B, Hq, Sq), label)


@pytest.mark.parametrize("fmt", ["blockp", "fp4", "nvfp4"])
@pytest.mark.parametrize("i", range(400, 416))
def test_prefill_formats_random_shapes(i, fmt):
    """The random-shape recipe in the contrast formats: block-scaled E4M3 P
    with the compensation as drawn; MXFP4 P/V and NVFP4 Q/K without it (where
    the compensated form of those two can move a P code across a rounding
    boundary on the last bit of the exponential, which an E2M1 step or the
    add-after-products order makes large enough to exceed a bar)."""
    B, Hq, Hkv, Sq, Skv, D, causal, smooth, fused, koff, qs = _random_prefill_case(i)
    if fmt != "blockp":
        smooth = False
    label = "%s-rand%d B%d H%d/%d S%d/%d D%d causal%d comp%d fused%d" % (fmt, i, B, Hq, Hkv, Sq, Skv, D, causal,
                                                                       smooth, fused)
    q, k, v = _rand_inputs(B, Hq, Hkv, Sq, Skv, D, seed=2000 + i, k_offset=koff, q_scale=qs)
    if fmt == "nvfp4":
        _check_prefill_nv(q, k, v, causal, 1.0 / math.sqrt(D), smooth, _all_rows(B, Hq, Sq), label)
    else:
        pv = qfa.QFA_PV_FP8_BLOCKP if fmt == "blockp" else qfa.QFA_PV_FP4
        _check_prefill(q, k, v, causal, 1.0 / math.sqrt(D), smooth, _all_rows(B, Hq, Sq), label, fused=fused, pv=pv)


def test_decode_nvfp4_varlen():
    B, Hq, Hkv, Smax, D = 3, 8, 2, 1000, 128
    q, k, v = _rand_inputs(B, Hq, Hkv, 1, Smax, D, seed=25, q_scale=2.0)
    kv_lens = [1000, 517, 0]
    scale = 1.0 / math.sqrt(D)
    c2, gq, gk = _nv_scales(q, k, scale)
    say("decode-nvfp4 varlen", tuple(k.shape), kv_lens)
    q4, q4s, _ = qfa.quantize_nvfp4(q, gq, prescale=c2)
    k4 = torch.zeros((B, Hkv, Smax, D // 2), dtype=torch.uint8, device="cuda")
    k4s = torch.zeros((B, Hkv, Smax, D // 16), dtype=torch.uint8, device="cuda")
    v8 = torch.zeros((B, Hkv, (Smax + 31) // 32, D, 32), dtype=torch.uint8, device="cuda")
    v8s = torch.zeros((B, Hkv, (Smax + 31) // 32, D), dtype=torch.uint8, device="cuda")
    for b, L in enumerate(kv_lens):   # each sequence's own tokens, as the cache writer stores them
        if L:
            kc, ksc, _ = qfa.quantize_nvfp4(k[b:b + 1, :, :L].contiguous(), gk)
            vc, vsc = qfa.quantize_v8(v[b:b + 1, :, :L].contiguous())
            k4[b:b + 1, :, :L], k4s[b:b + 1, :, :L] = kc, ksc
            v8[b:b + 1, :, :vc.shape[2]], v8s[b:b + 1, :, :vsc.shape[2]] = vc, vsc
    lens = torch.tensor(kv_lens, dtype=torch.int32, device="cuda")
    splits = 3
    wsb = qfa.qfa_decode_workspace_bytes(B, Hq, D, splits)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    O = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    used = qfa.qfa_fwd_decode_nvfp4(q4, q4s, k4, k4s, None, None, v8, v8s, B, Hq, Hkv, Smax, lens, D, scale, gq, gk,
                                    splits, ws, wsb, O, lse)
    torch.cuda.synchronize()
    assert used == splits
    rows = np.array([(b, h, 0) for b in range(B) for h in range(Hq)], dtype=np.int64)
    res = oracle.decode_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, scale, used, kv_lens=kv_lens,
                             nvfp4=(gq, gk))
    compare_o(to_np(O)[rows[:, 0], rows[:, 1]], res["O_q"], to_np(lse)[rows[:, 0], rows[:, 1]], res["lse_q"],
              "decode-nvfp4")


# ----------------------------------------------------------------------------- contrast formats at full size
@pytest.mark.parametrize("pv", [qfa.QFA_PV_FP8_BLOCKP, qfa.QFA_PV_FP4], ids=["blockp", "fp4"])
def test_prefill_formats_llama16k_sampled(pv):
    """The P/V contrast formats at the benchmarked size and launch (Q quantised in the kernel)."""
    w = WORKLOADS["llama16k"]
    inp = make_inputs(w, seed=0)
    rows = sample_rows(1, w.Hq, w.S_q, 96, seed=3, must=(0, 127, 128, 4095))
    _check_prefill(inp["q"], inp["k"], inp["v"], w.causal, w.scale, w.smooth, rows, "llama16k-pv%d" % pv,
                   fused=True, pv=pv)


def test_prefill_nvfp4_llama16k_sampled():
    w = WORKLOADS["llama16k"]
    inp = make_inputs(w, seed=0)
    rows = sample_rows(1, w.Hq, w.S_q, 96, seed=4, must=(0, 127, 128, 4095))
    _check_prefill_nv(inp["q"], inp["k"], inp["v"], w.causal, w.scale, w.smooth, rows, "llama16k-nvfp4")


@pytest.mark.parametrize("pv", [qfa.QFA_PV_FP8_BLOCKP, qfa.QFA_PV_FP4], ids=["blockp", "fp4"])
def test_decode_formats_workload_sampled(pv):
    """The P/V contrast formats on the B64 x 32768 decode workload, 16 splits."""
    w = WORKLOADS["decode"]
    inp = make_inputs(w, seed=0)
    used = _check_decode(inp["q"], inp["k"], inp["v"], w.num_splits, label="decode-B64-pv%d" % pv, seqs=[0, 42],
                         pv=pv)
    assert used == 16
