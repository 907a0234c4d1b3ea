"""KV-cache writer (qfa_kv_append) on the GPU.

Appending in chunks must leave exactly the bytes the quantisers write for the
whole sequence at once (quantise on write: hnwysp.cn MXAttention/MXFP4 notes,
sections 3.4 and 5.4): K codes and scales, K-bar with smoothing, V codes and
scales, including the V block and the K-bar tile an append starts inside.
Sequences of one batch have different lengths (kv_lens).  Decode on the
appended cache equals decode on the one-shot cache, and one sequence is also
checked against the oracle's quantisers.
"""
import math

import numpy as np
import pytest
import torch

import bit_quantized_attention_qk4pv8_amd as qfa
import oracle
from bit_quantized_attention_qk4pv8_amd.workloads import bf16_bits
from gpu_util import say, to_np

pytestmark = pytest.mark.gpu


def _data(B, Hkv, S, D, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    k = torch.randn((B, Hkv, S, D), generator=g, device="cuda")
    k += torch.randn((B, Hkv, 1, D), generator=g, device="cuda") * 3.0   # channel offsets: K-bar matters
    v = torch.randn((B, Hkv, S, D), generator=g, device="cuda")
    v[:, :, 7, :] *= 50.0                                                 # an outlier token inside a V block
    return k.to(torch.bfloat16), v.to(torch.bfloat16)


def _sl(c, b):
    return {k: (v[b:b + 1] if isinstance(v, torch.Tensor) else v) for k, v in c.items()}


def _check_against_one_shot(c, k, v, lens, smooth, label):
    for b, L in enumerate(lens):
        if L == 0:
            continue
        k4, k4s, kb = qfa.quantize_qk4(k[b:b + 1, :, :L].contiguous(), smooth=smooth)
        v8, v8s = qfa.quantize_v8(v[b:b + 1, :, :L].contiguous())
        nvb, nt = (L + 31) // 32, (L + 127) // 128
        assert torch.equal(c["k4"][b:b + 1, :, :L], k4), (label, b, "K codes")
        assert torch.equal(c["k4s"][b:b + 1, :, :L], k4s), (label, b, "K scales")
        assert torch.equal(c["v8"][b:b + 1, :, :nvb], v8), (label, b, "V codes")
        assert torch.equal(c["v8s"][b:b + 1, :, :nvb], v8s), (label, b, "V scales")
        if smooth:
            assert torch.equal(c["kbar"][b:b + 1, :, :nt], kb), (label, b, "K-bar")


@pytest.mark.parametrize("D,smooth", [(128, True), (128, False), (64, True)])
def test_append_in_chunks_equals_one_shot(D, smooth):
    B, Hkv, S = 3, 2, 1200
    k, v = _data(B, Hkv, S, D, seed=D + smooth)
    c = qfa.kv_cache(B, Hkv, S, D, smooth=smooth)
    lens = [0, 5, 200]
    for b, L0 in enumerate(lens):          # different starting lengths, one sequence at a time
        if L0:
            qfa.kv_append(_sl(c, b), k[b:b + 1, :, :L0].contiguous(), v[b:b + 1, :, :L0].contiguous())
    torch.cuda.synchronize()
    _check_against_one_shot(c, k, v, lens, smooth, "start")
    for n in (1, 31, 33, 128, 1, 97, 250, 3):   # chunks that start and end inside V blocks and K-bar tiles
        say("kv_append D", D, "smooth", smooth, "lens", lens, "n", n)
        kl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        kn = torch.stack([k[b, :, lens[b]:lens[b] + n] for b in range(B)]).contiguous()
        vn = torch.stack([v[b, :, lens[b]:lens[b] + n] for b in range(B)]).contiguous()
        qfa.kv_append(c, kn, vn, kv_lens=kl)
        torch.cuda.synchronize()
        lens = [L + n for L in lens]
        _check_against_one_shot(c, k, v, lens, smooth, "after +%d" % n)


def test_append_matches_oracle_and_feeds_decode():
    B, Hkv, Hq, S, D = 2, 2, 8, 700, 128
    k, v = _data(B, Hkv, S, D, seed=3)
    c = qfa.kv_cache(B, Hkv, S, D, smooth=True)
    lens = [0, 0]
    for n in (100, 1, 130, 64, 2):
        kl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        kn = torch.stack([k[b, :, lens[b]:lens[b] + n] for b in range(B)]).contiguous()
        vn = torch.stack([v[b, :, lens[b]:lens[b] + n] for b in range(B)]).contiguous()
        qfa.kv_append(c, kn, vn, kv_lens=kl)
        lens = [L + n for L in lens]
    torch.cuda.synchronize()
    L = lens[0]
    # the oracle's quantisers on the whole of sequence 1
    oc, os_, ok = oracle.quantize_qk4(bf16_bits(k[1:2, :, :L]), smooth=True)
    vc, vs = oracle.quantize_v8(bf16_bits(v[1:2, :, :L]))
    nvb, nt = (L + 31) // 32, (L + 127) // 128
    assert np.array_equal(to_np(c["k4"][1:2, :, :L]), oc)
    assert np.array_equal(to_np(c["k4s"][1:2, :, :L]), os_)
    assert np.array_equal(to_np(c["kbar"][1:2, :, :nt].view(torch.int16)).view(np.uint16), ok)
    assert np.array_equal(to_np(c["v8"][1:2, :, :nvb]), vc)
    assert np.array_equal(to_np(c["v8s"][1:2, :, :nvb]), vs)
    # decode on the appended cache == decode on a cache quantised in one pass
    g = torch.Generator(device="cuda").manual_seed(9)
    q = torch.randn((B, Hq, 1, D), generator=g, device="cuda").to(torch.bfloat16)
    kl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    O1, l1, _ = qfa.fwd_decode(None, None, c["k4"], c["k4s"], c["v8"], c["v8s"], S, 1 / math.sqrt(D), num_splits=3,
                               kv_lens=kl, kbar=c["kbar"], q_bf16=q)
    k4, k4s, kb = qfa.quantize_qk4(k[:, :, :L].contiguous(), smooth=True)
    v8, v8s = qfa.quantize_v8(v[:, :, :L].contiguous())
    O2, l2, _ = qfa.fwd_decode(None, None, k4, k4s, v8, v8s, L, 1 / math.sqrt(D), num_splits=3, kbar=kb, q_bf16=q)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(l1, l2)


def test_append_order_sensitive_kbar_matches_oracle():
    """Appends in chunks that split a K-bar tile whose channel sums binary64
    does not add exactly (values 2^60 apart): after every append the cache's
    K-bar must still be the oracle's token-order sum over the tile's present
    rows, and the K codes must match the oracle's quantiser bit for bit."""
    B, Hkv, S, D = 1, 2, 300, 128
    k, v = _data(B, Hkv, S, D, seed=21)
    kf = k.float()
    kf[0, 0, :, 0] = 1.0
    kf[0, 0, 3, 0], kf[0, 0, 90, 0] = 2.0 ** 60, -(2.0 ** 60)     # tile 0: the sum restarts at token 90
    kf[0, 1, 140, 5], kf[0, 1, 200, 5] = -(2.0 ** 70), 2.0 ** 70  # tile 1, the other KV head
    k = kf.to(torch.bfloat16)
    c = qfa.kv_cache(B, Hkv, S, D, smooth=True)
    L = 0
    for n in (60, 45, 60, 1, 100, 34):
        say("kv_append order-sensitive K-bar, at", L, "n", n)
        kl = torch.tensor([L], dtype=torch.int32, device="cuda")
        qfa.kv_append(c, k[:, :, L:L + n].contiguous(), v[:, :, L:L + n].contiguous(), kv_lens=kl)
        torch.cuda.synchronize()
        L += n
        oc, os_, ok = oracle.quantize_qk4(bf16_bits(k[:, :, :L]), smooth=True)
        nt = (L + 127) // 128
        assert np.array_equal(to_np(c["kbar"][:, :, :nt].view(torch.int16)).view(np.uint16), ok), ("K-bar", L)
        assert np.array_equal(to_np(c["k4"][:, :, :L]), oc), ("K codes", L)
        assert np.array_equal(to_np(c["k4s"][:, :, :L]), os_), ("K scales", L)


def _check_formats_one_shot(c, k, v, lens, smooth, pv, g, label):
    for b, L in enumerate(lens):
        if L == 0:
            continue
        ks = k[b:b + 1, :, :L].contiguous()
        if g > 0:
            k4, k4s, kb = qfa.quantize_nvfp4(ks, g, smooth=smooth)
        else:
            k4, k4s, kb = qfa.quantize_qk4(ks, smooth=smooth)
        vs = v[b:b + 1, :, :L].contiguous()
        v8, v8s = qfa.quantize_v4(vs) if pv == qfa.QFA_PV_FP4 else qfa.quantize_v8(vs)
        nvb, nt = (L + 31) // 32, (L + 127) // 128
        assert torch.equal(c["k4"][b:b + 1, :, :L], k4), (label, b, "K codes")
        assert torch.equal(c["k4s"][b:b + 1, :, :L], k4s), (label, b, "K scales")
        assert torch.equal(c["v8"][b:b + 1, :, :nvb], v8), (label, b, "V codes")
        assert torch.equal(c["v8s"][b:b + 1, :, :nvb], v8s), (label, b, "V scales")
        if smooth:
            assert torch.equal(c["kbar"][b:b + 1, :, :nt], kb), (label, b, "K-bar")


@pytest.mark.parametrize("pv,nv,smooth", [(qfa.QFA_PV_FP4, False, True), (qfa.QFA_PV_FP4, False, False),
                                          (qfa.QFA_PV_FP8, True, True), (qfa.QFA_PV_FP8, True, False)],
                         ids=["v4-smooth", "v4", "nvfp4k-smooth", "nvfp4k"])
def test_append_formats_in_chunks_equals_one_shot(pv, nv, smooth):
    """The cache writer for the contrast formats (MXFP4 V, NVFP4 K): chunked
    appends leave the bytes of the one-shot quantisers of that format, and the
    format's decode reads the appended cache (checked against the oracle
    without smoothing)."""
    B, Hkv, S, D = 3, 2, 700, 128
    k, v = _data(B, Hkv, S, D, seed=11 + pv + 2 * nv + 4 * smooth)
    g = qfa.nvfp4_tensor_scale(float(k.float().abs().max())) if nv else 0.0
    c = qfa.kv_cache(B, Hkv, S, D, smooth=smooth, pv_format=pv, k_tensor_scale=g)
    lens = [0, 5, 200]
    for b, L0 in enumerate(lens):
        if L0:
            qfa.kv_append(_sl(c, b), k[b:b + 1, :, :L0].contiguous(), v[b:b + 1, :, :L0].contiguous())
    for n in (1, 31, 33, 130, 97):
        say("kv_append formats pv", pv, "nvfp4 K", nv, "smooth", smooth, "lens", lens, "n", n)
        kl = torch.tensor(lens, dtype=torch.int32, device="cuda")
        kn = torch.stack([k[b, :, lens[b]:lens[b] + n] for b in range(B)]).contiguous()
        vn = torch.stack([v[b, :, lens[b]:lens[b] + n] for b in range(B)]).contiguous()
        qfa.kv_append(c, kn, vn, kv_lens=kl)
        torch.cuda.synchronize()
        lens = [L + n for L in lens]
        _check_formats_one_shot(c, k, v, lens, smooth, pv, g, "after +%d" % n)
    Hq = 8
    q = torch.randn((B, Hq, 1, D), device="cuda").to(torch.bfloat16)
    kl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    scale = 1 / math.sqrt(D)
    say("decode on the appended cache, lens", lens)
    if nv:
        c2 = qfa.qfa_exp2_scale(scale)
        gq = qfa.nvfp4_tensor_scale(float((q.float() * c2).abs().max()))
        q4, q4s, _ = qfa.quantize_nvfp4(q, gq, prescale=c2)
        wsb = qfa.qfa_decode_workspace_bytes(B, Hq, D, 3)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        O = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        qfa.qfa_fwd_decode_nvfp4(q4, q4s, c["k4"], c["k4s"], c["kbar"], q if smooth else None, c["v8"], c["v8s"],
                                 B, Hq, Hkv, S, kl, D, scale, gq, g, 3, ws, wsb, O, lse)
    else:
        O, lse, _ = qfa.fwd_decode(None, None, c["k4"], c["k4s"], c["v8"], c["v8s"], S, scale, num_splits=3,
                                   kv_lens=kl, kbar=c["kbar"], q_bf16=q, pv_format=pv)
    torch.cuda.synchronize()
    assert torch.isfinite(O).all()
    if not smooth:
        rows = np.array([(b, h, 0) for b in range(B) for h in range(Hq)], dtype=np.int64)
        full_k = torch.zeros((B, Hkv, S, D), dtype=torch.bfloat16, device="cuda")
        full_v = torch.zeros_like(full_k)
        for b, L in enumerate(lens):
            full_k[b, :, :L], full_v[b, :, :L] = k[b, :, :L], v[b, :, :L]
        res = oracle.decode_rows(bf16_bits(q), bf16_bits(full_k), bf16_bits(full_v), rows, scale, 3, kv_lens=lens,
                                 pv=oracle.PV_FP4 if pv == qfa.QFA_PV_FP4 else oracle.PV_FP8,
                                 nvfp4=(gq, g) if nv else None, exact=False)
        Og = to_np(O)[rows[:, 0], rows[:, 1]]
        assert np.abs(Og - res["O_q"]).max() < 3e-3
