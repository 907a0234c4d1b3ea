"""The C-ABI library: exports and host-side validation (no GPU needed).

Only calls that return before any HIP call are made here: version, status
strings, workspace sizing, the split heuristic, and argument validation that
rejects the call on the host.
"""
import ctypes
import json
import math
import os
import re

import pytest

import bit_quantized_attention_qk4pv8_amd as qfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qfa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qfa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_python_exports():
    assert declared_functions() == sorted(qfa.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = qfa.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_version_and_status_strings():
    assert qfa.qfa_version() == 10000
    assert qfa.status_string(0) == "QFA_OK"
    assert qfa.status_string(2) == "QFA_ERR_UNSUPPORTED"
    assert qfa.status_string(3) == "QFA_ERR_WORKSPACE"
    assert qfa.status_string(99) == "QFA_ERR_UNKNOWN"


def test_workspace_bytes_and_default_splits():
    # O partials (B*Hq*splits*D floats) and LSE partials, each padded to 256 bytes
    assert qfa.qfa_decode_workspace_bytes(64, 32, 128, 16) == 64 * 32 * 16 * 128 * 4 + 64 * 32 * 16 * 4
    assert qfa.qfa_decode_workspace_bytes(1, 1, 64, 1) == 256 + 256
    assert qfa.qfa_decode_workspace_bytes(0, 32, 128, 16) == 0
    assert qfa.qfa_decode_default_splits(64, 8, 32768) == 4        # 512 units -> 2048 target
    assert qfa.qfa_decode_default_splits(1, 8, 32768) == 256       # capped
    assert qfa.qfa_decode_default_splits(1, 1, 300) == 3           # never more splits than tiles
    assert qfa.qfa_decode_default_splits(1, 1, 0) == 1


def test_exp2_scale_is_the_binary32_product():
    import numpy as np
    for sc in (0.125, 1 / math.sqrt(128), 1 / math.sqrt(64), 1.0, 3e-3, 7.5):
        want = np.float32(sc) * np.float32(math.log2(math.e))   # both operands and the product in binary32
        assert np.float32(qfa.qfa_exp2_scale(sc)) == want


def _call_raw(fn, *args):
    return getattr(qfa.lib(), fn)(*args)


def test_validation_rejects_before_launch():
    P = ctypes.c_void_p
    fake = P(4096)          # 16-byte aligned, never dereferenced: validation fails first
    odd = P(4097)
    # block size and head dimension
    assert _call_raw("qfa_quantize_qk4", fake, 1, 1, 1, 64, 16, 0, 1.0, fake, fake, None, None) == qfa.QFA_ERR_UNSUPPORTED
    assert _call_raw("qfa_quantize_qk4", fake, 1, 1, 1, 48, 32, 0, 1.0, fake, fake, None, None) == qfa.QFA_ERR_UNSUPPORTED
    # kbar must be given iff smooth
    assert _call_raw("qfa_quantize_qk4", fake, 1, 1, 1, 64, 32, 1, 1.0, fake, fake, None, None) == qfa.QFA_ERR_INVALID_ARG
    assert _call_raw("qfa_quantize_qk4", fake, 1, 1, 1, 64, 32, 0, 1.0, fake, fake, fake, None) == qfa.QFA_ERR_INVALID_ARG
    # the Q prescale must be a finite positive number
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert _call_raw("qfa_quantize_qk4", fake, 1, 1, 1, 64, 32, 0, bad, fake, fake, None, None) == \
            qfa.QFA_ERR_INVALID_ARG
    # misaligned input
    assert _call_raw("qfa_quantize_v8", odd, 1, 1, 1, 64, 32, fake, fake, None) == qfa.QFA_ERR_INVALID_ARG
    # empty problem: nothing to do
    assert _call_raw("qfa_quantize_v8", None, 0, 1, 1, 64, 32, None, None, None) == qfa.QFA_OK
    F = ctypes.c_float
    pre = lambda Hq, Hkv, D, bs, kbar, qbf, O, scale=0.125: _call_raw(
        "qfa_fwd_prefill", fake, fake, fake, fake, kbar, qbf, fake, fake, 1, Hq, Hkv, 8, 8, D, 1, F(scale), bs, O,
        None, None)
    assert pre(4, 3, 128, 32, None, None, fake) == qfa.QFA_ERR_INVALID_ARG   # Hq % Hkv
    assert pre(4, 2, 96, 32, None, None, fake) == qfa.QFA_ERR_UNSUPPORTED    # D
    assert pre(4, 2, 128, 64, None, None, fake) == qfa.QFA_ERR_UNSUPPORTED   # block size
    assert pre(4, 2, 128, 32, fake, None, fake) == qfa.QFA_ERR_INVALID_ARG   # kbar without q_bf16
    assert pre(4, 2, 128, 32, None, None, None) == qfa.QFA_ERR_INVALID_ARG   # no output
    assert pre(4, 2, 128, 32, None, None, fake, scale=0.0) == qfa.QFA_ERR_INVALID_ARG
    # Q quantised in the kernel: q4 and q4s both NULL, and q_bf16 (aligned) required
    preq = lambda q4, q4s, qbf, kbar=None: _call_raw(
        "qfa_fwd_prefill", q4, q4s, fake, fake, kbar, qbf, fake, fake, 1, 4, 2, 8, 8, 128, 1, F(0.125), 32, fake,
        None, None)
    assert preq(None, fake, fake) == qfa.QFA_ERR_INVALID_ARG      # q4 NULL but q4s given
    assert preq(fake, None, fake) == qfa.QFA_ERR_INVALID_ARG      # q4s missing
    assert preq(None, None, None) == qfa.QFA_ERR_INVALID_ARG      # no Q at all
    assert preq(None, None, odd) == qfa.QFA_ERR_INVALID_ARG       # misaligned bf16 Q
    assert preq(odd, fake, None) == qfa.QFA_ERR_INVALID_ARG       # misaligned codes
    nsq = ctypes.c_int(1)
    assert _call_raw("qfa_fwd_decode", None, None, fake, fake, None, None, fake, fake, 2, 8, 2, 1024, None, 128,
                     F(0.1), 32, ctypes.byref(nsq), fake, ctypes.c_size_t(1 << 20), fake, None, None) == \
        qfa.QFA_ERR_INVALID_ARG                                   # decode: no Q at all
    # decode: workspace too small is reported before launch
    ns = ctypes.c_int(4)
    st = _call_raw("qfa_fwd_decode", fake, fake, fake, fake, None, None, fake, fake, 2, 8, 2, 1024, None, 128,
                   F(0.1), 32, ctypes.byref(ns), fake, ctypes.c_size_t(16), fake, None, None)
    assert st == qfa.QFA_ERR_WORKSPACE
    st = _call_raw("qfa_fwd_decode", fake, fake, fake, fake, None, None, fake, fake, 2, 8, 2, 1024, None, 128,
                   F(0.1), 32, None, fake, ctypes.c_size_t(1 << 30), fake, None, None)
    assert st == qfa.QFA_ERR_INVALID_ARG


def test_pv_format_validation():
    """The _ex entry points take the P/V format: an unknown one is an invalid
    argument (checked before anything else is read); every other check is the
    plain entry point's."""
    P = ctypes.c_void_p
    F = ctypes.c_float
    fake = P(4096)
    pre = lambda fmt, Hkv=2: _call_raw(
        "qfa_fwd_prefill_ex", fake, fake, fake, fake, None, None, fake, fake, 1, 4, Hkv, 8, 8, 128, 1, F(0.125), 32,
        fmt, fake, None, None)
    for bad in (-1, 3, 99):
        assert pre(bad) == qfa.QFA_ERR_INVALID_ARG
    assert pre(qfa.QFA_PV_FP8, Hkv=3) == qfa.QFA_ERR_INVALID_ARG       # Hq % Hkv, as for the plain call
    assert pre(qfa.QFA_PV_FP8_BLOCKP, Hkv=3) == qfa.QFA_ERR_INVALID_ARG
    ns = ctypes.c_int(4)
    dec = lambda fmt, ws=16: _call_raw(
        "qfa_fwd_decode_ex", fake, fake, fake, fake, None, None, fake, fake, 2, 8, 2, 1024, None, 128, F(0.1), 32,
        fmt, ctypes.byref(ns), fake, ctypes.c_size_t(ws), fake, None, None)
    assert dec(5) == qfa.QFA_ERR_INVALID_ARG
    assert dec(qfa.QFA_PV_FP8_BLOCKP) == qfa.QFA_ERR_WORKSPACE          # workspace too small, as before
    assert dec(qfa.QFA_PV_FP4) == qfa.QFA_ERR_WORKSPACE
    # the MXFP4 V quantiser validates like the E4M3 one
    assert _call_raw("qfa_quantize_v4", fake, 1, 1, 1, 64, 16, fake, fake, None) == qfa.QFA_ERR_UNSUPPORTED
    assert _call_raw("qfa_quantize_v4", P(4097), 1, 1, 1, 64, 32, fake, fake, None) == qfa.QFA_ERR_INVALID_ARG
    assert _call_raw("qfa_quantize_v4", None, 0, 1, 1, 64, 32, None, None, None) == qfa.QFA_OK
    # the plain entry points are the method's format
    assert _call_raw("qfa_fwd_prefill", fake, fake, fake, fake, None, None, fake, fake, 1, 4, 3, 8, 8, 128, 1,
                     F(0.125), 32, fake, None, None) == qfa.QFA_ERR_INVALID_ARG


def test_nvfp4_validation_and_tensor_scale():
    P = ctypes.c_void_p
    F = ctypes.c_float
    fake = P(4096)
    q = lambda bs=16, g=1.0, smooth=0, kbar=None: _call_raw(
        "qfa_quantize_nvfp4", fake, 1, 1, 1, 64, bs, smooth, F(1.0), F(g), fake, fake, kbar, None)
    assert q(bs=32) == qfa.QFA_ERR_UNSUPPORTED
    for bad in (0.0, -2.0, 3.0, 0.75, float("inf"), float("nan")):
        assert q(g=bad) == qfa.QFA_ERR_INVALID_ARG                    # the tensor scale is a power of two
    assert q(smooth=1) == qfa.QFA_ERR_INVALID_ARG                       # smoothing needs kbar
    assert _call_raw("qfa_quantize_nvfp4", None, 0, 1, 1, 64, 16, 0, F(1.0), F(0.5), None, None, None,
                     None) == qfa.QFA_OK
    pre = lambda q4, q4s, gq=1.0: _call_raw(
        "qfa_fwd_prefill_nvfp4", q4, q4s, fake, fake, None, fake, fake, fake, 1, 4, 2, 8, 8, 128, 1, F(0.125),
        F(gq), F(1.0), fake, None, None)
    assert pre(None, None) == qfa.QFA_ERR_INVALID_ARG                   # NVFP4 Q comes quantised
    assert pre(fake, fake, gq=3.0) == qfa.QFA_ERR_INVALID_ARG
    ns = ctypes.c_int(4)
    assert _call_raw("qfa_fwd_decode_nvfp4", fake, fake, fake, fake, None, None, fake, fake, 2, 8, 2, 1024, None,
                     128, F(0.1), F(1.0), F(0.25), ctypes.byref(ns), fake, ctypes.c_size_t(16), fake, None,
                     None) == qfa.QFA_ERR_WORKSPACE
    # the host helper picks the smallest power of two g with amax / (6 g) <= 448
    assert qfa.nvfp4_tensor_scale(6 * 448.0) == 1.0
    assert qfa.nvfp4_tensor_scale(6 * 448.0 * 1.0001) == 2.0
    assert qfa.nvfp4_tensor_scale(0.0) == 1.0
    for amax in (1e-3, 0.37, 5.0, 1234.5, 1e6):
        g = qfa.nvfp4_tensor_scale(amax)
        assert amax / (6 * g) <= 448.0 < amax / (6 * g / 2)


def test_kv_append_validation():
    P = ctypes.c_void_p
    fake, odd = P(4096), P(4097)
    app = lambda D=128, bs=32, n=4, kbar=None, ktail=None, knew=fake, vtail=fake: _call_raw(
        "qfa_kv_append", knew, fake, 2, 2, n, D, 1024, bs, None, fake, fake, kbar, fake, fake, ktail, vtail, None)
    assert app(bs=16) == qfa.QFA_ERR_UNSUPPORTED
    assert app(D=48) == qfa.QFA_ERR_UNSUPPORTED
    assert app(n=-1) == qfa.QFA_ERR_INVALID_ARG
    assert app(kbar=fake) == qfa.QFA_ERR_INVALID_ARG          # smoothing needs the K tail
    assert app(ktail=fake) == qfa.QFA_ERR_INVALID_ARG         # and the K tail needs smoothing
    assert app(knew=odd) == qfa.QFA_ERR_INVALID_ARG           # misaligned input
    assert app(vtail=None) == qfa.QFA_ERR_INVALID_ARG         # the V tail is always needed
    assert app(n=0, knew=None) == qfa.QFA_OK                  # nothing to append
    F = ctypes.c_float
    appx = lambda fmt=0, g=0.0: _call_raw(
        "qfa_kv_append_ex", fake, fake, 2, 2, 4, 128, 1024, 32, None, fake, fake, None, fake, fake, None, fake, fmt,
        F(g), None)
    assert appx(fmt=7) == qfa.QFA_ERR_INVALID_ARG             # unknown V format
    assert appx(g=3.0) == qfa.QFA_ERR_INVALID_ARG             # the NVFP4 tensor scale is a power of two
    assert appx(g=-1.0) == qfa.QFA_ERR_INVALID_ARG


def test_kv_cache_byte_formula_matches_printed_example():
    """Byte accounting used for the decode roofline reproduces the KV-cache
    formula example printed in the MXFP4 notes (section 1.1)."""
    from bit_quantized_attention_qk4pv8_amd.roofline import kv_cache_bytes, decode_algorithmic_bytes
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "kv_cache_bytes.json")))
    per_tok_layer = kv_cache_bytes(layers=1, kv_heads=g["kv_heads"], head_dim=g["head_dim"], seq_len=1,
                                   bytes_per_element=g["bytes_per_element"], batch=1)
    assert per_tok_layer == g["bytes_per_token_per_layer"]
    assert kv_cache_bytes(g["layers"], g["kv_heads"], g["head_dim"], 1, g["bytes_per_element"], 1) == \
        g["bytes_per_token_all_layers"]
    assert kv_cache_bytes(g["layers"], g["kv_heads"], g["head_dim"], g["seq_len"], g["bytes_per_element"],
                          g["batch"]) == g["total_bytes_128k"]
    # QK4 / V8 with E8M0 scales: 64 + 4 + 128 + 4 = 200 bytes per token per kv head at D = 128
    assert decode_algorithmic_bytes(B=1, Hq=1, Hkv=1, L=1, D=128, include_q_o=False) == 200
    assert decode_algorithmic_bytes(B=64, Hq=32, Hkv=8, L=32768, D=128) == 3357016064


def test_probe_library_loads_and_exports_its_symbols():
    """The test-only HIP library of GPU-side pins (tests/hip) is built and
    resolves every symbol; it is separate from libqfa."""
    import sys
    sys.path.insert(0, os.path.join(ROOT, "tests", "hip"))
    import build_probe
    L = build_probe.load()
    for name in build_probe.SYMBOLS:
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value, name
    assert not any(hasattr(qfa.lib(), name) for name in build_probe.SYMBOLS)
