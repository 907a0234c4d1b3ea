"""CPU oracle for the QK4PV8 attention forward pass -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never loads it and shares no code with it.
The arithmetic lives in ``qfa_oracle.c`` (plain C, binary64); this module only
marshals numpy arrays through ctypes and groups query rows by (batch, kv head).

Sources, by page title and section:
  * "MpFA: Hardware-Efficient Train-Free QK4V8 FlashAttention Kernels on
    Blackwell GPUs", abstract -- the method (QK 4-bit, PV 8-bit, online P
    quantisation, rank-one smoothing compensation, prefill/decode partitioning).
  * "FlashAttention压到4位" tutorial, sections "注意力慢在哪儿" (online softmax,
    LSE) and "FP4 只有约 15 个可表示的数" (E2M1 values, MXFP4 block of 32 with
    an E8M0 scale), "Direct-P" (denominator from the rounded codes).
  * hnwysp.cn MXAttention/MXFP4 notes, sections 2.3 and 5.2 (block quantiser).

Parity status of each function is recorded in the repository's design notes;
the method-accuracy numbers (error of the quantised result against exact
attention) are "parity unpinned": the pages print no operator-level figure.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qfa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

TILE = 128
BLOCK = 32

# How P is quantised (tile_p in qfa_oracle.c)
P_EXACT, P_E4M3, P_E4M3_BLOCK, P_E2M1_BLOCK = 0, 1, 2, 3
# P/V formats of the whole path: the method (QK4PV8, one P scale per row), FP8 P
# with one E8M0 scale per (row, 32 keys), and MXFP4 P and V ("QK4PV4").
PV_FP8, PV_FP8_BLOCKP, PV_FP4 = 0, 1, 2
_P_MODE_OF_PV = {PV_FP8: P_E4M3, PV_FP8_BLOCKP: P_E4M3_BLOCK, PV_FP4: P_E2M1_BLOCK}


# -ffp-contract=off: every operation rounds as written (no fused multiply-add
# contraction), so the binary32 and binary64 steps are the ones stated in
# qfa_oracle.c.  x86-64-v3 (AVX2, FMA) runs on any current x86 server host.
CFLAGS = ["-std=gnu11", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]


def build(force: bool = False, out: Optional[str] = None, march: Optional[str] = None) -> str:
    """Compile the oracle with gcc (plain C11, OpenMP).  out/march build a
    separate copy (e.g. -march=native for timing on the host that runs it)."""
    target = out or _LIB
    if force or out or not os.path.exists(target) or os.path.getmtime(target) < os.path.getmtime(_SRC):
        tmp = target + ".tmp%d" % os.getpid()
        flags = [f if not (march and f.startswith("-march=")) else "-march=" + march for f in CFLAGS]
        cmd = ["gcc"] + flags + [_SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, target)
    return target


_active = None  # path of a separately built copy in use (use_library), else the in-tree build


def use_library(path: str) -> None:
    """Load the oracle from another build of the same source (e.g. one built
    with -march=native on the host that times it) from here on."""
    global _lib, _active
    _active = path
    _lib = None


def lib():
    global _lib
    if _lib is None:
        if _active is None:
            build()
        L = ctypes.CDLL(_active or _LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        F = ctypes.c_float
        D = ctypes.c_double
        L.orc_e2m1_value.restype = D
        L.orc_e2m1_value.argtypes = [I]
        L.orc_e2m1_encode.restype = I
        L.orc_e2m1_encode.argtypes = [D]
        L.orc_e4m3_value.restype = D
        L.orc_e4m3_value.argtypes = [I]
        L.orc_e4m3_encode.restype = I
        L.orc_e4m3_encode.argtypes = [D]
        L.orc_e8m0_value.restype = D
        L.orc_e8m0_value.argtypes = [I]
        L.orc_mx_exponent.restype = I
        L.orc_mx_exponent.argtypes = [D, I]
        L.orc_bf16_value.restype = D
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_from_double.restype = ctypes.c_uint16
        L.orc_bf16_from_double.argtypes = [D]
        L.orc_quantize_qk4.restype = None
        L.orc_quantize_qk4.argtypes = [P, I64, I64, I64, I64, I, F, P, P, P]
        L.orc_quantize_v8.restype = None
        L.orc_quantize_v8.argtypes = [P, I64, I64, I64, I64, P, P]
        L.orc_dequant_qk4.restype = None
        L.orc_dequant_qk4.argtypes = [P, P, I64, I64, P]
        L.orc_dequant_v8.restype = None
        L.orc_dequant_v8.argtypes = [P, P, I64, I64, P]
        L.orc_quantize_nvfp4.restype = None
        L.orc_quantize_nvfp4.argtypes = [P, I64, I64, I64, I64, I, F, F, P, P, P]
        L.orc_dequant_nvfp4.restype = None
        L.orc_dequant_nvfp4.argtypes = [P, P, I64, I64, D, P]
        L.orc_quantize_v4.restype = None
        L.orc_quantize_v4.argtypes = [P, I64, I64, I64, I64, P, P]
        L.orc_dequant_v4.restype = None
        L.orc_dequant_v4.argtypes = [P, P, I64, I64, P]
        L.orc_attn_exact_rows.restype = None
        L.orc_attn_exact_rows.argtypes = [P, P, I64, P, P, I64, I64, I64, I, D, P, P]
        L.orc_attn_quant_rows.restype = None
        L.orc_attn_quant_rows.argtypes = [P, P, P, I64, P, P, P, I64, I64, I64, I, F, I64, I, I, P, P]
        for nm in ("orc_e4m3_encode_array", "orc_e2m1_encode_array"):
            getattr(L, nm).restype = None
            getattr(L, nm).argtypes = [P, I64, P]
        L.orc_bf16_from_double_array.restype = None
        L.orc_bf16_from_double_array.argtypes = [P, I64, P]
        L.orc_num_threads.restype = I
        L.orc_num_threads.argtypes = []
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------------------- codecs
def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e2m1_encode(v: float) -> int:
    return lib().orc_e2m1_encode(float(v))


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(float(v))


def e8m0_value(code: int) -> float:
    return lib().orc_e8m0_value(int(code))


def mx_exponent(amax: float, k: int) -> int:
    return lib().orc_mx_exponent(float(amax), int(k))


def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(int(bits))


def bf16_from_double(v: float) -> int:
    return lib().orc_bf16_from_double(float(v))


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float64).ravel()
    out = np.empty(x.size, np.uint8)
    lib().orc_e4m3_encode_array(_p(x), x.size, _p(out))
    return out


def e2m1_encode_array(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float64).ravel()
    out = np.empty(x.size, np.uint8)
    lib().orc_e2m1_encode_array(_p(x), x.size, _p(out))
    return out


def bf16_from_double_array(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float64).ravel()
    out = np.empty(x.size, np.uint16)
    lib().orc_bf16_from_double_array(_p(x), x.size, _p(out))
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact binary64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------- quantizers
LOG2E_F32 = np.float32(1.44269502162933349609375)


def exp2_scale(softmax_scale: float) -> float:
    """c2 = fl32(softmax_scale * log2 e): the factor Q is multiplied by before
    it is quantised, so that Q'K^T is the exponent argument in log2 units."""
    return float(np.float32(softmax_scale) * LOG2E_F32)


def quantize_qk4(x_bits: np.ndarray, smooth: bool = False, prescale: float = 1.0):
    """x [B,H,S,D] bf16 bits -> (codes [B,H,S,D/2] u8, scales [B,H,S,D/32] u8,
    kbar [B,H,ceil(S/128),D] bf16 bits or None).  Elements are multiplied by
    prescale in binary32 before quantisation (Q: exp2_scale(softmax_scale))."""
    x = _c(x_bits, np.uint16)
    B, H, S, D = x.shape
    codes = np.empty((B, H, S, D // 2), np.uint8)
    scales = np.empty((B, H, S, D // BLOCK), np.uint8)
    nt = (S + TILE - 1) // TILE
    kbar = np.empty((B, H, nt, D), np.uint16) if smooth else None
    lib().orc_quantize_qk4(_p(x), B, H, S, D, int(bool(smooth)), float(np.float32(prescale)), _p(codes),
                           _p(scales), _p(kbar))
    return codes, scales, kbar


def nvfp4_tensor_scale(amax: float) -> float:
    """Per-tensor NVFP4 scale as a power of two: the smallest 2^k with
    amax / (6 * 2^k) <= 448 (E2M1 max 6, E4M3 max 448); 1 for an all-zero tensor."""
    if not (amax > 0.0) or not math.isfinite(amax):
        return 1.0
    k = math.ceil(math.log2(amax / (6.0 * 448.0)))
    while amax / (6.0 * 2.0**k) > 448.0:
        k += 1
    while k > -126 and amax / (6.0 * 2.0**(k - 1)) <= 448.0:
        k -= 1
    return 2.0**k


def quantize_nvfp4(x_bits: np.ndarray, g: float, smooth: bool = False, prescale: float = 1.0):
    """x [B,H,S,D] bf16 bits -> NVFP4 (codes [B,H,S,D/2] u8, E4M3 scales [B,H,S,D/16] u8,
    kbar or None) with per-tensor scale g (a power of two)."""
    x = _c(x_bits, np.uint16)
    B, H, S, D = x.shape
    codes = np.empty((B, H, S, D // 2), np.uint8)
    scales = np.empty((B, H, S, D // 16), np.uint8)
    nt = (S + TILE - 1) // TILE
    kbar = np.empty((B, H, nt, D), np.uint16) if smooth else None
    lib().orc_quantize_nvfp4(_p(x), B, H, S, D, int(bool(smooth)), float(np.float32(prescale)), float(g), _p(codes),
                             _p(scales), _p(kbar))
    return codes, scales, kbar


def dequant_nvfp4(codes: np.ndarray, scales: np.ndarray, g: float) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    D = codes.shape[-1] * 2
    rows = codes.size // (D // 2)
    out = np.empty(codes.shape[:-1] + (D,), np.float64)
    lib().orc_dequant_nvfp4(_p(codes), _p(scales), rows, D, float(g), _p(out))
    return out


def quantize_v8(v_bits: np.ndarray):
    """v [B,H,S,D] bf16 bits -> (codes [B,H,ceil(S/32),D,32] u8, scales [B,H,ceil(S/32),D] u8)."""
    v = _c(v_bits, np.uint16)
    B, H, S, D = v.shape
    nb = (S + BLOCK - 1) // BLOCK
    codes = np.empty((B, H, nb, D, BLOCK), np.uint8)
    scales = np.empty((B, H, nb, D), np.uint8)
    lib().orc_quantize_v8(_p(v), B, H, S, D, _p(codes), _p(scales))
    return codes, scales


def quantize_v4(v_bits: np.ndarray):
    """v [B,H,S,D] bf16 bits -> MXFP4 (codes [B,H,ceil(S/32),D,16] u8, scales [B,H,ceil(S/32),D] u8)."""
    v = _c(v_bits, np.uint16)
    B, H, S, D = v.shape
    nb = (S + BLOCK - 1) // BLOCK
    codes = np.empty((B, H, nb, D, BLOCK // 2), np.uint8)
    scales = np.empty((B, H, nb, D), np.uint8)
    lib().orc_quantize_v4(_p(v), B, H, S, D, _p(codes), _p(scales))
    return codes, scales


def dequant_v4(codes: np.ndarray, scales: np.ndarray, S: int) -> np.ndarray:
    """One (b, h) slice: codes [nb,D,16], scales [nb,D] -> [S,D]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    D = codes.shape[-2]
    out = np.empty((S, D), np.float64)
    lib().orc_dequant_v4(_p(codes), _p(scales), S, D, _p(out))
    return out


def _quant_dequant_v(vq: np.ndarray, L: int, pv: int) -> np.ndarray:
    """V of one (b, kv head) [1,1,L,D] -> decoded [L,D] in the format of pv."""
    if pv == PV_FP4:
        vc, vs = quantize_v4(vq)
        return dequant_v4(vc[0, 0], vs[0, 0], L)
    vc, vs = quantize_v8(vq)
    return dequant_v8(vc[0, 0], vs[0, 0], L)


def dequant_qk4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    D = codes.shape[-1] * 2
    rows = codes.size // (D // 2)
    out = np.empty(codes.shape[:-1] + (D,), np.float64)
    lib().orc_dequant_qk4(_p(codes), _p(scales), rows, D, _p(out))
    return out


def dequant_v8(codes: np.ndarray, scales: np.ndarray, S: int) -> np.ndarray:
    """One (b, h) slice: codes [nb,D,32], scales [nb,D] -> [S,D]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    D = codes.shape[-2]
    out = np.empty((S, D), np.float64)
    lib().orc_dequant_v8(_p(codes), _p(scales), S, D, _p(out))
    return out


# ----------------------------------------------------------------------------- attention cores
def attn_exact_rows(Q, qpos, K, V, Sq, causal, softmax_scale):
    """(a) exact FP64 softmax attention for rows Q [n,D] against one kv head."""
    Q = _c(Q, np.float64)
    K = _c(K, np.float64)
    V = _c(V, np.float64)
    qpos = _c(qpos, np.int64)
    n, D = Q.shape
    L = K.shape[0]
    O = np.zeros((n, D), np.float64)
    lse = np.zeros(n, np.float64)
    lib().orc_attn_exact_rows(_p(Q), _p(qpos), n, _p(K), _p(V), L, Sq, D, int(bool(causal)),
                              float(softmax_scale), _p(O), _p(lse))
    return O, lse


def attn_quant_rows(Q, qpos, K, V, Sq, causal, softmax_scale, Qc=None, Kbar=None, split_tiles=0,
                    quantize_p=True, fp32_arg=True, p_mode=None):
    """(c) the method's online-softmax schedule for rows Q [n,D] of one kv head.
    Q holds pre-scaled query rows q' = c2 q (see exp2_scale), so Q K^T is in
    log2 units; softmax_scale still enters the compensation term.  p_mode
    (P_EXACT .. P_E2M1_BLOCK) overrides quantize_p (True: P_E4M3, False:
    P_EXACT)."""
    if p_mode is None:
        p_mode = P_E4M3 if quantize_p else P_EXACT
    Q = _c(Q, np.float64)
    K = _c(K, np.float64)
    V = _c(V, np.float64)
    Qc = None if Qc is None else _c(Qc, np.float64)
    Kbar = None if Kbar is None else _c(Kbar, np.float64)
    qpos = _c(qpos, np.int64)
    n, D = Q.shape
    L = K.shape[0]
    O = np.zeros((n, D), np.float64)
    lse = np.zeros(n, np.float64)
    lib().orc_attn_quant_rows(_p(Q), _p(Qc), _p(qpos), n, _p(K), _p(Kbar), _p(V), L, Sq, D,
                              int(bool(causal)), float(np.float32(softmax_scale)), int(split_tiles),
                              int(p_mode), int(bool(fp32_arg)), _p(O), _p(lse))
    return O, lse


# ----------------------------------------------------------------------------- whole-path drivers
def _rows_by_group(rows: np.ndarray, Hq: int, Hkv: int):
    """rows [n,3] of (b, h, i) -> {(b, g): indices}"""
    G = Hq // Hkv
    groups = {}
    for idx, (b, h, _) in enumerate(rows):
        groups.setdefault((int(b), int(h) // G), []).append(idx)
    return groups


def prefill_rows(q_bits, k_bits, v_bits, rows: Sequence, causal: bool, softmax_scale: float,
                 smooth: bool = False, exact: bool = True, pv: int = PV_FP8, nvfp4=None):
    """Quantise Q/K/V with the oracle's quantizers and evaluate the listed rows.

    q_bits [B,Hq,Sq,D], k_bits/v_bits [B,Hkv,Skv,D] (bf16 bit patterns, uint16).
    rows: array [n,3] of (b, h, i).  Returns dict with O_q, lse_q (method) and,
    if exact, O_x, lse_x (exact FP64 attention on the bf16 inputs).  pv picks
    the P/V format: PV_FP8 (the method), PV_FP8_BLOCKP or PV_FP4.  nvfp4 =
    (g_q, g_k): Q and K in NVFP4 with those per-tensor scales instead of MXFP4.
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    B, Hq, Sq, D = q_bits.shape
    Hkv, Skv = k_bits.shape[1], k_bits.shape[2]
    G = Hq // Hkv
    n = rows.shape[0]
    out = {"O_q": np.zeros((n, D)), "lse_q": np.zeros(n)}
    if exact:
        out["O_x"] = np.zeros((n, D))
        out["lse_x"] = np.zeros(n)
    for (b, g), idx in _rows_by_group(rows, Hq, Hkv).items():
        idx = np.asarray(idx)
        r = rows[idx]
        kq = np.ascontiguousarray(k_bits[b:b + 1, g:g + 1])
        vq = np.ascontiguousarray(v_bits[b:b + 1, g:g + 1])
        if nvfp4 is None:
            kc, ks, kb = quantize_qk4(kq, smooth=smooth)
            Kd = dequant_qk4(kc, ks)[0, 0]
        else:
            kc, ks, kb = quantize_nvfp4(kq, nvfp4[1], smooth=smooth)
            Kd = dequant_nvfp4(kc, ks, nvfp4[1])[0, 0]
        Vd = _quant_dequant_v(vq, Skv, pv)
        Kbar = bf16_to_f64(kb[0, 0]) if smooth else None
        # query rows: quantise each needed (b, h) head once
        Qd = np.zeros((len(idx), D))
        Qc = np.zeros((len(idx), D))
        for h in np.unique(r[:, 1]):
            sel = np.nonzero(r[:, 1] == h)[0]
            qh = np.ascontiguousarray(q_bits[b:b + 1, h:h + 1])
            if nvfp4 is None:
                qc_, qs_, _ = quantize_qk4(qh, prescale=exp2_scale(softmax_scale))
                qd = dequant_qk4(qc_, qs_)[0, 0]
            else:
                qc_, qs_, _ = quantize_nvfp4(qh, nvfp4[0], prescale=exp2_scale(softmax_scale))
                qd = dequant_nvfp4(qc_, qs_, nvfp4[0])[0, 0]
            Qd[sel] = qd[r[sel, 2]]
            Qc[sel] = bf16_to_f64(q_bits[b, h][r[sel, 2]])
        O, lse = attn_quant_rows(Qd, r[:, 2], Kd, Vd, Sq, causal, softmax_scale,
                                 Qc=Qc if smooth else None, Kbar=Kbar, p_mode=_P_MODE_OF_PV[pv])
        out["O_q"][idx] = O
        out["lse_q"][idx] = lse
        if exact:
            Ox, lx = attn_exact_rows(bf16_to_f64(q_bits[b][r[:, 1], r[:, 2]]), r[:, 2],
                                     bf16_to_f64(k_bits[b, g]), bf16_to_f64(v_bits[b, g]), Sq, causal,
                                     softmax_scale)
            out["O_x"][idx] = Ox
            out["lse_x"][idx] = lx
    return out


def prefill_rows_from_codes(q4, q4s, k4, k4s, v8, v8s, rows: Sequence, causal: bool, softmax_scale: float,
                            q_bits=None, kbar_bits=None) -> dict:
    """(c) for the listed rows (b, h, i) of tensors the oracle has already
    quantised (quantize_qk4 of Q with prescale exp2_scale(softmax_scale), of K,
    and quantize_v8 of V); q_bits and kbar_bits (bf16) give the compensation
    term when K was smoothed.  Decodes each KV head and the rows' Q, then runs
    the online schedule.  Returns O_q, lse_q."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    B, Hq, Sq, Dh = q4.shape
    D = 2 * Dh
    Hkv, Skv = k4.shape[1], k4.shape[2]
    n = rows.shape[0]
    out = {"O_q": np.zeros((n, D)), "lse_q": np.zeros(n)}
    for (b, g), idx in _rows_by_group(rows, Hq, Hkv).items():
        idx = np.asarray(idx)
        r = rows[idx]
        Kd = dequant_qk4(k4[b, g], k4s[b, g])
        Vd = dequant_v8(v8[b, g], v8s[b, g], Skv)
        Qd = dequant_qk4(q4[b][r[:, 1], r[:, 2]], q4s[b][r[:, 1], r[:, 2]])
        smooth = kbar_bits is not None
        Qc = bf16_to_f64(q_bits[b][r[:, 1], r[:, 2]]) if smooth else None
        Kbar = bf16_to_f64(kbar_bits[b, g]) if smooth else None
        O, lse = attn_quant_rows(Qd, r[:, 2], Kd, Vd, Sq, causal, softmax_scale, Qc=Qc, Kbar=Kbar)
        out["O_q"][idx] = O
        out["lse_q"][idx] = lse
    return out


def decode_rows(q_bits, k_bits, v_bits, rows: Sequence, softmax_scale: float, num_splits: int,
                kv_lens: Optional[Sequence[int]] = None, exact: bool = True, pv: int = PV_FP8, nvfp4=None):
    """Decode (one query token per sequence) with the split-KV schedule.

    q_bits [B,Hq,1,D]; k_bits/v_bits [B,Hkv,Smax,D].  rows [n,3] of (b, h, 0).
    kv_lens[b] keys of sequence b are used (default: all).  Split s of sequence
    b covers tiles [s*T, (s+1)*T) with T = ceil(ceil(L_b/128)/num_splits).
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    B, Hq, _, D = q_bits.shape
    Hkv, Smax = k_bits.shape[1], k_bits.shape[2]
    n = rows.shape[0]
    out = {"O_q": np.zeros((n, D)), "lse_q": np.zeros(n)}
    if exact:
        out["O_x"] = np.zeros((n, D))
        out["lse_x"] = np.zeros(n)
    for (b, g), idx in _rows_by_group(rows, Hq, Hkv).items():
        idx = np.asarray(idx)
        r = rows[idx]
        L = int(kv_lens[b]) if kv_lens is not None else Smax
        nt = (L + TILE - 1) // TILE
        per = max(1, -(-nt // max(1, num_splits)))
        kq = np.ascontiguousarray(k_bits[b:b + 1, g:g + 1, :L])
        vq = np.ascontiguousarray(v_bits[b:b + 1, g:g + 1, :L])
        if nvfp4 is None:
            kc, ks, _ = quantize_qk4(kq)
            Kd = dequant_qk4(kc, ks)[0, 0]
        else:
            kc, ks, _ = quantize_nvfp4(kq, nvfp4[1])
            Kd = dequant_nvfp4(kc, ks, nvfp4[1])[0, 0]
        Vd = _quant_dequant_v(vq, L, pv)
        Qd = np.zeros((len(idx), D))
        for j, (bb, h, _) in enumerate(r):
            qh = np.ascontiguousarray(q_bits[bb:bb + 1, h:h + 1])
            if nvfp4 is None:
                qc_, qs_, _ = quantize_qk4(qh, prescale=exp2_scale(softmax_scale))
                Qd[j] = dequant_qk4(qc_, qs_)[0, 0, 0]
            else:
                qc_, qs_, _ = quantize_nvfp4(qh, nvfp4[0], prescale=exp2_scale(softmax_scale))
                Qd[j] = dequant_nvfp4(qc_, qs_, nvfp4[0])[0, 0, 0]
        O, lse = attn_quant_rows(Qd, np.zeros(len(idx), np.int64), Kd, Vd, 1, False, softmax_scale,
                                 split_tiles=per, p_mode=_P_MODE_OF_PV[pv])
        out["O_q"][idx] = O
        out["lse_q"][idx] = lse
        if exact:
            Ox, lx = attn_exact_rows(bf16_to_f64(q_bits[b][r[:, 1], 0]), np.zeros(len(idx), np.int64),
                                     bf16_to_f64(k_bits[b, g, :L]), bf16_to_f64(v_bits[b, g, :L]), 1,
                                     False, softmax_scale)
            out["O_x"][idx] = Ox
            out["lse_x"][idx] = lx
    return out


def num_threads() -> int:
    return lib().orc_num_threads()
