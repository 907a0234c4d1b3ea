"""Python binding of libqfa, the QK4PV8 attention forward library for MI355X.

Every function named ``qfa_*`` mirrors the C entry point of the same name in
``include/qfa.h``: it only marshals torch tensors (device memory) and the
current HIP stream into the call, and raises ``QfaError`` on a non-OK status.
All arithmetic runs in the HIP kernels of ``libqfa.so``; there is no fallback
path -- if the library is not built, importing works but the first call raises.

The ``quantize_*`` / ``fwd_*`` helpers allocate the outputs with torch and call
the ``qfa_*`` functions.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqfa.so")

QFA_OK = 0
QFA_ERR_INVALID_ARG = 1
QFA_ERR_UNSUPPORTED = 2
QFA_ERR_WORKSPACE = 3
QFA_ERR_HIP = 4

# P/V formats (qfa_pv_format): the method, FP8 P with a scale per (row, 32
# keys), MXFP4 P and V
QFA_PV_FP8 = 0
QFA_PV_FP8_BLOCKP = 1
QFA_PV_FP4 = 2

EXPORTS = (
    "qfa_quantize_qk4", "qfa_quantize_v8", "qfa_fwd_prefill", "qfa_fwd_decode",
    "qfa_decode_workspace_bytes", "qfa_decode_default_splits", "qfa_exp2_scale", "qfa_kv_append",
    "qfa_fwd_prefill_ex", "qfa_fwd_decode_ex", "qfa_quantize_v4",
    "qfa_quantize_nvfp4", "qfa_fwd_prefill_nvfp4", "qfa_fwd_decode_nvfp4", "qfa_kv_append_ex",
    "qfa_status_string", "qfa_version", "qfa_fwd_decode_noalloc",
)

# Capacity of the library-owned decode scratch of qfa_fwd_decode_noalloc (include/qfa.h)
QFA_DECODE_NOALLOC_MAX_BYTES = 32 << 20

_lib = None


class QfaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s" % (fn, status_string(status)))


def lib() -> ctypes.CDLL:
    """Load libqfa.so (built in-tree by ``python -m bit_quantized_attention_qk4pv8_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libqfa.so is not built; run `python -m bit_quantized_attention_qk4pv8_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.qfa_quantize_qk4.restype = I
        L.qfa_quantize_qk4.argtypes = [P, I, I, I, I, I, I, F, P, P, P, P]
        L.qfa_quantize_v8.restype = I
        L.qfa_quantize_v8.argtypes = [P, I, I, I, I, I, P, P, P]
        L.qfa_quantize_nvfp4.restype = I
        L.qfa_quantize_nvfp4.argtypes = [P, I, I, I, I, I, I, F, F, P, P, P, P]
        L.qfa_fwd_prefill_nvfp4.restype = I
        L.qfa_fwd_prefill_nvfp4.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, F, F, P, P, P]
        L.qfa_fwd_decode_nvfp4.restype = I
        L.qfa_fwd_decode_nvfp4.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, P, I, F, F, F, ctypes.POINTER(I), P,
                                           SZ, P, P, P]
        L.qfa_quantize_v4.restype = I
        L.qfa_quantize_v4.argtypes = [P, I, I, I, I, I, P, P, P]
        L.qfa_fwd_prefill.restype = I
        L.qfa_fwd_prefill.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, P, P]
        L.qfa_fwd_decode.restype = I
        L.qfa_fwd_decode.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, P, I, F, I, ctypes.POINTER(I), P, SZ, P,
                                     P, P]
        L.qfa_fwd_decode_noalloc.restype = I
        L.qfa_fwd_decode_noalloc.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, P, I, F, I, ctypes.POINTER(I), P,
                                             P, P]
        L.qfa_fwd_prefill_ex.restype = I
        L.qfa_fwd_prefill_ex.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, I, P, P, P]
        L.qfa_fwd_decode_ex.restype = I
        L.qfa_fwd_decode_ex.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, P, I, F, I, I, ctypes.POINTER(I), P,
                                        SZ, P, P, P]
        L.qfa_decode_workspace_bytes.restype = SZ
        L.qfa_decode_workspace_bytes.argtypes = [I, I, I, I]
        L.qfa_decode_default_splits.restype = I
        L.qfa_decode_default_splits.argtypes = [I, I, I]
        L.qfa_kv_append_ex.restype = I
        L.qfa_kv_append_ex.argtypes = [P, P, I, I, I, I, I, I, P, P, P, P, P, P, P, P, I, F, P]
        L.qfa_kv_append.restype = I
        L.qfa_kv_append.argtypes = [P, P, I, I, I, I, I, I, P, P, P, P, P, P, P, P, P]
        L.qfa_exp2_scale.restype = F
        L.qfa_exp2_scale.argtypes = [F]
        L.qfa_status_string.restype = ctypes.c_char_p
        L.qfa_status_string.argtypes = [I]
        L.qfa_version.restype = I
        L.qfa_version.argtypes = []
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().qfa_status_string(int(status)).decode()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libqfa must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != QFA_OK:
        raise QfaError(fn, status)


def _u16(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


# ----------------------------------------------------------------------------- C entry points
def qfa_version() -> int:
    return lib().qfa_version()


def qfa_decode_workspace_bytes(B: int, Hq: int, D: int, num_splits: int) -> int:
    return lib().qfa_decode_workspace_bytes(B, Hq, D, num_splits)


def qfa_decode_default_splits(B: int, Hkv: int, S_kv_max: int) -> int:
    return lib().qfa_decode_default_splits(B, Hkv, S_kv_max)


def qfa_exp2_scale(softmax_scale: float) -> float:
    return lib().qfa_exp2_scale(float(softmax_scale))


def qfa_quantize_qk4(x, B, H, S, D, block_size, smooth, prescale, codes, scales, kbar, stream=None):
    _check("qfa_quantize_qk4", lib().qfa_quantize_qk4(_ptr(_u16(x)), B, H, S, D, block_size, int(smooth),
                                                      float(prescale), _ptr(codes), _ptr(scales), _ptr(kbar),
                                                      _stream(stream)))


def qfa_quantize_v8(v, B, H, S, D, block_size, codes, scales, stream=None):
    _check("qfa_quantize_v8", lib().qfa_quantize_v8(_ptr(_u16(v)), B, H, S, D, block_size, _ptr(codes),
                                                    _ptr(scales), _stream(stream)))


def qfa_quantize_nvfp4(x, B, H, S, D, block_size, smooth, prescale, tensor_scale, codes, scales, kbar,
                       stream=None):
    _check("qfa_quantize_nvfp4", lib().qfa_quantize_nvfp4(
        _ptr(_u16(x)), B, H, S, D, block_size, int(smooth), float(prescale), float(tensor_scale), _ptr(codes),
        _ptr(scales), _ptr(None if kbar is None else _u16(kbar)), _stream(stream)))


def qfa_fwd_prefill_nvfp4(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_q, S_kv, D, causal, softmax_scale,
                          q_tensor_scale, k_tensor_scale, O, lse, stream=None):
    _check("qfa_fwd_prefill_nvfp4", lib().qfa_fwd_prefill_nvfp4(
        _ptr(q4), _ptr(q4s), _ptr(k4), _ptr(k4s), _ptr(None if kbar is None else _u16(kbar)),
        _ptr(None if q_bf16 is None else _u16(q_bf16)), _ptr(v8), _ptr(v8s), B, Hq, Hkv, S_q, S_kv, D,
        int(causal), float(softmax_scale), float(q_tensor_scale), float(k_tensor_scale), _ptr(O), _ptr(lse),
        _stream(stream)))


def qfa_fwd_decode_nvfp4(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_kv_max, kv_lens, D, softmax_scale,
                         q_tensor_scale, k_tensor_scale, num_splits, workspace, workspace_bytes, O, lse,
                         stream=None) -> int:
    ns = ctypes.c_int(int(num_splits))
    _check("qfa_fwd_decode_nvfp4", lib().qfa_fwd_decode_nvfp4(
        _ptr(q4), _ptr(q4s), _ptr(k4), _ptr(k4s), _ptr(None if kbar is None else _u16(kbar)),
        _ptr(None if q_bf16 is None else _u16(q_bf16)), _ptr(v8), _ptr(v8s), B, Hq, Hkv, S_kv_max,
        _ptr(kv_lens), D, float(softmax_scale), float(q_tensor_scale), float(k_tensor_scale), ctypes.byref(ns),
        _ptr(workspace), int(workspace_bytes), _ptr(O), _ptr(lse), _stream(stream)))
    return ns.value


def qfa_quantize_v4(v, B, H, S, D, block_size, codes, scales, stream=None):
    _check("qfa_quantize_v4", lib().qfa_quantize_v4(_ptr(_u16(v)), B, H, S, D, block_size, _ptr(codes),
                                                    _ptr(scales), _stream(stream)))


def qfa_fwd_prefill(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_q, S_kv, D, causal, softmax_scale,
                    block_size, O, lse, stream=None):
    _check("qfa_fwd_prefill", lib().qfa_fwd_prefill(
        _ptr(q4), _ptr(q4s), _ptr(k4), _ptr(k4s), _ptr(None if kbar is None else _u16(kbar)),
        _ptr(None if q_bf16 is None else _u16(q_bf16)), _ptr(v8), _ptr(v8s), B, Hq, Hkv, S_q, S_kv, D,
        int(causal), float(softmax_scale), block_size, _ptr(O), _ptr(lse), _stream(stream)))


def qfa_fwd_decode(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_kv_max, kv_lens, D, softmax_scale,
                   block_size, num_splits, workspace, workspace_bytes, O, lse, stream=None) -> int:
    ns = ctypes.c_int(int(num_splits))
    _check("qfa_fwd_decode", lib().qfa_fwd_decode(
        _ptr(q4), _ptr(q4s), _ptr(k4), _ptr(k4s), _ptr(None if kbar is None else _u16(kbar)),
        _ptr(None if q_bf16 is None else _u16(q_bf16)), _ptr(v8), _ptr(v8s), B, Hq, Hkv, S_kv_max,
        _ptr(kv_lens), D, float(softmax_scale), block_size, ctypes.byref(ns), _ptr(workspace),
        int(workspace_bytes), _ptr(O), _ptr(lse), _stream(stream)))
    return ns.value


def qfa_fwd_decode_noalloc(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_kv_max, kv_lens, D,
                           softmax_scale, block_size, num_splits, O, lse, stream=None) -> int:
    ns = ctypes.c_int(int(num_splits))
    _check("qfa_fwd_decode_noalloc", lib().qfa_fwd_decode_noalloc(
        _ptr(q4), _ptr(q4s), _ptr(k4), _ptr(k4s), _ptr(None if kbar is None else _u16(kbar)),
        _ptr(None if q_bf16 is None else _u16(q_bf16)), _ptr(v8), _ptr(v8s), B, Hq, Hkv, S_kv_max,
        _ptr(kv_lens), D, float(softmax_scale), block_size, ctypes.byref(ns), _ptr(O), _ptr(lse), _stream(stream)))
    return ns.value


def qfa_fwd_prefill_ex(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_q, S_kv, D, causal, softmax_scale,
                       block_size, pv_format, O, lse, stream=None):
    _check("qfa_fwd_prefill_ex", lib().qfa_fwd_prefill_ex(
        _ptr(q4), _ptr(q4s), _ptr(k4), _ptr(k4s), _ptr(None if kbar is None else _u16(kbar)),
        _ptr(None if q_bf16 is None else _u16(q_bf16)), _ptr(v8), _ptr(v8s), B, Hq, Hkv, S_q, S_kv, D,
        int(causal), float(softmax_scale), block_size, int(pv_format), _ptr(O), _ptr(lse), _stream(stream)))


def qfa_fwd_decode_ex(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_kv_max, kv_lens, D, softmax_scale,
                      block_size, pv_format, num_splits, workspace, workspace_bytes, O, lse, stream=None) -> int:
    ns = ctypes.c_int(int(num_splits))
    _check("qfa_fwd_decode_ex", lib().qfa_fwd_decode_ex(
        _ptr(q4), _ptr(q4s), _ptr(k4), _ptr(k4s), _ptr(None if kbar is None else _u16(kbar)),
        _ptr(None if q_bf16 is None else _u16(q_bf16)), _ptr(v8), _ptr(v8s), B, Hq, Hkv, S_kv_max,
        _ptr(kv_lens), D, float(softmax_scale), block_size, int(pv_format), ctypes.byref(ns), _ptr(workspace),
        int(workspace_bytes), _ptr(O), _ptr(lse), _stream(stream)))
    return ns.value


def qfa_kv_append_ex(k_new, v_new, B, Hkv, n_new, D, S_kv_max, block_size, kv_lens, k4, k4s, kbar, v8, v8s,
                     k_tail, v_tail, pv_format, k_tensor_scale, stream=None):
    _check("qfa_kv_append_ex", lib().qfa_kv_append_ex(
        _ptr(_u16(k_new)), _ptr(_u16(v_new)), B, Hkv, n_new, D, S_kv_max, block_size, _ptr(kv_lens), _ptr(k4),
        _ptr(k4s), _ptr(None if kbar is None else _u16(kbar)), _ptr(v8), _ptr(v8s),
        _ptr(None if k_tail is None else _u16(k_tail)), _ptr(_u16(v_tail)), int(pv_format), float(k_tensor_scale),
        _stream(stream)))


def qfa_kv_append(k_new, v_new, B, Hkv, n_new, D, S_kv_max, block_size, kv_lens, k4, k4s, kbar, v8, v8s, k_tail,
                  v_tail, stream=None):
    _check("qfa_kv_append", lib().qfa_kv_append(
        _ptr(_u16(k_new)), _ptr(_u16(v_new)), B, Hkv, n_new, D, S_kv_max, block_size, _ptr(kv_lens), _ptr(k4),
        _ptr(k4s), _ptr(None if kbar is None else _u16(kbar)), _ptr(v8), _ptr(v8s),
        _ptr(None if k_tail is None else _u16(k_tail)), _ptr(_u16(v_tail)), _stream(stream)))


# ----------------------------------------------------------------------------- allocating helpers
def kv_cache(B: int, Hkv: int, S_kv_max: int, D: int, smooth: bool = False, device="cuda",
             pv_format: int = QFA_PV_FP8, k_tensor_scale: float = 0.0):
    """Empty pre-quantised KV cache (the layouts the decode entry points read) plus the bf16
    tails qfa_kv_append keeps between calls.  pv_format QFA_PV_FP4: V in MXFP4;
    k_tensor_scale > 0: K in NVFP4 with that tensor scale."""
    nvb, nt = (S_kv_max + 31) // 32, (S_kv_max + 127) // 128
    u8 = dict(dtype=torch.uint8, device=device)
    ks = D // 16 if k_tensor_scale > 0 else D // 32
    vr = 16 if pv_format == QFA_PV_FP4 else 32
    c = {"k4": torch.zeros((B, Hkv, S_kv_max, D // 2), **u8), "k4s": torch.zeros((B, Hkv, S_kv_max, ks), **u8),
         "v8": torch.zeros((B, Hkv, nvb, D, vr), **u8), "v8s": torch.zeros((B, Hkv, nvb, D), **u8),
         "v_tail": torch.zeros((B, Hkv, 128, D), dtype=torch.bfloat16, device=device),
         "kbar": None, "k_tail": None, "S": S_kv_max, "pv_format": pv_format, "k_tensor_scale": k_tensor_scale}
    if smooth:
        c["kbar"] = torch.zeros((B, Hkv, nt, D), dtype=torch.bfloat16, device=device)
        c["k_tail"] = torch.zeros((B, Hkv, 128, D), dtype=torch.bfloat16, device=device)
    return c


def kv_append(cache, k_new: torch.Tensor, v_new: torch.Tensor, kv_lens=None, stream=None):
    """Append bf16 k_new, v_new [B,Hkv,n,D] at kv_lens (device int32 [B] or None = empty cache)."""
    B, Hkv, n, D = k_new.shape
    qfa_kv_append_ex(k_new, v_new, B, Hkv, n, D, cache["S"], 32, kv_lens, cache["k4"], cache["k4s"], cache["kbar"],
                     cache["v8"], cache["v8s"], cache["k_tail"], cache["v_tail"], cache.get("pv_format", QFA_PV_FP8),
                     cache.get("k_tensor_scale", 0.0), stream)


def quantize_qk4(x: torch.Tensor, smooth: bool = False, prescale: float = 1.0, stream=None):
    """x bf16 [B,H,S,D] on the GPU -> (codes u8 [B,H,S,D/2], scales u8 [B,H,S,D/32], kbar bf16 or None).

    Q takes prescale = qfa_exp2_scale(softmax_scale), K takes 1."""
    B, H, S, D = x.shape
    codes = torch.empty((B, H, S, D // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, H, S, D // 32), dtype=torch.uint8, device=x.device)
    kbar = torch.empty((B, H, (S + 127) // 128, D), dtype=torch.bfloat16, device=x.device) if smooth else None
    qfa_quantize_qk4(x, B, H, S, D, 32, smooth, prescale, codes, scales, kbar, stream)
    return codes, scales, kbar


def quantize_v8(v: torch.Tensor, stream=None):
    """v bf16 [B,H,S,D] -> (codes u8 [B,H,ceil(S/32),D,32], scales u8 [B,H,ceil(S/32),D])."""
    B, H, S, D = v.shape
    nb = (S + 31) // 32
    codes = torch.empty((B, H, nb, D, 32), dtype=torch.uint8, device=v.device)
    scales = torch.empty((B, H, nb, D), dtype=torch.uint8, device=v.device)
    qfa_quantize_v8(v, B, H, S, D, 32, codes, scales, stream)
    return codes, scales


def nvfp4_tensor_scale(amax: float) -> float:
    """Per-tensor NVFP4 scale: the smallest power of two g with amax / (6 g) <= 448
    (1 for an all-zero or non-finite amax).  Host arithmetic only."""
    amax = float(amax)
    if not (amax > 0.0) or not math.isfinite(amax):
        return 1.0
    m, e = math.frexp(amax / (6.0 * 448.0))  # value = m * 2^e, m in [0.5, 1)
    k = e - 1 if m == 0.5 else e             # smallest k with 2^k >= value
    return math.ldexp(1.0, max(k, -126))


def quantize_nvfp4(x: torch.Tensor, tensor_scale: float, smooth: bool = False, prescale: float = 1.0, stream=None):
    """x bf16 [B,H,S,D] -> NVFP4 (codes u8 [B,H,S,D/2], E4M3 scales u8 [B,H,S,D/16], kbar or None)."""
    B, H, S, D = x.shape
    codes = torch.empty((B, H, S, D // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, H, S, D // 16), dtype=torch.uint8, device=x.device)
    kbar = torch.empty((B, H, (S + 127) // 128, D), dtype=torch.bfloat16, device=x.device) if smooth else None
    qfa_quantize_nvfp4(x, B, H, S, D, 16, smooth, prescale, tensor_scale, codes, scales, kbar, stream)
    return codes, scales, kbar


def quantize_v4(v: torch.Tensor, stream=None):
    """v bf16 [B,H,S,D] -> MXFP4 (codes u8 [B,H,ceil(S/32),D,16], scales u8 [B,H,ceil(S/32),D])."""
    B, H, S, D = v.shape
    nb = (S + 31) // 32
    codes = torch.empty((B, H, nb, D, 16), dtype=torch.uint8, device=v.device)
    scales = torch.empty((B, H, nb, D), dtype=torch.uint8, device=v.device)
    qfa_quantize_v4(v, B, H, S, D, 32, codes, scales, stream)
    return codes, scales


def fwd_prefill(q4, q4s, k4, k4s, v8, v8s, S_kv: int, causal: bool, softmax_scale: float, kbar=None,
                q_bf16=None, with_lse: bool = True, pv_format: int = QFA_PV_FP8, stream=None):
    """q4/q4s None: the kernel quantises q_bf16 [B,Hq,S_q,D] itself.  pv_format
    picks the P/V format (v8/v8s then hold V in that format)."""
    if q4 is None:
        B, Hq, S_q, D = q_bf16.shape
    else:
        B, Hq, S_q, Dh = q4.shape
        D = Dh * 2
    Hkv = k4.shape[1]
    O = torch.empty((B, Hq, S_q, D), dtype=torch.float32, device=k4.device)
    lse = torch.empty((B, Hq, S_q), dtype=torch.float32, device=k4.device) if with_lse else None
    qfa_fwd_prefill_ex(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_q, S_kv, D, causal, softmax_scale,
                       32, pv_format, O, lse, stream)
    return O, lse


def fwd_decode(q4, q4s, k4, k4s, v8, v8s, S_kv_max: int, softmax_scale: float, num_splits: int = 0,
               kv_lens=None, kbar=None, q_bf16=None, workspace=None, pv_format: int = QFA_PV_FP8, stream=None):
    """q4 [B,Hq,1,D/2] (or None: the kernel quantises q_bf16 [B,Hq,1,D]);
    returns (O [B,Hq,D], lse [B,Hq], splits used)."""
    if q4 is None:
        B, Hq, _, D = q_bf16.shape
    else:
        B, Hq, _, Dh = q4.shape
        D = Dh * 2
    Hkv = k4.shape[1]
    splits = num_splits if num_splits > 0 else qfa_decode_default_splits(B, Hkv, S_kv_max)
    nbytes = qfa_decode_workspace_bytes(B, Hq, D, splits)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=k4.device)
    O = torch.empty((B, Hq, D), dtype=torch.float32, device=k4.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=k4.device)
    used = qfa_fwd_decode_ex(q4, q4s, k4, k4s, kbar, q_bf16, v8, v8s, B, Hq, Hkv, S_kv_max, kv_lens, D,
                             softmax_scale, 32, pv_format, splits, workspace, workspace.numel(), O, lse, stream)
    return O, lse, used
