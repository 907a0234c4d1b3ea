"""Algorithmic work and roofline accounting for the QK4PV8 path on MI355X.

Peaks are AMD's published dense figures for MI355X: MXFP4 10.1 PFLOP/s,
FP8 5.0 PFLOP/s, BF16 2.5 PFLOP/s, HBM3E 8 TB/s.

Prefill: Q K^T runs on MXFP4 and P V on FP8, so the time at 100% of the MFMA
roofline is F_QK / P_fp4 + F_PV / P_fp8 (+ F_comp / P_bf16 for the rank-one
compensation), with F_QK = F_PV = 2 D per visible (query, key) pair; masked
pairs are not counted.  The "blended" peak is total FLOPs over that time.

Decode: bytes of the KV cache actually read -- per token per kv head D/2 bytes
of K codes, D/32 of K scales, D of V codes, D/32 of V scales (200 B at D=128)
-- plus the bf16 query and the FP32 output, following the KV-cache byte
formula of the MXFP4 notes (section 1.1): 2 x layers x kv heads x head dim x
sequence x bytes x batch for an unquantised cache.
"""
from __future__ import annotations

PEAK_FP4 = 10.1e15
PEAK_FP8 = 5.0e15
PEAK_BF16 = 2.5e15
PEAK_HBM = 8.0e12


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int, bytes_per_element: float,
                   batch: int) -> int:
    return int(2 * layers * kv_heads * head_dim * seq_len * bytes_per_element * batch)


def decode_algorithmic_bytes(B: int, Hq: int, Hkv: int, L: int, D: int, include_q_o: bool = True,
                             v_fp4: bool = False, k_nvfp4: bool = False) -> int:
    """v_fp4: V held in MXFP4 (D/2 bytes of codes per token) instead of E4M3;
    k_nvfp4: K's scales are E4M3 per 16 channels (D/16 bytes per token)."""
    per_tok = D // 2 + (D // 16 if k_nvfp4 else D // 32) + (D // 2 if v_fp4 else D) + D // 32
    total = B * Hkv * L * per_tok
    if include_q_o:
        total += B * Hq * D * 2 + B * Hq * D * 4
    return total


def prefill_roof_seconds(flops_qkpv: float, comp_flops: float = 0.0, pv_fp4: bool = False,
                         qk_bf16: bool = False) -> float:
    """pv_fp4: P V also on the MXFP4 MFMA (the full-FP4 contrast case);
    qk_bf16: Q K^T on the bf16 MFMA (the NVFP4 emulation)."""
    half = flops_qkpv / 2.0
    return (half / (PEAK_BF16 if qk_bf16 else PEAK_FP4) + half / (PEAK_FP4 if pv_fp4 else PEAK_FP8)
            + comp_flops / PEAK_BF16)


def blended_peak(flops_qkpv: float, comp_flops: float = 0.0, pv_fp4: bool = False, qk_bf16: bool = False) -> float:
    return (flops_qkpv + comp_flops) / prefill_roof_seconds(flops_qkpv, comp_flops, pv_fp4, qk_bf16)
