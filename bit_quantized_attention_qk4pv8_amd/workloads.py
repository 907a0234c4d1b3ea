"""Seeded synthetic workloads shaped like the pages' attention layers.

This module only draws inputs; it holds none of the method's arithmetic.  It
serves both the GPU path and the CPU oracle (the tests hand the same bf16
tensors to each side).  Every tensor is standard-normal float32 drawn by a
seeded torch generator on the target device, shaped/perturbed as listed below,
then rounded to bf16 (round to nearest even, torch's conversion).

Workloads (the pages measure on Llama-3.1-8B / Qwen3-14B serving and five
unnamed benchmark suites; these synthetic tensors stand in for them):
  tiny     B1 Hq2 Hkv2 S256 D64, non-causal, scale 1/8
  llama16k B1 Hq32 Hkv8 S16384 D128 causal; 4 of 128 K channels and 2 of 128 Q
           channels scaled x20 (indices drawn by the seed, shared by all heads
           and tokens)
  qwen32k  B1 Hq40 Hkv8 S32768 D128 causal, rank-one compensation on; K gets a
           per-(kv head, channel) offset ~ N(0, 3^2) shared by all tokens
  long128k B1 Hq32 Hkv8 S131072 D128 causal; exactly floor(0.01 S) K rows
           (tokens) per kv head, chosen by the seed, scaled x8 across all D
  decode   B64, one query token each, Hq32 Hkv8 D128, 32768 cached keys per
           sequence, 16 KV splits + log-sum-exp merge
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    S_q: int
    S_kv: int
    D: int
    causal: bool
    smooth: bool
    decode: bool = False
    num_splits: int = 0
    softmax_scale: float = 0.0
    notes: str = ""

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale else 1.0 / math.sqrt(self.D)

    def pairs(self) -> int:
        """Visible (query, key) pairs = unmasked score elements."""
        if not self.causal:
            return self.B * self.Hq * self.S_q * self.S_kv
        off = self.S_kv - self.S_q
        tot = 0
        # rows i see min(S_kv, max(0, i + off + 1)) keys
        lo = max(0, -off)
        n_full_start = max(lo, self.S_kv - off)  # rows from here see all keys
        for_rows = range(lo, min(self.S_q, n_full_start))
        tot = sum(i + off + 1 for i in for_rows)
        if n_full_start < self.S_q:
            tot += (self.S_q - n_full_start) * self.S_kv
        return self.B * self.Hq * tot

    def flops(self) -> float:
        """Algorithmic FLOPs: 2D for Q K^T plus 2D for P V per visible pair."""
        return 4.0 * self.D * self.pairs()

    def comp_flops(self) -> float:
        """Rank-one compensation term: 2D per (row, visible 128-key tile)."""
        if not self.smooth:
            return 0.0
        tiles = 0
        off = self.S_kv - self.S_q
        for i in range(self.S_q):
            last = min(self.S_kv - 1, i + off) if self.causal else self.S_kv - 1
            if last >= 0:
                tiles += last // 128 + 1
        return 2.0 * self.D * self.B * self.Hq * tiles


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 2, 2, 256, 256, 64, False, False, softmax_scale=0.125),
    "llama16k": Workload("llama16k", 1, 32, 8, 16384, 16384, 128, True, False),
    "qwen32k": Workload("qwen32k", 1, 40, 8, 32768, 32768, 128, True, True),
    "long128k": Workload("long128k", 1, 32, 8, 131072, 131072, 128, True, False),
    "decode": Workload("decode", 64, 32, 8, 1, 32768, 128, False, False, decode=True, num_splits=16),
}


def _gen(seed: int, tag: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + tag) & 0x7FFFFFFFFFFFFFFF)
    return g


def _randn(shape, seed, tag, device) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(seed, tag, device), device=device, dtype=torch.float32)


def make_inputs(w: Workload, seed: int = 0, device="cuda", S_override: Optional[int] = None,
                B_override: Optional[int] = None) -> Dict[str, object]:
    """Draw q [B,Hq,S_q,D], k, v [B,Hkv,S_kv,D] as bf16 on `device` for workload w.

    S_override shrinks the sequence (same recipe) for quick tests; B_override
    shrinks the decode batch.  Returns the tensors and the drawn indices.
    """
    B = B_override or w.B
    S_kv = S_override or w.S_kv
    S_q = 1 if w.decode else (S_override or w.S_q)
    meta: Dict[str, object] = {}
    q = _randn((B, w.Hq, S_q, w.D), seed, 1, device)
    v_tag, k_tag = 3, 2
    if w.name == "llama16k":
        g = _gen(seed, 10, "cpu")
        kc = torch.randperm(w.D, generator=g)[:4].sort().values
        qc = torch.randperm(w.D, generator=g)[:2].sort().values
        meta["k_outlier_channels"] = kc.tolist()
        meta["q_outlier_channels"] = qc.tolist()
        q[..., qc.to(device)] *= 20.0
    k = torch.empty((B, w.Hkv, S_kv, w.D), dtype=torch.bfloat16, device=device)
    v = torch.empty((B, w.Hkv, S_kv, w.D), dtype=torch.bfloat16, device=device)
    for b in range(B):  # per sequence: bounded peak memory for the decode cache
        kb = _randn((w.Hkv, S_kv, w.D), seed, 1000 * b + k_tag, device)
        if w.name == "llama16k":
            kb[..., torch.tensor(meta["k_outlier_channels"], device=device)] *= 20.0
        elif w.name == "qwen32k":
            off = _randn((w.Hkv, 1, w.D), seed, 11, device) * 3.0
            kb += off
        elif w.name == "long128k":
            n_out = int(math.floor(0.01 * S_kv))
            g = _gen(seed, 12, "cpu")
            rows = torch.stack([torch.randperm(S_kv, generator=g)[:n_out] for _ in range(w.Hkv)])
            meta.setdefault("k_outlier_rows_per_head", n_out)
            for hh in range(w.Hkv):
                kb[hh, rows[hh].to(device)] *= 8.0
        k[b] = kb.to(torch.bfloat16)
        del kb
        v[b] = _randn((w.Hkv, S_kv, w.D), seed, 1000 * b + v_tag, device).to(torch.bfloat16)
    return {"q": q.to(torch.bfloat16), "k": k, "v": v, "meta": meta, "B": B, "S_q": S_q, "S_kv": S_kv}


def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns on the host (for the oracle)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")
