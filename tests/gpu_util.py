"""Shared helpers of the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import bit_quantized_attention_qk4pv8_amd as qfa
import oracle
from bit_quantized_attention_qk4pv8_amd.workloads import bf16_bits

# Parity bar for O against oracle (c), and for LSE
O_MAX_ABS = 3e-3
O_REL_L2 = 1e-3
LSE_MAX_ABS = 1e-3


def say(*args):
    """Progress line, flushed before the GPU step it names."""
    print("[gpu-test %s]" % time.strftime("%H:%M:%S"), *args, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bf16_from_f32(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def compare_o(O_gpu: np.ndarray, O_orc: np.ndarray, lse_gpu=None, lse_orc=None, label=""):
    O_gpu = np.asarray(O_gpu, np.float64)
    diff = np.abs(O_gpu - O_orc)
    max_abs = float(diff.max()) if diff.size else 0.0
    den = float(np.linalg.norm(O_orc))
    rel = float(np.linalg.norm(O_gpu - O_orc) / den) if den > 0 else float(np.linalg.norm(O_gpu))
    say("%s O max-abs %.3e rel-L2 %.3e (bar %.0e / %.0e)" % (label, max_abs, rel, O_MAX_ABS, O_REL_L2))
    assert np.isfinite(O_gpu).all(), "non-finite O"
    assert max_abs <= O_MAX_ABS, (label, max_abs)
    assert rel <= O_REL_L2, (label, rel)
    if lse_gpu is not None:
        lg = np.asarray(lse_gpu, np.float64)
        both_inf = np.isneginf(lg) & np.isneginf(lse_orc)
        assert (np.isneginf(lg) == np.isneginf(lse_orc)).all(), "LSE -inf pattern differs"
        d = np.abs(np.where(both_inf, 0.0, lg - np.where(both_inf, 0.0, lse_orc)))
        say("%s LSE max-abs %.3e" % (label, float(d.max()) if d.size else 0.0))
        assert d.max() <= LSE_MAX_ABS if d.size else True
    return max_abs, rel


def sample_rows(B, H, S, n, seed, must=(0, 127, 128)):
    """Seeded sample of (b, h, i) rows including fixed positions and the last row."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(B):
        for h in range(H):
            for i in list(must) + [S - 1]:
                if 0 <= i < S:
                    rows.add((b, h, i))
    while len(rows) < min(n, B * H * S):
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(S))))
    return np.array(sorted(rows), dtype=np.int64)
