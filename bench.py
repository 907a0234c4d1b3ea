#!/usr/bin/env python3
"""Benchmark of the QK4PV8 attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long128k]
                    [--no-cpu-baseline] [--no-configs] [--no-variants] [--no-parity]
                    [--only all|prefill|decode|copy|stream]

Headline step (`value`): the whole prefill hot path over the long-context
workload (B1, Hq32/Hkv8, S131072, D128, causal; 1% of K rows x8; bf16 inputs
resident in HBM): quantise K to MXFP4 and V to FP8, then the prefill kernel,
which quantises Q to MXFP4 itself (q4 = NULL: the same codes as the quantiser
pass).  `value` is algorithmic TFLOP/s of the whole step (4 D FLOPs per
visible query/key pair; masked pairs not counted).  The roofline object is
the prefill kernel's, timed with HIP events on the stream it is launched on,
against the blended MXFP4 (Q K^T) / FP8 (P V) MFMA peak.

`configs` holds one record per workload -- tiny, llama16k, qwen32k (rank-one
compensation on, and the same inputs with it off), long128k, decode -- each
with its kernel time, roofline fraction, parity against the CPU oracle on
sampled rows (O max-abs and relative L2, LSE max-abs) and the error of the
GPU output against exact FP64 attention on the same rows (relative L2,
cosine; reported, not bounded).  The decode half of the metric (B64 x 32768
cached keys, 16 KV splits + LSE merge) is also reported under `decode` in
GB/s.  `variants` times the contrast formats (FP8 P with a scale per (row, 32
keys); MXFP4 P and V; NVFP4 Q and K) on llama16k and the decode workload.

`cpu_baseline` is the oracle (plain C, binary64) built with -march=native on
this host and timed on a bounded sample of the headline workload's rows,
with the CPU model, the thread count and the full-workload time
extrapolated by visible-pair count.

`--only prefill|decode` runs just that half (for hardware-counter passes);
`--only copy` a plain 1 GiB device copy (the calibration kernel of the
FETCH_SIZE / WRITE_SIZE counters); `--only stream` a 4 GiB row-wise device
sum (the read-bandwidth ceiling quoted beside the decode).
"""
import argparse
import hashlib
import json
import os
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QK4PV8 fwd prefill TFLOP/s + decode KV GB/s on 1×MI355X; % roofline"
COPY_BYTES = 1 << 30
STREAM_BYTES = 4 << 30
CPU_TARGET_S = 15.0
PARITY_ROWS = {"tiny": None, "llama16k": 384, "qwen32k": 320, "long128k": 256}
DATA = {
    "tiny": "seeded synthetic bf16 Q/K/V ~ N(0,1) (no weights or datasets)",
    "llama16k": "seeded synthetic bf16 ~ N(0,1) shaped like Llama-3.1-8B attention; 4 of 128 K channels and 2 of "
                "128 Q channels x20 (no weights or datasets)",
    "qwen32k": "seeded synthetic bf16 ~ N(0,1) shaped like Qwen3-14B attention; K with a per-(kv head, channel) "
               "offset ~ N(0, 3^2) (no weights or datasets)",
    "long128k": "seeded synthetic bf16 ~ N(0,1) at 128K context; 1% of K rows per kv head x8 (no weights or "
                "datasets)",
    "decode": "seeded synthetic bf16 ~ N(0,1); KV cache quantised once, untimed (no weights or datasets)",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # 100 untimed steps bring the clocks to steady state (after 10 the prefill
    # kernel still ran 5-6% slower)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="long128k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-variants", action="store_true")
    p.add_argument("--no-configs", action="store_true")
    p.add_argument("--no-parity", action="store_true")
    p.add_argument("--only", default="all", choices=("all", "prefill", "decode", "copy", "stream"))
    return p.parse_args()


def log(*a):
    print("[bench %s]" % time.strftime("%H:%M:%S"), *a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- reference kernels
def _timed_torch(fn, warmup, steps):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def stream_read_gbs(warmup=20, steps=50):
    """GB/s of a row-wise sum over 4 GiB (rows of 16 KB, a 1 MiB result): the
    device read bandwidth a streaming kernel can approach (a full reduction
    to one scalar reads at only about 4 TB/s, so it would understate this)."""
    import torch
    x = torch.ones(STREAM_BYTES // 4, dtype=torch.float32, device="cuda:0").view(-1, 4096)
    ms = _timed_torch(lambda: x.sum(dim=1), warmup, steps)
    del x
    return STREAM_BYTES / (ms * 1e-3) / 1e9


def run_stream(args):
    gbs = stream_read_gbs(args.warmup, args.steps)
    print(json.dumps({"stream_bytes_read": STREAM_BYTES, "GB/s": round(gbs, 1)}), flush=True)


def run_copy(args):
    """A plain 1 GiB device copy; its counter readings calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ms = _timed_torch(lambda: dst.copy_(src), args.warmup, args.steps)
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "ms": round(ms, 4),
                      "GB/s": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1)}), flush=True)


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_quantized_attention_qk4pv8_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(name, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("source_hash") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------- parity on sampled rows
def _errors(Og, lg, res):
    import numpy as np
    d = np.abs(Og - res["O_q"])
    den = np.linalg.norm(res["O_q"])
    fin = np.isfinite(res["lse_q"]) & np.isfinite(lg)
    out = {"rows": int(Og.shape[0]),
           "O_max_abs": float(d.max()) if d.size else 0.0,
           "O_rel_l2": float(np.linalg.norm(Og - res["O_q"]) / den) if den > 0 else 0.0,
           "lse_max_abs": float(np.abs(lg[fin] - res["lse_q"][fin]).max()) if fin.any() else 0.0}
    out["pass"] = bool(out["O_max_abs"] <= 3e-3 and out["O_rel_l2"] <= 1e-3 and out["lse_max_abs"] <= 1e-3
                       and np.isfinite(Og).all())
    ok = np.isfinite(res["lse_x"])
    ex, g = res["O_x"][ok], Og[ok]
    vs = {"rel_l2": float(np.linalg.norm(g - ex) / np.linalg.norm(ex)),
          "cosine": float(np.sum(g * ex) / (np.linalg.norm(g) * np.linalg.norm(ex)))}
    return out, vs


def prefill_parity(w, inp, O, lse, nrows, seed=1):
    import numpy as np
    import torch
    import oracle
    from bit_quantized_attention_qk4pv8_amd.workloads import bf16_bits
    B, Hq, S = w.B, w.Hq, w.S_q
    if nrows is None:
        rows = np.array([(b, h, i) for b in range(B) for h in range(Hq) for i in range(S)], dtype=np.int64)
    else:
        rng = np.random.default_rng(seed)
        must = {(0, h, i) for h in range(Hq) for i in (0, 127, 128, S - 1)}
        rows = set(must)
        while len(rows) < nrows:
            rows.add((0, int(rng.integers(Hq)), int(rng.integers(S))))
        rows = np.array(sorted(rows), dtype=np.int64)
    idx = [torch.from_numpy(rows[:, c]).to(O.device) for c in range(3)]
    Og = O[idx[0], idx[1], idx[2]].double().cpu().numpy()
    lg = lse[idx[0], idx[1], idx[2]].double().cpu().numpy()
    res = oracle.prefill_rows(bf16_bits(inp["q"]), bf16_bits(inp["k"]), bf16_bits(inp["v"]), rows, w.causal,
                              w.scale, smooth=w.smooth, exact=True)
    return _errors(Og, lg, res)


# ----------------------------------------------------------------------------- prefill
def run_prefill(w, args, dev, stream, smooth=None, inp=None, parity=True, step_mode=True):
    """Time the prefill path of workload w (compensation per w unless smooth is
    given).  step_mode: each step quantises K and V, then runs the prefill with
    Q quantised in the kernel; otherwise K/V are quantised once and only the
    prefill kernel is timed.  Returns (record, inputs)."""
    import numpy as np
    import torch
    import bit_quantized_attention_qk4pv8_amd as qfa
    from bit_quantized_attention_qk4pv8_amd import roofline as rl
    from bit_quantized_attention_qk4pv8_amd.workloads import make_inputs
    smooth = w.smooth if smooth is None else smooth
    if inp is None:
        inp = make_inputs(w, seed=0, device=dev)
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, Hq, Hkv, S, D = w.B, w.Hq, w.Hkv, w.S_q, w.D
    nt = (S + 127) // 128
    k4 = torch.empty((B, Hkv, S, D // 2), dtype=torch.uint8, device=dev)
    k4s = torch.empty((B, Hkv, S, D // 32), dtype=torch.uint8, device=dev)
    kbar = torch.empty((B, Hkv, nt, D), dtype=torch.bfloat16, device=dev) if smooth else None
    v8 = torch.empty((B, Hkv, (S + 31) // 32, D, 32), dtype=torch.uint8, device=dev)
    v8s = torch.empty((B, Hkv, (S + 31) // 32, D), dtype=torch.uint8, device=dev)
    O = torch.empty((B, Hq, S, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def quant_kv():
        qfa.qfa_quantize_qk4(k, B, Hkv, S, D, 32, int(smooth), 1.0, k4, k4s, kbar, stream)
        qfa.qfa_quantize_v8(v, B, Hkv, S, D, 32, v8, v8s, stream)

    def step(i=None):
        if step_mode:
            quant_kv()
        if i is not None:
            ev[i][0].record(stream)
        qfa.qfa_fwd_prefill(None, None, k4, k4s, kbar, q, v8, v8s, B, Hq, Hkv, S, S, D, int(w.causal), w.scale, 32,
                            O, lse, stream)
        if i is not None:
            ev[i][1].record(stream)

    if not step_mode:
        quant_kv()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    flops = w.flops()
    comp = w.comp_flops() if smooth else 0.0
    achieved = (flops + comp) / (kern_ms * 1e-3) / 1e12
    peak = rl.blended_peak(flops, comp) / 1e12
    rec = {
        "shape": {"B": B, "Hq": Hq, "Hkv": Hkv, "S_q": S, "S_kv": S, "D": D, "causal": w.causal,
                  "compensation": bool(smooth)},
        "data": DATA[w.name],
        "kernel": "qfa::k_prefill<%d,%s,0>" % (D, "true" if smooth else "false"),
        "kernel_ms": round(kern_ms, 4),
        "ms_per_step" if step_mode else "ms_per_launch": round(ms_step, 4),
        "algorithmic_flop_per_launch": flops + comp,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 2), "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4)},
    }
    if step_mode:
        rec["step"] = "quantise K (MXFP4%s) + V (FP8), then the prefill kernel with Q quantised in-kernel" % (
            ", with K-mean smoothing" if smooth else "")
        rec["step_TFLOP/s"] = round(flops / (ms_step * 1e-3) / 1e12, 2)
    if parity and not args.no_parity:
        tp = time.perf_counter()
        wp = w if smooth == w.smooth else _with_smooth(w, smooth)
        par, vs = prefill_parity(wp, inp, O, lse, PARITY_ROWS.get(w.name))
        rec["parity"] = dict(par, bar={"O_max_abs": 3e-3, "O_rel_l2": 1e-3, "lse_max_abs": 1e-3})
        rec["vs_exact_fp64"] = vs
        log("%s parity %s vs-exact %s (%.1f s)" % (w.name, par, vs, time.perf_counter() - tp))
    del O, lse, k4, k4s, kbar, v8, v8s
    return rec, inp


def _with_smooth(w, smooth):
    import dataclasses
    return dataclasses.replace(w, smooth=smooth)


def run_prefill_variants(w, args, dev, stream, inp):
    """The contrast formats on workload w, prefill kernels only (inputs quantised once)."""
    import numpy as np
    import torch
    import bit_quantized_attention_qk4pv8_amd as qfa
    from bit_quantized_attention_qk4pv8_amd import roofline as rl
    q, k, v = inp["q"], inp["k"], inp["v"]
    B, Hq, Hkv, S, D = w.B, w.Hq, w.Hkv, w.S_q, w.D
    O = torch.empty((B, Hq, S, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    flops, comp = w.flops(), w.comp_flops()
    out = {}

    def time_it(launch):
        vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i in range(args.warmup + args.steps):
            j = i - args.warmup
            if j >= 0:
                vev[j][0].record(stream)
            launch()
            if j >= 0:
                vev[j][1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in vev]))

    k4, k4s, kbar = qfa.quantize_qk4(k, smooth=w.smooth)
    for name, pv in (("qk4pv8_blockp", qfa.QFA_PV_FP8_BLOCKP), ("qk4pv4", qfa.QFA_PV_FP4)):
        fp4 = pv == qfa.QFA_PV_FP4
        vq, vqs = qfa.quantize_v4(v) if fp4 else qfa.quantize_v8(v)
        vk = time_it(lambda: qfa.qfa_fwd_prefill_ex(None, None, k4, k4s, kbar, q, vq, vqs, B, Hq, Hkv, S, S, D,
                                                     int(w.causal), w.scale, 32, pv, O, lse, stream))
        vach = (flops + comp) / (vk * 1e-3) / 1e12
        vpeak = rl.blended_peak(flops, comp, pv_fp4=fp4) / 1e12
        out[name] = {"prefill": {"workload": w.name, "kernel_ms": round(vk, 4), "achieved": round(vach, 2),
                                 "peak": round(vpeak, 2), "unit": "TFLOP/s", "frac": round(vach / vpeak, 4),
                                 "kernel": "qfa::k_prefill<%d,%s,%d>" % (D, "true" if w.smooth else "false", pv)}}
        del vq, vqs
    # NVFP4 Q and K (emulated on the bf16 MFMA), P and V as in the method
    c2 = qfa.qfa_exp2_scale(w.scale)
    gq = qfa.nvfp4_tensor_scale(float((q.float() * c2).abs().max()))
    gk = qfa.nvfp4_tensor_scale(float(k.float().abs().max()))
    q4n, q4ns, _ = qfa.quantize_nvfp4(q, gq, prescale=c2)
    k4n, k4ns, kbn = qfa.quantize_nvfp4(k, gk, smooth=w.smooth)
    v8, v8s = qfa.quantize_v8(v)
    vk = time_it(lambda: qfa.qfa_fwd_prefill_nvfp4(q4n, q4ns, k4n, k4ns, kbn, q if w.smooth else None, v8, v8s, B, Hq,
                                                   Hkv, S, S, D, int(w.causal), w.scale, gq, gk, O, lse, stream))
    vach = (flops + comp) / (vk * 1e-3) / 1e12
    vpeak = rl.blended_peak(flops, comp, qk_bf16=True) / 1e12
    out["nvfp4_qk"] = {"prefill": {"workload": w.name, "kernel_ms": round(vk, 4), "achieved": round(vach, 2),
                                   "peak": round(vpeak, 2), "unit": "TFLOP/s", "frac": round(vach / vpeak, 4),
                                   "kernel": "qfa::k_prefill<%d,%s,3>" % (D, "true" if w.smooth else "false"),
                                   "note": "Q K^T emulated on the bf16 MFMA; peak counts it at bf16"}}
    return out


# ----------------------------------------------------------------------------- decode
def run_decode(args, dev, stream, src, variants):
    import numpy as np
    import torch
    import bit_quantized_attention_qk4pv8_amd as qfa
    import oracle
    from bit_quantized_attention_qk4pv8_amd import roofline as rl
    from bit_quantized_attention_qk4pv8_amd.workloads import WORKLOADS, bf16_bits, make_inputs
    wd = WORKLOADS["decode"]
    di = make_inputs(wd, seed=0, device=dev)
    Bd, Hqd, Hkvd, L, Dd = di["B"], wd.Hq, wd.Hkv, wd.S_kv, wd.D
    k4d, k4sd, _ = qfa.quantize_qk4(di["k"])
    v8d, v8sd = qfa.quantize_v8(di["v"])
    qd = di["q"]
    splits = wd.num_splits
    wsb = qfa.qfa_decode_workspace_bytes(Bd, Hqd, Dd, splits)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    Od = torch.empty((Bd, Hqd, Dd), dtype=torch.float32, device=dev)
    lsed = torch.empty((Bd, Hqd), dtype=torch.float32, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def dstep(i=None):
        if i is not None:
            ev[i][0].record(stream)
        qfa.qfa_fwd_decode(None, None, k4d, k4sd, None, qd, v8d, v8sd, Bd, Hqd, Hkvd, L, None, Dd, wd.scale,
                           32, splits, ws, wsb, Od, lsed, stream)
        if i is not None:
            ev[i][1].record(stream)

    torch.cuda.synchronize()
    for _ in range(args.warmup):
        dstep()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        dstep(i)
    torch.cuda.synchronize()
    d_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    d_kern = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    dbytes = rl.decode_algorithmic_bytes(Bd, Hqd, Hkvd, L, Dd)
    gbs = dbytes / (d_kern * 1e-3) / 1e9
    rec = {
        "metric": "decode KV GB/s", "value": round(gbs, 1), "unit": "GB/s",
        "ms_per_step": round(d_ms, 4), "kernel_ms": round(d_kern, 4), "data": DATA["decode"],
        "shape": {"B": Bd, "Hq": Hqd, "Hkv": Hkvd, "S_kv": L, "D": Dd, "num_splits": splits},
        "kernel": "qfa::k_decode_split<128,false,0> + k_decode_merge<128>",
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": rl.PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(gbs * 1e9 / rl.PEAK_HBM, 4),
                     "traffic": traffic_from_profile("decode_b64_traffic.json", src)},
        "algorithmic_bytes_per_launch": dbytes,
    }
    if not args.no_parity:
        seqs = [0, 21, 42, 63]
        rows = np.array([(b, h, 0) for b in seqs for h in range(Hqd)], dtype=np.int64)
        Og = Od.double().cpu().numpy()[rows[:, 0], rows[:, 1]]
        lg = lsed.double().cpu().numpy()[rows[:, 0], rows[:, 1]]
        qb = bf16_bits(qd)
        kb = bf16_bits(di["k"][seqs])
        vb = bf16_bits(di["v"][seqs])
        rloc = rows.copy()
        rloc[:, 0] = np.repeat(np.arange(len(seqs)), Hqd)
        res = oracle.decode_rows(qb[seqs], kb, vb, rloc, wd.scale, splits, exact=True)
        par, vs = _errors(Og, lg, res)
        rec["parity"] = dict(par, bar={"O_max_abs": 3e-3, "O_rel_l2": 1e-3, "lse_max_abs": 1e-3},
                             sample="4 whole sequences (all 32 heads), sequences %s" % seqs)
        rec["vs_exact_fp64"] = vs
        log("decode parity %s vs-exact %s" % (par, vs))
    ceil_gbs = stream_read_gbs()
    rec["stream_read_ceiling"] = {"GB/s": round(ceil_gbs, 1), "frac": round(gbs / ceil_gbs, 4),
                                  "kernel": "row-wise sum of 4 GiB (torch)"}
    var = {}
    if variants:
        vd = di["v"]
        for name, pv in (("qk4pv8_blockp", qfa.QFA_PV_FP8_BLOCKP), ("qk4pv4", qfa.QFA_PV_FP4)):
            fp4 = pv == qfa.QFA_PV_FP4
            del v8d, v8sd
            v8d, v8sd = qfa.quantize_v4(vd) if fp4 else qfa.quantize_v8(vd)
            vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            for i in range(args.warmup + args.steps):
                j = i - args.warmup
                if j >= 0:
                    vev[j][0].record(stream)
                qfa.qfa_fwd_decode_ex(None, None, k4d, k4sd, None, qd, v8d, v8sd, Bd, Hqd, Hkvd, L, None, Dd,
                                      wd.scale, 32, pv, splits, ws, wsb, Od, lsed, stream)
                if j >= 0:
                    vev[j][1].record(stream)
            torch.cuda.synchronize()
            vk = float(np.mean([a.elapsed_time(b) for a, b in vev]))
            vb_ = rl.decode_algorithmic_bytes(Bd, Hqd, Hkvd, L, Dd, v_fp4=fp4)
            vg = vb_ / (vk * 1e-3) / 1e9
            var[name] = {"kernel_ms": round(vk, 4), "achieved": round(vg, 1), "peak": rl.PEAK_HBM / 1e9,
                         "unit": "GB/s", "frac": round(vg * 1e9 / rl.PEAK_HBM, 4),
                         "algorithmic_bytes_per_launch": vb_}
        c2 = qfa.qfa_exp2_scale(wd.scale)
        gq = qfa.nvfp4_tensor_scale(float((qd.float() * c2).abs().max()))
        gk = qfa.nvfp4_tensor_scale(float(di["k"].float().abs().max()))
        q4n, q4ns, _ = qfa.quantize_nvfp4(qd, gq, prescale=c2)
        k4n, k4ns, _ = qfa.quantize_nvfp4(di["k"], gk)
        del v8d, v8sd
        v8d, v8sd = qfa.quantize_v8(vd)
        vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i in range(args.warmup + args.steps):
            j = i - args.warmup
            if j >= 0:
                vev[j][0].record(stream)
            qfa.qfa_fwd_decode_nvfp4(q4n, q4ns, k4n, k4ns, None, None, v8d, v8sd, Bd, Hqd, Hkvd, L, None, Dd,
                                     wd.scale, gq, gk, splits, ws, wsb, Od, lsed, stream)
            if j >= 0:
                vev[j][1].record(stream)
        torch.cuda.synchronize()
        vk = float(np.mean([a.elapsed_time(b) for a, b in vev]))
        vb_ = rl.decode_algorithmic_bytes(Bd, Hqd, Hkvd, L, Dd, k_nvfp4=True)
        vg = vb_ / (vk * 1e-3) / 1e9
        var["nvfp4_qk"] = {"kernel_ms": round(vk, 4), "achieved": round(vg, 1), "peak": rl.PEAK_HBM / 1e9,
                           "unit": "GB/s", "frac": round(vg * 1e9 / rl.PEAK_HBM, 4),
                           "algorithmic_bytes_per_launch": vb_}
    return rec, var


# ----------------------------------------------------------------------------- CPU baseline (oracle)
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_cpu_baseline(w, inp):
    """The oracle timed on this host: its quantisers over the workload's full
    Q, K and V tensors, then its attention (c) over a seeded sample of rows
    on those codes, grown until one call lasts about CPU_TARGET_S / 2 or more.
    The full-workload time is extrapolated as quantisers + attention x
    (visible pairs of the workload / visible pairs of the sample)."""
    import numpy as np
    import oracle
    from bit_quantized_attention_qk4pv8_amd.workloads import bf16_bits
    build = "-O3 -march=native (built on this host)"
    try:
        path = os.path.join(tempfile.gettempdir(), "liboracle_native_%d.so" % os.getpid())
        oracle.build(out=path, march="native")
        oracle.use_library(path)
    except Exception as e:  # the shipped portable build still measures the oracle
        build = "-O3 -march=x86-64-v3 (native build failed: %s)" % e
    qb, kb, vb = bf16_bits(inp["q"]), bf16_bits(inp["k"]), bf16_bits(inp["v"])
    Hq, S, D = w.Hq, w.S_q, w.D
    tq0 = time.perf_counter()
    q4, q4s, _ = oracle.quantize_qk4(qb, prescale=oracle.exp2_scale(w.scale))
    k4, k4s, kbar = oracle.quantize_qk4(kb, smooth=w.smooth)
    v8, v8s = oracle.quantize_v8(vb)
    tq = time.perf_counter() - tq0
    rng = np.random.default_rng(0)

    def sample(n_rows):
        must = [(0, h, i) for h in range(Hq) for i in (0, 127, 128, S - 1)]
        rows = np.concatenate([np.array(must, np.int64),
                               np.stack([np.zeros(n_rows, np.int64), rng.integers(0, Hq, n_rows),
                                         rng.integers(0, S, n_rows)], axis=1)])
        tc0 = time.perf_counter()
        oracle.prefill_rows_from_codes(q4, q4s, k4, k4s, v8, v8s, rows, w.causal, w.scale,
                                       q_bits=qb if w.smooth else None, kbar_bits=kbar)
        dt = time.perf_counter() - tc0
        pairs = int(sum((r[2] + 1) if w.causal else S for r in rows))
        return dt, pairs, len(rows)

    n_rows = 2048
    while True:
        dt, pairs, nr = sample(n_rows)
        if dt >= CPU_TARGET_S / 2 or n_rows >= S * Hq // 4:
            break
        n_rows = int(min(S * Hq // 4, n_rows * min(16.0, CPU_TARGET_S / max(dt, 1e-3))))
    total_pairs = w.pairs()
    qbytes = 2 * (qb.size + kb.size + vb.size)
    return {"value": round(4.0 * D * pairs / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(), "build": build,
            "sample": "attention (c) on %d seeded query rows of %s (rows 0, 127, 128 and the last of every head "
                      "among them): %d visible query/key pairs in %.1f s, on codes from the oracle's quantisers "
                      "(full Q, K, V: %.1f s, %.2f GB/s of bf16 input)"
                      % (nr, w.name, pairs, dt, tq, qbytes / tq / 1e9),
            "attention_s": round(dt, 2), "quantisers_s": round(tq, 2),
            "extrapolated_full_workload_s": round(tq + dt * total_pairs / pairs, 1),
            "extrapolation": "quantisers %.1f s + attention %.2f s x (workload pairs %d / sampled pairs %d)"
                             % (tq, dt, total_pairs, pairs)}


# ----------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(each GPU would run its own shard with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.only == "copy":
        run_copy(args)
        return
    if args.only == "stream":
        run_stream(args)
        return

    import torch

    from bit_quantized_attention_qk4pv8_amd.workloads import WORKLOADS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    src = source_hash()
    w = WORKLOADS[args.workload]
    out = {}
    head_inp = None
    if args.only in ("all", "prefill"):
        log("headline prefill step", w.name)
        rec, head_inp = run_prefill(w, args, dev, stream, parity=args.only == "all")
        rec["roofline"]["traffic"] = traffic_from_profile("prefill_%s_traffic.json" % w.name, src)
        rec["roofline"]["kernel"] = rec["kernel"]
        rec["roofline"]["kernel_ms"] = rec["kernel_ms"]
        rec["roofline"]["algorithmic_flop_per_launch"] = rec["algorithmic_flop_per_launch"]
        out.update({
            "metric": METRIC,
            "value": rec["step_TFLOP/s"],
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": rec["ms_per_step"],
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "mxfp4(QK)+fp8(PV), fp32 accumulate",
            "data": DATA[w.name],
            "config": dict({"workload": w.name}, **rec["shape"], step=rec["step"]),
            "roofline": rec["roofline"],
        })
        out["configs"] = {w.name: rec}
    if args.only == "all" and not args.no_configs:
        for name in ("tiny", "llama16k", "qwen32k", "long128k"):
            if name == w.name:
                continue
            log("config", name)
            wc = WORKLOADS[name]
            rec, inp = run_prefill(wc, args, dev, stream, step_mode=False)
            rec["roofline"]["traffic"] = traffic_from_profile("prefill_%s_traffic.json" % name, src)
            if wc.smooth:
                log("config", name, "compensation off")
                off, _ = run_prefill(wc, args, dev, stream, smooth=False, inp=inp, step_mode=False)
                rec["compensation_off"] = off
                rec["compensation_overhead"] = round(rec["kernel_ms"] / off["kernel_ms"] - 1.0, 4)
            out["configs"][name] = rec
            if name == "llama16k" and not args.no_variants:
                log("variants on", name)
                out["variants"] = run_prefill_variants(wc, args, dev, stream, inp)
            del inp
            torch.cuda.empty_cache()
    if args.only in ("all", "decode") and not args.no_decode:
        log("decode")
        drec, dvar = run_decode(args, dev, stream, src, variants=args.only == "all" and not args.no_variants)
        out["decode"] = drec
        out.setdefault("configs", {})["decode"] = drec
        for name, v in dvar.items():
            out.setdefault("variants", {}).setdefault(name, {})["decode"] = v
    if args.only == "all" and not args.no_cpu_baseline and head_inp is not None:
        log("cpu baseline")
        out["cpu_baseline"] = run_cpu_baseline(w, head_inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
