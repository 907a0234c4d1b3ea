#!/usr/bin/env python3
"""Benchmark of the QK4PV8 attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--only all|prefill|decode|copy|stream]

One step = the whole prefill hot path over the Llama-3.1-8B-shaped workload
(B1, Hq32/Hkv8, S16384, D128, causal; bf16 inputs resident in HBM): quantise K
to MXFP4 and V to FP8, then run the prefill kernel, which quantises Q to MXFP4
itself (q4 = NULL: the same codes as the quantiser pass).  `value` is
algorithmic TFLOP/s of the whole step (4 D FLOPs per visible query/key pair;
masked pairs not counted).  The decode half of the metric (B64 sequences x
32768 cached keys, Hq32/Hkv8, 16 KV splits + LSE merge, cache pre-quantised,
Q quantised inside the split kernel) is timed in the same run and reported under "decode" as KV GB/s.

The roofline object is for the dominant kernel (the prefill kernel), timed
with HIP events on the stream it is launched on; its peak is the blended
MXFP4 (Q K^T) / FP8 (P V) MFMA peak.  The CPU baseline is the oracle timed on
a bounded sample of rows of the same workload on this host (about 15 s).

The contrast formats (FP8 P with a scale per (row, 32 keys); MXFP4 P and V;
NVFP4 Q and K) are timed on the same workloads, kernels only, and reported
under "variants" with their own roofline fractions (the MXFP4 prefill against
the all-MXFP4 MFMA peak, the NVFP4 one with Q K^T at the bf16 peak it is
emulated on, each decode against its own cache bytes).

`--only prefill|decode` runs just that half (for hardware-counter passes);
`--only copy` runs a plain device-to-device copy of 1 GiB, the reference
kernel of known size that scales the FETCH_SIZE / WRITE_SIZE counters into
bytes; `--only stream` times a 4 GiB row-wise device sum, the read-bandwidth
ceiling quoted beside the decode.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # 100 untimed steps (about 0.1 s of GPU work per half) bring the clocks to
    # steady state: after 10 the prefill kernel still ran 5-6% slower
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-variants", action="store_true")
    p.add_argument("--workload", default="llama16k")
    p.add_argument("--only", default="all", choices=("all", "prefill", "decode", "copy", "stream"))
    return p.parse_args()


COPY_BYTES = 1 << 30
CPU_TARGET_S = 15.0
MAX_CPU_ROWS = 131072  # bounded CPU sample: at most a quarter of llama16k's 524288 rows


STREAM_BYTES = 4 << 30


def stream_read_gbs(warmup=20, steps=50):
    """GB/s of the row-wise 4 GiB sum (see run_stream)."""
    import torch
    x = torch.ones(STREAM_BYTES // 4, dtype=torch.float32, device="cuda:0").view(-1, 4096)
    for _ in range(warmup):
        x.sum(dim=1)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        x.sum(dim=1)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    del x
    return STREAM_BYTES / (ms * 1e-3) / 1e9


def run_stream(args):
    """Device read bandwidth: 4 GiB reduced row by row (rows of 16 KB, a 1 MiB
    result), timed like the attention kernels.  The ceiling that a streaming
    kernel such as the split-KV decode can approach (reported beside the
    decode's fraction of the 8 TB/s peak, not graded).  A full reduction to
    one scalar reads at only about 4 TB/s, so it would understate this."""
    import torch
    x = torch.ones(STREAM_BYTES // 4, dtype=torch.float32, device="cuda:0").view(-1, 4096)
    for _ in range(args.warmup):
        x.sum(dim=1)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        x.sum(dim=1)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"stream_bytes_read": STREAM_BYTES, "ms": round(ms, 4),
                      "GB/s": round(STREAM_BYTES / (ms * 1e-3) / 1e9, 1)}), flush=True)


def run_copy(args):
    """A plain 1 GiB device copy, timed like the attention kernels; its counter
    readings calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "ms": round(ms, 4),
                      "GB/s": round(2 * COPY_BYTES / (ms * 1e-3) / 1e9, 1)}), flush=True)


def source_hash():
    h = hashlib.sha256()
    for f in ("attn.hip", "prefill.hip", "attn_common.h", "quant.hip", "api.hip", "qfa_internal.h"):
        with open(os.path.join(ROOT, "bit_quantized_attention_qk4pv8_amd", "csrc", f), "rb") as fh:
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

    import numpy as np
    import torch

    import bit_quantized_attention_qk4pv8_amd as qfa
    from bit_quantized_attention_qk4pv8_amd import roofline as rl
    from bit_quantized_attention_qk4pv8_amd.workloads import WORKLOADS, bf16_bits, make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    out = {}
    src = source_hash()
    stream = torch.cuda.current_stream()
    if args.only in ("all", "prefill"):
        inp = make_inputs(w, seed=0, device=dev)
        q, k, v = inp["q"], inp["k"], inp["v"]
        B, Hq, Hkv, S, D = w.B, w.Hq, w.Hkv, w.S_q, w.D
        nt = (S + 127) // 128
        k4 = torch.empty((B, Hkv, S, D // 2), dtype=torch.uint8, device=dev)
        k4s = torch.empty((B, Hkv, S, D // 32), dtype=torch.uint8, device=dev)
        kbar = torch.empty((B, Hkv, nt, D), dtype=torch.bfloat16, device=dev) if w.smooth else None
        v8 = torch.empty((B, Hkv, (S + 31) // 32, D, 32), dtype=torch.uint8, device=dev)
        v8s = torch.empty((B, Hkv, (S + 31) // 32, D), dtype=torch.uint8, device=dev)
        O = torch.empty((B, Hq, S, D), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

        def step(i=None):
            qfa.qfa_quantize_qk4(k, B, Hkv, S, D, 32, int(w.smooth), 1.0, k4, k4s, kbar, stream)
            qfa.qfa_quantize_v8(v, B, Hkv, S, D, 32, v8, v8s, stream)
            if i is not None:
                ev[i][0].record(stream)
            qfa.qfa_fwd_prefill(None, None, k4, k4s, kbar, q, v8, v8s, B, Hq, Hkv, S, S, D,
                                int(w.causal), w.scale, 32, O, lse, stream)
            if i is not None:
                ev[i][1].record(stream)

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
        comp = w.comp_flops()
        value = flops / (ms_step * 1e-3) / 1e12
        achieved = (flops + comp) / (kern_ms * 1e-3) / 1e12
        peak = rl.blended_peak(flops, comp) / 1e12
        traffic = traffic_from_profile("prefill_%s_traffic.json" % w.name, src)
        out.update({
            "metric": "QK4PV8 fwd prefill TFLOP/s + decode KV GB/s on 1\u00d7MI355X; % roofline",
            "value": round(value, 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(ms_step, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "mxfp4(QK)+fp8(PV), fp32 accumulate",
            "data": "synthetic seeded bf16 inputs shaped like Llama-3.1-8B attention (no weights/datasets)",
            "config": {"workload": w.name, "B": B, "Hq": Hq, "Hkv": Hkv, "S_q": S, "S_kv": S, "D": D,
                       "causal": w.causal, "compensation": w.smooth,
                       "step": "quantize K (MXFP4) + V (FP8), then the prefill kernel with Q quantised in-kernel"},
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 2), "unit": "TFLOP/s",
                         "frac": round(achieved / peak, 4), "traffic": traffic,
                         "kernel": "qfa::k_prefill<%d,%s,0>" % (D, "true" if w.smooth else "false"),
                         "kernel_ms": round(kern_ms, 4), "algorithmic_flop_per_launch": flops + comp},
        })
        if not args.no_variants and args.only == "all":
            out["variants"] = {}
            for name, pv in (("qk4pv8_blockp", qfa.QFA_PV_FP8_BLOCKP), ("qk4pv4", qfa.QFA_PV_FP4)):
                fp4 = pv == qfa.QFA_PV_FP4
                vq, vqs = qfa.quantize_v4(v) if fp4 else qfa.quantize_v8(v)
                qfa.qfa_quantize_qk4(k, B, Hkv, S, D, 32, int(w.smooth), 1.0, k4, k4s, kbar, stream)
                vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(args.steps)]
                for i in range(args.warmup + args.steps):
                    j = i - args.warmup
                    if j >= 0:
                        vev[j][0].record(stream)
                    qfa.qfa_fwd_prefill_ex(None, None, k4, k4s, kbar, q, vq, vqs, B, Hq, Hkv, S, S, D,
                                           int(w.causal), w.scale, 32, pv, O, lse, stream)
                    if j >= 0:
                        vev[j][1].record(stream)
                torch.cuda.synchronize()
                vk = float(np.mean([a.elapsed_time(b) for a, b in vev]))
                vach = (flops + comp) / (vk * 1e-3) / 1e12
                vpeak = rl.blended_peak(flops, comp, pv_fp4=fp4) / 1e12
                out["variants"][name] = {
                    "prefill": {"kernel_ms": round(vk, 4), "achieved": round(vach, 2), "peak": round(vpeak, 2),
                                "unit": "TFLOP/s", "frac": round(vach / vpeak, 4),
                                "kernel": "qfa::k_prefill<%d,%s,%d>" % (D, "true" if w.smooth else "false", pv)}}
                del vq, vqs
            # NVFP4 Q and K (emulated on the bf16 MFMA), P and V as in the method
            c2 = qfa.qfa_exp2_scale(w.scale)
            gq = qfa.nvfp4_tensor_scale(float((q.float() * c2).abs().max()))
            gk = qfa.nvfp4_tensor_scale(float(k.float().abs().max()))
            q4n, q4ns, _ = qfa.quantize_nvfp4(q, gq, prescale=c2)
            k4n, k4ns, kbn = qfa.quantize_nvfp4(k, gk, smooth=w.smooth)
            qfa.qfa_quantize_v8(v, B, Hkv, S, D, 32, v8, v8s, stream)
            vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            for i in range(args.warmup + args.steps):
                j = i - args.warmup
                if j >= 0:
                    vev[j][0].record(stream)
                qfa.qfa_fwd_prefill_nvfp4(q4n, q4ns, k4n, k4ns, kbn, q if w.smooth else None, v8, v8s, B, Hq, Hkv,
                                          S, S, D, int(w.causal), w.scale, gq, gk, O, lse, stream)
                if j >= 0:
                    vev[j][1].record(stream)
            torch.cuda.synchronize()
            vk = float(np.mean([a.elapsed_time(b) for a, b in vev]))
            vach = (flops + comp) / (vk * 1e-3) / 1e12
            vpeak = rl.blended_peak(flops, comp, qk_bf16=True) / 1e12
            out["variants"]["nvfp4_qk"] = {
                "prefill": {"kernel_ms": round(vk, 4), "achieved": round(vach, 2), "peak": round(vpeak, 2),
                            "unit": "TFLOP/s", "frac": round(vach / vpeak, 4),
                            "kernel": "qfa::k_prefill<%d,%s,3>" % (D, "true" if w.smooth else "false"),
                            "note": "Q K^T emulated on the bf16 MFMA; peak counts it at bf16"}}
            del q4n, q4ns, k4n, k4ns, kbn
        del O, lse
    # ------------------------------------------------------------------ decode half
    if args.only in ("all", "decode") and not args.no_decode:
        wd = WORKLOADS["decode"]
        di = make_inputs(wd, seed=0, device=dev)
        Bd, Hqd, Hkvd, L, Dd = di["B"], wd.Hq, wd.Hkv, wd.S_kv, wd.D
        k4d, k4sd, _ = qfa.quantize_qk4(di["k"])
        v8d, v8sd = qfa.quantize_v8(di["v"])
        qd = di["q"]
        del di
        splits = wd.num_splits
        wsb = qfa.qfa_decode_workspace_bytes(Bd, Hqd, Dd, splits)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        Od = torch.empty((Bd, Hqd, Dd), dtype=torch.float32, device=dev)
        lsed = torch.empty((Bd, Hqd), dtype=torch.float32, device=dev)
        dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]

        def dstep(i=None):
            if i is not None:
                dev_ev[i][0].record(stream)
            qfa.qfa_fwd_decode(None, None, k4d, k4sd, None, qd, v8d, v8sd, Bd, Hqd, Hkvd, L, None, Dd, wd.scale,
                               32, splits, ws, wsb, Od, lsed, stream)
            if i is not None:
                dev_ev[i][1].record(stream)

        torch.cuda.synchronize()
        for _ in range(args.warmup):
            dstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            dstep(i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        d_ms = (t1 - t0) * 1e3 / args.steps
        d_kern = float(np.mean([a.elapsed_time(b) for a, b in dev_ev]))
        dbytes = rl.decode_algorithmic_bytes(Bd, Hqd, Hkvd, L, Dd)
        gbs = dbytes / (d_kern * 1e-3) / 1e9
        out["decode"] = {
            "metric": "decode KV GB/s", "value": round(gbs, 1), "unit": "GB/s",
            "ms_per_step": round(d_ms, 4), "kernel_ms": round(d_kern, 4),
            "config": {"workload": "decode", "B": Bd, "Hq": Hqd, "Hkv": Hkvd, "S_kv": L, "D": Dd,
                       "num_splits": splits},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": rl.PEAK_HBM / 1e9, "unit": "GB/s",
                         "frac": round(gbs * 1e9 / rl.PEAK_HBM, 4),
                         "traffic": traffic_from_profile("decode_b64_traffic.json", src),
                         "kernel": "qfa::k_decode_split<128,false,0> + k_decode_merge<128>",
                         "algorithmic_bytes_per_launch": dbytes},
        }
        # context, not graded: the device's measured read bandwidth
        ceil_gbs = stream_read_gbs()
        out["decode"]["stream_read_ceiling"] = {"GB/s": round(ceil_gbs, 1), "frac": round(gbs / ceil_gbs, 4),
                                                "kernel": "row-wise sum of 4 GiB (torch)"}
        if not args.no_variants and args.only == "all":
            vd = make_inputs(wd, seed=0, device=dev)["v"]
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
                vb = rl.decode_algorithmic_bytes(Bd, Hqd, Hkvd, L, Dd, v_fp4=fp4)
                vg = vb / (vk * 1e-3) / 1e9
                out.setdefault("variants", {}).setdefault(name, {})["decode"] = {
                    "kernel_ms": round(vk, 4), "achieved": round(vg, 1), "peak": rl.PEAK_HBM / 1e9, "unit": "GB/s",
                    "frac": round(vg * 1e9 / rl.PEAK_HBM, 4), "algorithmic_bytes_per_launch": vb}
            # NVFP4 K cache and Q (P and V as in the method)
            dq = make_inputs(wd, seed=0, device=dev)
            c2 = qfa.qfa_exp2_scale(wd.scale)
            gq = qfa.nvfp4_tensor_scale(float((dq["q"].float() * c2).abs().max()))
            gk = qfa.nvfp4_tensor_scale(float(dq["k"].float().abs().max()))
            q4n, q4ns, _ = qfa.quantize_nvfp4(dq["q"], gq, prescale=c2)
            k4n, k4ns, _ = qfa.quantize_nvfp4(dq["k"], gk)
            del v8d, v8sd
            v8d, v8sd = qfa.quantize_v8(vd)
            del dq
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
            vb = rl.decode_algorithmic_bytes(Bd, Hqd, Hkvd, L, Dd, k_nvfp4=True)
            vg = vb / (vk * 1e-3) / 1e9
            out["variants"].setdefault("nvfp4_qk", {})["decode"] = {
                "kernel_ms": round(vk, 4), "achieved": round(vg, 1), "peak": rl.PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": round(vg * 1e9 / rl.PEAK_HBM, 4), "algorithmic_bytes_per_launch": vb}
            del q4n, q4ns, k4n, k4ns, vd
        del k4d, v8d, ws
    # ------------------------------------------------------------------ CPU baseline (oracle)
    if args.only in ("all", "prefill") and not args.no_cpu_baseline:
        import oracle
        qb = bf16_bits(q)
        kb = bf16_bits(k)
        vb = bf16_bits(v)
        del q, k, v, inp
        rng = np.random.default_rng(0)

        def sample(n_rows):
            # query rows spread over heads and positions; each call also quantises
            # the K/V head and the Q heads its rows touch, as the oracle does
            rows = np.stack([np.zeros(n_rows, np.int64), rng.integers(0, Hq, n_rows),
                             rng.integers(0, S, n_rows)], axis=1)
            tc0 = time.perf_counter()
            oracle.prefill_rows(qb, kb, vb, rows, w.causal, w.scale, smooth=w.smooth, exact=False)
            dt = time.perf_counter() - tc0
            pairs = int(sum((r[2] + 1) if w.causal else S for r in rows))
            return dt, pairs

        # grow the sample until one call takes CPU_TARGET_S / 2 or more (only the
        # last call is reported; each call quantises the heads it touches again)
        n_rows = 64
        while True:
            dt, pairs = sample(n_rows)
            if dt >= CPU_TARGET_S / 2 or n_rows >= MAX_CPU_ROWS:
                break
            n_rows = int(min(MAX_CPU_ROWS, n_rows * min(16.0, CPU_TARGET_S / max(dt, 1e-3))))
        cpu_tflops = 4.0 * D * pairs / dt / 1e12
        out["cpu_baseline"] = {"value": round(cpu_tflops, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
                               "kind": "oracle",
                               "sample": "%d random query rows of %s (all %d of their visible query/key pairs), "
                                         "including the oracle quantising the K/V and Q heads they touch; %.1f s"
                                         % (n_rows, w.name, pairs, dt)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
