"""Benchmark of the packed Q1 decode path on one MI355X.

Timed step (the headline): one pass of the packed narrow-M matmul over the FFN
up/gate projection shape (K=5120, N=17408, symmetric fp16 scales, bf16
activations, bf16 output) for every M in 1..8 -- eight launches.  ``value`` is
the effective HBM bandwidth over packed words plus scales (the bytes the method
must read) for the whole step.  Each launch reads a different copy of the
weights, rotating through more copies than the 256 MB last-level cache holds,
so reads come from HBM.

The same run also measures, once each, the other rows of the path (tied LM head
M=1, down projection, embedding gather, dequantisation, the wide M=512 fallback
and the fused FFN) and times the CPU oracle on a bounded sample of the headline
workload.  Prints one JSON line.
"""
import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "Q1 GEMV effective HBM GB/s (% of 8 TB/s) at M=1..8; GEMM TFLOP/s at M=512"
ROTATE_BYTES = 1 << 30  # rotate weight copies over at least 1 GiB (> 256 MB MALL + L2)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--quick", action="store_true", help="headline step only (for profiling)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: every box here has a single MI355X and the path has no multi-GPU "
              f"leg (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_decode_q1_amd as Q
    import q1_synth as S

    torch.cuda.set_device(0)
    Q.load_library()
    if not Q.q1_device_supported(0):
        raise SystemExit(Q.q1_last_error())
    stream = torch.cuda.current_stream()

    def xdev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    def copies(w, nbytes):
        """Device copies of a packed weight, enough to cover ROTATE_BYTES."""
        base = Q.PackedQ1.from_host(w)
        n = max(2, math.ceil(ROTATE_BYTES / nbytes))
        out = [base]
        for _ in range(n - 1):
            out.append(Q.PackedQ1(base.packed.clone(), base.scales.clone(),
                                  None if base.biases is None else base.biases.clone(), base.N, base.K))
        return out

    class EventTimer:
        """Per-launch durations from HIP events recorded on the launch stream."""

        def __init__(self, n):
            self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            self.i = 0

        def run(self, fn):
            a, b = self.ev[self.i]
            a.record(stream)
            fn()
            b.record(stream)
            self.i += 1

        def times_ms(self):
            torch.cuda.synchronize()
            return [a.elapsed_time(b) for a, b in self.ev[:self.i]]

    # ------------------------------------------------------------------ headline step
    wl2 = S.workload(2)
    w2 = wl2.weights["w"]
    bytes2 = w2.metric_bytes
    W2 = copies(w2, bytes2)
    x2 = xdev(wl2.x["x"])
    y2 = torch.empty(8, w2.N, dtype=torch.bfloat16, device="cuda")
    Ms = list(range(1, 9))
    rot = [0]

    def step(timer=None):
        for M in Ms:
            W = W2[rot[0] % len(W2)]
            rot[0] += 1
            fn = lambda: Q.q1_qmm(x2[:M], W, y=y2[:M])
            if timer is None:
                fn()
            else:
                timer.run(fn)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer = EventTimer(args.steps * len(Ms))
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step(timer)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    per_launch = np.array(timer.times_ms()).reshape(args.steps, len(Ms))
    ms_per_step = total_ms / args.steps
    value = len(Ms) * bytes2 / (ms_per_step * 1e-3) / 1e9
    kern_us = per_launch.mean(axis=0) * 1e3
    avg_launch_us = float(per_launch.mean() * 1e3)
    achieved = bytes2 / (avg_launch_us * 1e-6) / 1e9
    per_m = {str(M): {"us": round(float(kern_us[i]), 2), "GB/s": round(bytes2 / (kern_us[i] * 1e-6) / 1e9, 1),
                      "pct_hbm": round(100 * bytes2 / (kern_us[i] * 1e-6) / 1e9 / HBM_PEAK_GBS, 1)}
             for i, M in enumerate(Ms)}

    detail = {"ffn_up_5120x17408_sym_f16_per_M": per_m}

    def measure(fn_list, iters, bytes_per, flops_per=None):
        """Mean per-launch microseconds over `iters` rounds of fn_list."""
        for fn in fn_list[:2]:
            fn()
        tm = EventTimer(iters * len(fn_list))
        for it in range(iters):
            for fn in fn_list:
                tm.run(fn)
        t = np.array(tm.times_ms()).mean() * 1e3
        r = {"us": round(float(t), 2)}
        if bytes_per:
            r["GB/s"] = round(bytes_per / (t * 1e-6) / 1e9, 1)
            r["pct_hbm"] = round(100 * r["GB/s"] / HBM_PEAK_GBS, 1)
        if flops_per:
            r["TFLOP/s"] = round(flops_per / (t * 1e-6) / 1e12, 1)
            r["pct_bf16_mfma"] = round(100 * r["TFLOP/s"] / BF16_PEAK_TFLOPS, 1)
        return r

    if not args.quick:
        # tied LM head, M=1, fp32 logits
        wl4 = S.workload(4)
        w4 = wl4.weights["w"]
        W4 = copies(w4, w4.metric_bytes)
        x4 = xdev(wl4.x["x"])
        y4 = torch.empty(1, w4.N, dtype=torch.float32, device="cuda")
        detail["lm_head_5120x152064_M1"] = measure([(lambda W=W: Q.q1_qmm(x4, W, y=y4)) for W in W4], 4,
                                                   w4.metric_bytes)
        # embedding gather of 4096 ids -> bf16 rows (read packed rows + scales, write bf16)
        ids = torch.from_numpy(wl4.ids).cuda()
        emb = torch.empty(4096, w4.K, dtype=torch.bfloat16, device="cuda")
        g_bytes = 4096 * (w4.K // 8 + w4.K // 128 * 2) + 4096 * w4.K * 2
        detail["embed_gather_4096_rows"] = measure([lambda: Q.q1_embed_rows(ids, W4[0], out=emb)], 20, g_bytes)
        del W4, emb
        # down projection, affine bf16, M=1..8
        wl3 = S.workload(3)
        w3 = wl3.weights["w"]
        W3 = copies(w3, w3.metric_bytes)
        x3 = xdev(wl3.x["x"])
        y3 = torch.empty(9, w3.N, dtype=torch.bfloat16, device="cuda")
        d3 = {}
        for M in Ms:
            d3[str(M)] = measure([(lambda W=W, M=M: Q.q1_qmm(x3[:M], W, y=y3[:M])) for W in W3], 1,
                                 w3.metric_bytes)
        detail["ffn_down_17408x5120_affine_bf16_per_M"] = d3
        del W3
        # wide fallback at M=512: dequant to bf16 + MFMA GEMM (config 5a)
        wl5 = S.workload(5)
        g5 = wl5.weights["gate"]
        G5 = Q.PackedQ1.from_host(g5)
        x5 = xdev(wl5.x["x"])
        deq = torch.empty(g5.N, g5.K, dtype=torch.bfloat16, device="cuda")
        deq_bytes = g5.metric_bytes + g5.N * g5.K * 2
        detail["dequant_17408x5120_to_bf16"] = measure([lambda: Q.q1_dequantize(G5, out=deq)], 10, deq_bytes)
        y5 = torch.empty(512, g5.N, dtype=torch.bfloat16, device="cuda")
        flops = 2.0 * 512 * g5.N * g5.K
        detail["wide_M512_dequant_plus_gemm"] = measure([lambda: Q.q1_qmm(x5, G5, y=y5)], 10, None, flops)
        # fused FFN, M=1..8 (three matrices, all symmetric fp16)
        FF = [Q.PackedQ1.from_host(wl5.weights[k]) for k in ("gate", "up", "down")]
        ffn_bytes = sum(wl5.weights[k].metric_bytes for k in ("gate", "up", "down"))
        reps = max(2, math.ceil(ROTATE_BYTES / ffn_bytes))
        FFc = [FF] + [[Q.PackedQ1(t.packed.clone(), t.scales.clone(), None, t.N, t.K) for t in FF]
                      for _ in range(reps - 1)]
        yf = torch.empty(8, 5120, dtype=torch.bfloat16, device="cuda")
        df = {}
        for M in Ms:
            df[str(M)] = measure([(lambda F=F, M=M: Q.q1_ffn(x5[:M], *F, y=yf[:M])) for F in FFc], 2, ffn_bytes)
        detail["fused_ffn_5120_17408_per_M"] = df
        torch.cuda.synchronize()

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        cores = len(os.sched_getaffinity(0))
        rows = np.arange(0, w2.N, 4)  # every 4th output row of the headline matrix
        sample_bytes = rows.size * (w2.K // 8 + w2.K // 128 * 2)
        t = time.perf_counter()
        for M in Ms:
            O.qmm_ref(wl2.x["x"][:M], w2.packed, w2.scales, None, w2.meta, True, w2.K, row_index=rows)
        dt = time.perf_counter() - t
        cpu = {"value": round(len(Ms) * sample_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"oracle qmm_ref (fp32 dequant + fp64 matmul) on every 4th row ({rows.size} of {w2.N}) of "
                         f"the K=5120 N=17408 matrix for M=1..8; {dt:.1f} s on {platform.processor() or 'host'}",
               "seconds": round(dt, 2)}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "ffn_up_projection_K5120_N17408_sym_f16_M1to8", "K": 5120, "N": 17408,
                   "M": "1..8", "group_size": 128, "metadata": "fp16 symmetric", "x": "bf16", "y": "bf16",
                   "bytes_per_launch": bytes2},
        "roofline": {"bound": "hbm", "kernel": "q1_gemv_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_us": round(avg_launch_us, 2),
                     "bytes_per_launch": bytes2},
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
