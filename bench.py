"""Benchmark of the packed Q1 decode path on one MI355X.

Timed step (the headline): one pass of the packed narrow-M matmul over the FFN
up/gate projection shape (K=5120, N=17408, symmetric fp16 scales, bf16
activations, bf16 output) for every M in 1..8 -- eight launches.  ``value`` is
the effective HBM bandwidth over packed words plus scales (the bytes the method
must read) for the whole step.  Each launch reads a different copy of the
weights, rotating through more copies than the 256 MB last-level cache holds,
so reads come from HBM.

``roofline`` covers the dominant kernel of the step (the matrix-core kernel,
M = 2..8): its average launch duration comes from HIP events around runs of
back-to-back launches on the launch stream (so it includes the short dispatch
gap between kernels), and its HBM traffic from the committed rocprofv3 counter
summary when that summary was taken from the current kernel sources.

The same run also measures, once each, the other rows of the path (tied LM head
M=1, down projection, embedding gather, dequantisation, the wide M=512 product,
the fused FFN, the sign packer and the symmetric-bias check), a read ceiling
(one launch that only reads the same number of bytes, for the headline and the
tied-head sizes), and times the CPU oracle on a bounded sample of the headline
workload.  Prints one JSON line.
"""
import argparse
import hashlib
import json
import math
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
METRIC = "Q1 GEMV effective HBM GB/s (% of 8 TB/s) at M=1..8; GEMM TFLOP/s at M=512"
ROTATE_BYTES = 1 << 30  # rotate weight copies over at least 1 GiB (> 256 MB MALL + L2)
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "q1_mma_kernel_ffn_up_K5120_N17408_M2to8_pmc.txt")
DOMINANT = "q1_mma_kernel"
DOMINANT_MS = list(range(2, 9))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--quick", action="store_true", help="headline step only (for profiling)")
    p.add_argument("--copy-calib", action="store_true",
                   help="also run a plain 256 MiB device copy (reference for the HBM byte counters)")
    p.add_argument("--only", default="",
                   help="comma-separated detail rows to run instead of the whole bench (for profiling): "
                        + ",".join(ROWS) + "; prints those rows only")
    return p.parse_args()


ROWS = ["headline", "lm_head", "gather", "down", "dequant", "pack", "symcheck", "wide", "wide_dense", "ffn",
        "ffn_single"]


def source_sha256() -> str:
    """Hash of the kernel sources (identifies which build a counter profile belongs to)."""
    d = os.path.join(ROOT, "gemm_decode_q1_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".inc", ".h", ".cpp")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()


def read_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is missing or was taken from other sources."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m_sha = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m_sha or not m_b or m_sha.group(1) != source_sha256():
        return None
    return float(m_b.group(1))


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

    def capture(fns):
        """A HIP graph of the launches in `fns` (after one eager run of each)."""
        for fn in fns:
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for fn in fns:
                fn()
        return g

    def replay_us(g, nlaunch, reps):
        """Mean microseconds per launch over `reps` back-to-back replays of g,
        from two HIP events on the stream the replays run on."""
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * nlaunch)

    def run_batch(fns, reps):
        """Mean microseconds per launch of `fns`, launched back to back from a
        graph replay (the host's per-call cost does not enter).  The list is
        repeated until the graph holds at least 20 launches, so the host's
        cost of launching the graph itself is spread over them too."""
        k = max(1, math.ceil(20 / len(fns)))
        return replay_us(capture(fns * k), len(fns) * k, reps)

    def ws_for(M, W):
        n = Q.q1_qmm_workspace_bytes(M, W)
        return torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda") if n else None

    def bw(nbytes, us):
        gbs = nbytes / (us * 1e-6) / 1e9
        return {"us": round(us, 2), "GB/s": round(gbs, 1), "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 1)}

    only = [r for r in args.only.split(",") if r]
    for r in only:
        if r not in ROWS:
            raise SystemExit(f"unknown row {r!r}; rows: {', '.join(ROWS)}")

    def want(row):
        return not only or row in only

    Ms = list(range(1, 9))
    detail = {}
    value = ms_per_step = achieved = dom_us = None
    ceiling2 = None

    big = torch.empty(ROTATE_BYTES + (256 << 20), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def read_ceiling(nbytes):
        """One launch that only reads nbytes with 16-byte loads (consecutive
        launches read consecutive slices of 1 GiB, so from HBM): what a single
        launch of that size can reach on this part."""
        nb = nbytes // 16 * 16
        n = max(2, ROTATE_BYTES // nb)
        return bw(nb, run_batch([(lambda i=i: Q.q1_stream_read(big[i * nb:(i + 1) * nb], sink)) for i in range(n)], 3))

    # ------------------------------------------------------------------ headline step
    wl2 = S.workload(2)
    w2 = wl2.weights["w"]
    bytes2 = w2.metric_bytes
    if want("headline"):
        W2 = copies(w2, bytes2)
        x2 = xdev(wl2.x["x"])
        ws2 = {M: ws_for(M, W2[0]) for M in Ms}
        ys = [torch.empty(M, w2.N, dtype=torch.bfloat16, device="cuda") for M in Ms]

        # One step = the eight launches; consecutive steps take the next copies
        # of the weights.  The timed steps run as replays of a graph that holds
        # `steps` steps (captured once), checked against an eager run first.
        def step_fns(first_copy):
            return [(lambda M=M, W=W2[(first_copy + i) % len(W2)]: Q.q1_qmm(x2[:M], W, y=ys[M - 1],
                                                                              workspace=ws2[M]))
                    for i, M in enumerate(Ms)]

        fns = [fn for s_ in range(args.steps) for fn in step_fns(s_ * len(Ms))]
        for fn in fns[-len(Ms):]:
            fn()
        torch.cuda.synchronize()
        eager = [y.clone() for y in ys]
        g_step = capture(fns)
        for _ in range(max(1, args.warmup)):
            g_step.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(eager, ys)):
            raise SystemExit("graph replay of the step differs from the eager result")
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        g_step.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        ms_per_step = t0.elapsed_time(t1) / args.steps
        value = len(Ms) * bytes2 / (ms_per_step * 1e-3) / 1e9
        del g_step

        # per-M launch durations (back-to-back launches over the rotating copies)
        per_m = {}
        for M in Ms:
            us = run_batch([(lambda W=W, M=M: Q.q1_qmm(x2[:M], W, y=ys[M - 1], workspace=ws2[M])) for W in W2], 3)
            per_m[str(M)] = bw(bytes2, us)
        dom_us = float(np.mean([per_m[str(M)]["us"] for M in DOMINANT_MS]))
        ceiling2 = read_ceiling(bytes2)
        achieved = bytes2 / (dom_us * 1e-6) / 1e9
        detail.update({"ffn_up_5120x17408_sym_f16_per_M": per_m, "read_ceiling_12533760_bytes": ceiling2,
                       "kernels": {"M=1": "q1_gemv_kernel (nibble tables)",
                                   "M=2..8": "q1_mma_kernel (fp8 x fp4 MFMA)"}})
        del W2
    traffic = read_traffic()

    if args.copy_calib:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    wl4 = S.workload(4) if (want("lm_head") or want("gather")) and not args.quick else None
    if wl4 is not None:
        w4 = wl4.weights["w"]
        W4 = copies(w4, w4.metric_bytes)
        if want("lm_head"):
            # tied LM head, M=1, fp32 logits
            x4 = xdev(wl4.x["x"])
            y4 = torch.empty(1, w4.N, dtype=torch.float32, device="cuda")
            ws4 = ws_for(1, W4[0])
            detail["lm_head_5120x152064_M1"] = bw(w4.metric_bytes, run_batch(
                [(lambda W=W: Q.q1_qmm(x4, W, y=y4, workspace=ws4)) for W in W4], 3))
            detail["read_ceiling_109486080_bytes"] = read_ceiling(w4.metric_bytes)
        if want("gather"):
            # embedding gather of 4096 ids -> bf16 rows (read packed rows + scales, write bf16)
            ids = torch.from_numpy(wl4.ids).cuda()
            emb = torch.empty(4096, w4.K, dtype=torch.bfloat16, device="cuda")
            g_bytes = 4096 * (w4.K // 8 + w4.K // 128 * 2) + 4096 * w4.K * 2
            detail["embed_gather_4096_rows"] = bw(g_bytes, run_batch([lambda: Q.q1_embed_rows(ids, W4[0], out=emb)], 20))
            del emb
        del W4

    if not args.quick and (want("down") or want("symcheck")):
        wl3 = S.workload(3)
        w3 = wl3.weights["w"]
        if want("down"):
            # down projection, affine bf16, M=1..8
            W3 = copies(w3, w3.metric_bytes)
            x3 = xdev(wl3.x["x"])
            y3 = torch.empty(9, w3.N, dtype=torch.bfloat16, device="cuda")
            ws3 = {M: ws_for(M, W3[0]) for M in Ms}
            detail["ffn_down_17408x5120_affine_bf16_per_M"] = {
                str(M): bw(w3.metric_bytes, run_batch(
                    [(lambda W=W, M=M: Q.q1_qmm(x3[:M], W, y=y3[:M], workspace=ws3[M])) for W in W3], 2))
                for M in Ms}
            del W3
        if want("symcheck"):
            # symmetric check of the down projection's affine metadata (scales + biases read)
            W3c = Q.PackedQ1.from_host(w3)
            sc_bytes = 2 * w3.N * (w3.K // 128) * 2
            detail["check_symmetric_5120x17408_bf16"] = bw(sc_bytes, run_batch([lambda: Q.q1_check_symmetric(W3c)], 20))
            del W3c

    if not args.quick and any(want(r) for r in ("dequant", "pack", "wide", "wide_dense", "ffn", "ffn_single")):
        wl5 = S.workload(5)
        g5 = wl5.weights["gate"]
        G5 = Q.PackedQ1.from_host(g5)
        x5 = xdev(wl5.x["x"])
        if want("dequant") or want("pack"):
            deq = torch.empty(g5.N, g5.K, dtype=torch.bfloat16, device="cuda")
            deq_bytes = g5.metric_bytes + g5.N * g5.K * 2
            detail["dequant_17408x5120_to_bf16"] = bw(deq_bytes, run_batch([lambda: Q.q1_dequantize(G5, out=deq)], 10))
            if want("pack"):
                # sign packer on the same shape: read the bf16 matrix, write words and scales
                pk_bytes = g5.N * g5.K * 2 + g5.metric_bytes
                detail["pack_signs_17408x5120_bf16_to_q1"] = bw(pk_bytes, run_batch(
                    [lambda: Q.q1_pack_signs(deq, torch.float16)], 10))
            del deq
        flops = 2.0 * 512 * g5.N * g5.K
        y5 = torch.empty(512, g5.N, dtype=torch.bfloat16, device="cuda")
        if want("wide"):
            # wide M=512 product on the FFN gate shape: activation image (fp8
            # hi/lo operands) + fp8 x fp4 matrix-core kernel from the packed words
            ws5 = ws_for(512, G5)
            us = run_batch([lambda: Q.q1_qmm(x5, G5, y=y5, workspace=ws5)], 10)
            tf = flops / (us * 1e-6) / 1e12
            # each activation row is two fp8 operand rows (hi + lo/16), so the
            # matrix cores issue twice the useful flops, at the fp8 rate
            detail["wide_M512_qmm_5120x17408"] = {"us": round(us, 2), "TFLOP/s": round(tf, 1),
                                                  "pct_bf16_mfma": round(100 * tf / BF16_PEAK_TFLOPS, 1),
                                                  "mfma_issue_pct_fp8": round(100 * 2 * tf / FP8_PEAK_TFLOPS, 1)}
            del ws5
        if want("wide_dense"):
            # the pages' dense fallback at the same size: dequantise to bf16 in
            # the workspace, then the bf16 MFMA GEMM (both launches timed)
            os.environ["Q1_WIDE_KERNEL"] = "dequant"
            try:
                wsd = ws_for(512, G5)
                us = run_batch([lambda: Q.q1_qmm(x5, G5, y=y5, workspace=wsd)], 5)
            finally:
                del os.environ["Q1_WIDE_KERNEL"]
            tf = flops / (us * 1e-6) / 1e12
            detail["wide_M512_dense_fallback_5120x17408"] = {"us": round(us, 2), "TFLOP/s": round(tf, 1),
                                                             "pct_bf16_mfma": round(100 * tf / BF16_PEAK_TFLOPS, 1)}
            del wsd
        if want("ffn") or want("ffn_single"):
            # fused FFN, M=1..8 (three matrices, all symmetric fp16)
            FF = [Q.PackedQ1.from_host(wl5.weights[k]) for k in ("gate", "up", "down")]
            ffn_bytes = sum(wl5.weights[k].metric_bytes for k in ("gate", "up", "down"))
            reps = max(2, math.ceil(ROTATE_BYTES / ffn_bytes))
            FFc = [FF] + [[Q.PackedQ1(t.packed.clone(), t.scales.clone(), None, t.N, t.K) for t in FF]
                          for _ in range(reps - 1)]
            yf = torch.empty(8, 5120, dtype=torch.bfloat16, device="cuda")
            wsf = {M: torch.zeros(max(Q.q1_ffn_workspace_bytes(M, *FF), 256), dtype=torch.uint8, device="cuda")
                   for M in Ms}
            if want("ffn"):
                detail["fused_ffn_5120_17408_per_M"] = {
                    str(M): bw(ffn_bytes, run_batch(
                        [(lambda F=F, M=M: Q.q1_ffn(x5[:M], *F, y=yf[:M], workspace=wsf[M])) for F in FFc], 2))
                    for M in Ms}
            if want("ffn_single"):
                # the same FFN as one persistent launch (Q1_FFN_KERNEL=single)
                os.environ["Q1_FFN_KERNEL"] = "single"
                try:
                    wss = {M: torch.zeros(max(Q.q1_ffn_workspace_bytes(M, *FF), 256), dtype=torch.uint8,
                                          device="cuda") for M in Ms}
                    detail["ffn_single_launch_5120_17408_per_M"] = {
                        str(M): bw(ffn_bytes, run_batch(
                            [(lambda F=F, M=M: Q.q1_ffn(x5[:M], *F, y=yf[:M], workspace=wss[M])) for F in FFc], 2))
                        for M in Ms}
                finally:
                    del os.environ["Q1_FFN_KERNEL"]
            del FFc
        torch.cuda.synchronize()

    if only:
        print(json.dumps({"only": only, "detail": detail}), flush=True)
        return

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        cores = len(os.sched_getaffinity(0))
        # whole-matrix calls at M = 1, 2, .., 8, 1, .. until 10 s of CPU work
        # have passed (one call takes a few seconds)
        t = time.perf_counter()
        calls = []
        while True:
            M = Ms[len(calls) % len(Ms)]
            O.qmm_ref(wl2.x["x"][:M], w2.packed, w2.scales, None, w2.meta, True, w2.K)
            calls.append(M)
            dt = time.perf_counter() - t
            if dt >= 10.0:
                break
        cpu = {"value": round(len(calls) * bytes2 / dt / 1e9, 3), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": f"oracle qmm_ref (fp32 dequant + fp64 matmul) over the whole K=5120 N=17408 matrix, "
                         f"{len(calls)} calls at M={','.join(map(str, calls))}, {dt:.1f} s on "
                         f"{platform.processor() or 'host'}",
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
        # M = 1: fp32 table sums; M = 2..8: fp8 (E4M3, each activation as
        # hi + lo/16) times fp4 (E2M1) bit codes on the matrix cores, fp32
        # accumulation; every weight is used exactly
        "dtype": "fp8(hi+lo)xfp4->f32",
        "data": "synthetic",
        "config": {"workload": "ffn_up_projection_K5120_N17408_sym_f16_M1to8", "K": 5120, "N": 17408,
                   "M": "1..8", "group_size": 128, "metadata": "fp16 symmetric", "x": "bf16", "y": "bf16",
                   "bytes_per_launch": bytes2},
        "roofline": {"bound": "hbm", "kernel": DOMINANT, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "avg_launch_us": round(dom_us, 2), "launches": "M=2..8", "bytes_per_launch": bytes2,
                     "read_ceiling_GB/s": ceiling2["GB/s"]},
        "cpu_baseline": cpu,
        "detail": detail,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
