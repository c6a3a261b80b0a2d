"""Benchmark: fused linear cross-entropy forward+backward on one MI355X.

One step = one flce_forward_backward call over the whole batch (logits GEMM,
row CE with in-place dlogits, grad_X GEMM and grad_W GEMM for every chunk,
then the loss reduction), with the inputs already resident in HBM. The default
workload is the Llama-3-8B-shaped head: N 32768 tokens (batch 8 x seq 4096),
H 4096, V 128256, bf16 inputs with fp32 accumulation, Zipf(1.1) targets with
10% ignored, mean reduction.

Prints one JSON line with tokens/s, the fraction of the bf16 MFMA peak over
the step, the roofline of the dominant kernel (measured with HIP events on the
library's stream), peak device bytes, and the FP64 oracle timed on the host
cores on a bounded sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12    # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_head_bf16")
    ap.add_argument("--chunk-rows", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def gpu_inputs(torch, inp):
    import numpy as np

    def dev(a, bf16):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if bf16 else np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if bf16 else t).cuda()

    bf16 = inp["dtype"] == "bf16"
    return (dev(inp["X"], bf16), dev(inp["W"], bf16), dev(inp["bias"], bf16),
            dev(inp["targets"], False))


def cpu_baseline(inp, cfg, target_s):
    """Time the FP64 oracle on the first R rows of the same inputs (full W)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import flce_oracle as O

    X = np.asarray(inp["X_f32"], dtype=np.float64)
    W = np.asarray(inp["W_f32"], dtype=np.float64)
    b = None if inp["bias_f32"] is None else np.asarray(inp["bias_f32"], dtype=np.float64)
    y = inp["targets"]

    def run(rows):
        t0 = time.perf_counter()
        O.flce(X[:rows], W, y[:rows], bias=b, reduction=cfg["reduction"], row_block=1024)
        return time.perf_counter() - t0

    # Fit t(rows) = fixed + per_row * rows from two probes, then size the
    # sample to about target_s seconds.
    t64, t128 = run(64), run(128)
    per_row = max((t128 - t64) / 64.0, 1e-6)
    fixed = max(t64 - 64 * per_row, 0.0)
    rows = int(min(len(y), max(128, (target_s - fixed) / per_row)))
    rows = max(128, rows // 64 * 64)
    t = run(rows)
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
                  or [1])
    return {
        "value": rows / t,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"FP64 NumPy oracle (flce: materialised logits per 1024-row block, loss + "
                   f"grad_X + grad_W{' + grad_bias' if b is not None else ''}) on the first "
                   f"{rows} of {len(y)} token rows with the full [{W.shape[0]}, {W.shape[1]}] head; "
                   f"inputs upcast to float64 before timing; {t:.1f} s on {threads} BLAS threads"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    from linear_cross_entropy_03_amd import binding as B
    from linear_cross_entropy_03_amd import synth

    cfg = dict(synth.WORKLOADS[args.workload])
    if cfg["kind"] != "flce":
        sys.exit("bench workload must be an FLCE workload")
    N, H, V = cfg["N"], cfg["H"], cfg["V"]
    dt = B.BF16 if cfg["dtype"] == "bf16" else B.F32
    torch.cuda.set_device(0)
    log(f"generating {args.workload}: N={N} H={H} V={V} {cfg['dtype']}")
    t0 = time.time()
    inp = synth.make_workload(args.workload)
    log(f"inputs ready in {time.time() - t0:.1f}s; uploading")
    X, W, bias, y = gpu_inputs(torch, inp)

    chunk, splits = B.flce_plan(N, H, V, dt, args.chunk_rows)
    ws_bytes = B.flce_workspace_bytes(N, H, V, dt, args.chunk_rows)
    loss = torch.empty((1,), dtype=torch.float32, device="cuda")
    gX = torch.empty((N, H), dtype=torch.float32, device="cuda")
    gW = torch.empty((V, H), dtype=torch.float32, device="cuda")
    gb = torch.empty((V,), dtype=torch.float32, device="cuda") if bias is not None else None
    torch.cuda.synchronize()
    io_bytes = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ws = torch.empty((ws_bytes,), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        B.flce_forward_backward(X, W, y, bias=bias, reduction=cfg["reduction"], grad_X=gX,
                                grad_W=gW, grad_bias=gb, loss=loss, workspace=ws,
                                chunk_rows=args.chunk_rows, stream=stream)

    log(f"plan: chunk_rows={chunk} dx_splits={splits} workspace={ws_bytes / 2**30:.2f} GiB; warmup")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if B.flce_check_device_error(ws) != B.OK:
        sys.exit("device reported an out-of-range target")

    log(f"timing {args.steps} steps")
    B.flce_timing_reset()
    B.flce_timing_enable(True)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    B.flce_timing_enable(False)
    ms = start.elapsed_time(stop) / args.steps
    peak = torch.cuda.max_memory_allocated()

    # Per-kernel roofline from the library's HIP events over the timed region.
    e = 2 if cfg["dtype"] == "bf16" else 4
    gemm_flops_per_step = 2.0 * N * H * V
    kernels = {}
    for kind in ("logits_gemm", "grad_x_gemm", "grad_w_gemm", "row_ce", "other"):
        tot_ms, launches = B.flce_timing_read(kind)
        if launches == 0:
            continue
        entry = {"ms_per_launch": tot_ms / launches, "launches": launches}
        if kind.endswith("gemm"):
            per_launch = gemm_flops_per_step * args.steps / launches
            entry.update(bound="mfma", unit="TFLOP/s", algorithmic_per_launch=per_launch,
                         achieved=per_launch / (tot_ms / launches * 1e-3) / 1e12,
                         peak=PEAK_BF16_FLOPS / 1e12)
        elif kind == "row_ce":
            per_launch = 2.0 * N * V * e * args.steps / launches
            entry.update(bound="hbm", unit="GB/s", algorithmic_per_launch=per_launch,
                         achieved=per_launch / (tot_ms / launches * 1e-3) / 1e9,
                         peak=PEAK_HBM_BYTES / 1e9)
        if "achieved" in entry:
            entry["frac"] = entry["achieved"] / entry["peak"]
        entry["share_of_step"] = tot_ms / args.steps / ms
        kernels[kind] = entry
    B.flce_timing_reset()
    dom_kind = max((k for k in kernels if "achieved" in kernels[k]),
                   key=lambda k: kernels[k]["ms_per_launch"] * kernels[k]["launches"])
    dom = kernels[dom_kind]
    roofline = {"kernel": dom_kind, "bound": dom["bound"], "achieved": dom["achieved"],
                "peak": dom["peak"], "unit": dom["unit"], "frac": dom["frac"], "traffic": None,
                "algorithmic_per_launch": dom["algorithmic_per_launch"]}

    tokens_per_s = N / (ms * 1e-3)
    step_flops = 6.0 * N * H * V
    result = {
        "metric": "FLCE fwd+bwd tokens/s + % bf16 MFMA peak at H4096 V128256; peak HBM bytes",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic (seeded numpy: X~N(0,1), W~N(0,0.02), "
                + ("Zipf(1.1) targets" if cfg.get("target_dist") == "zipf" else "uniform targets")
                + ", 10% ignore_index)",
        "config": {"workload": args.workload, "N": N, "H": H, "V": V, "reduction": cfg["reduction"],
                   "bias": bias is not None, "chunk_rows": chunk, "dx_splits": splits,
                   "parallelism": "single GPU"},
        "mfma_frac_step": step_flops / (ms * 1e-3) / PEAK_BF16_FLOPS,
        "step_tflops": step_flops / (ms * 1e-3) / 1e12,
        "peak_bytes": peak,
        "extra_bytes": peak - io_bytes,
        "chunk_logits_bytes": chunk * ((V + 7) // 8 * 8) * e,
        "materialised_logits_bytes": N * V * e,
        "roofline": roofline,
        "kernels": kernels,
        "loss": float(loss.item()),
    }
    if not args.no_cpu_baseline:
        log("timing the FP64 oracle on a CPU sample")
        del ws, gX, gW
        result["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
