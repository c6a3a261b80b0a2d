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

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_FLOPS = 2.5e15   # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12    # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_head_bf16")
    ap.add_argument("--chunk-rows", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-ce", action="store_true", help="skip the standalone CE measurement")
    ap.add_argument("--no-vp", action="store_true",
                    help="skip the vocabulary-parallel shard measurement")
    ap.add_argument("--no-mh", action="store_true", help="skip the multi-head measurement")
    ap.add_argument("--no-g16", action="store_true",
                    help="skip the 16-bit-gradient measurement")
    ap.add_argument("--no-distill", action="store_true", help="skip the distillation measurement")
    ap.add_argument("--no-dpo", action="store_true", help="skip the DPO measurement")
    ap.add_argument("--no-packing", action="store_true",
                    help="run the FLCE step with row packing off (every row through the "
                         "products, ignored ones included)")
    ap.add_argument("--no-unpacked", action="store_true",
                    help="skip the comparison steps with row packing off")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other full-size workloads (Llama-3.2-1B head, 256k vocabulary)")
    ap.add_argument("--no-eager", action="store_true",
                    help="skip the PyTorch eager context measurement")
    ap.add_argument("--profile-step", action="store_true",
                    help="for rocprofv3 counter runs: a 1 GiB device copy (counter calibration), "
                         "then one warmup and one timed FLCE step; prints nothing else")
    ap.add_argument("--counters-from", nargs="+", metavar="PMC_DIR",
                    help="summarise rocprofv3 --pmc runs of --profile-step per kernel class into "
                         "profiles/counters_<workload>.json and exit")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs of --profile-step (FETCH_SIZE, "
                         "WRITE_SIZE) into profiles/traffic_<workload>.json and exit")
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

    # Fit t(rows) = fixed + per_row * rows from two probes (each pays the
    # fixed cost of the [V, H] float64 grad_W), then size the sample to about
    # target_s seconds; a flat probe pair falls back to the larger probe's
    # average, and the sample never exceeds a quarter of the rows.
    t256, t768 = run(256), run(768)
    per_row = (t768 - t256) / 512.0
    if per_row <= 0.2 * t768 / 768.0:
        per_row = t768 / 768.0
    fixed = max(t768 - 768 * per_row, 0.0)
    rows = int((target_s - fixed) / per_row)
    rows = max(256, min(rows, len(y) // 4) // 64 * 64)
    t = run(rows)
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
                  or [1])
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         model)
    except OSError:
        pass
    return {
        "value": rows / t,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": model,
        "affinity_cores": len(os.sched_getaffinity(0)),
        "sample": (f"FP64 NumPy oracle (flce: materialised logits per 1024-row block, loss + "
                   f"grad_X + grad_W{' + grad_bias' if b is not None else ''}) on the first "
                   f"{rows} of {len(y)} token rows with the full [{W.shape[0]}, {W.shape[1]}] head; "
                   f"inputs upcast to float64 before timing; {t:.1f} s on {threads} BLAS threads"),
    }


KERNEL_KINDS = {  # kernel-name fragment -> kind reported by the timing hooks
    "k_ring<true, true, 0": "logits_gemm",     # X W^T (both operands k-contiguous)
    "k_ring<true, false": "grad_x_gemm",       # dZ W
    "k_ring<false, ": "grad_w_gemm",           # dZ^T X (X transposed, or as stored)
    "k_row_ce": "row_ce",
}


def code_tokens(text):
    """C++ source without comments and with whitespace runs collapsed, so that
    comment and layout edits do not count as kernel changes (string literals
    in the HIP sources hold no comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    """Hash of the HIP sources' code (comments and layout ignored); traffic
    figures are valid only for this hash."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_cross_entropy_03_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update((f + "\n" + code_tokens(fh.read())).encode())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def summarise_traffic(workload, fetch_dir, write_dir):
    """Per-launch HBM bytes per kernel class from FETCH_SIZE / WRITE_SIZE runs
    (KiB per dispatch), each scaled by the same counter's reading for the
    1 GiB device copy that --profile-step runs first."""
    import csv
    import glob

    def per_kernel(d, counter):
        path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    out = {"workload": workload, "source_hash": kernel_source_hash(), "copy_bytes": 1 << 30,
           "kernels": {}}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = per_kernel(d, counter)
        copy = [v for k, v in vals.items() if "copyBuffer" in k or "copy_kernel" in k]
        if not copy:
            raise SystemExit(f"no copy kernel found in {d}")
        copy_kib = float(np.median(copy[0]))
        factor = (1 << 30) / (copy_kib * 1024.0)
        out[f"{counter}_copy_kib"] = copy_kib
        out[f"{counter}_factor"] = factor
        for name, v in vals.items():
            kind = next((k2 for frag, k2 in KERNEL_KINDS.items() if frag in name), None)
            if kind is None:
                continue
            e = out["kernels"].setdefault(kind, {})
            # second step's dispatches (the first step is warmup)
            e[counter.lower() + "_bytes"] = float(np.mean(v[len(v) // 2:])) * 1024.0 * factor
    for e in out["kernels"].values():
        e["traffic_bytes"] = e.get("fetch_size_bytes", 0.0) + e.get("write_size_bytes", 0.0)
    with open(traffic_path(workload), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def summarise_counters(workload, dirs):
    """Per kernel class, the mean per dispatch over the timed step (the second
    half of the dispatches) of every counter in one or more rocprofv3 --pmc
    runs of --profile-step; writes profiles/counters_<workload>.json and
    prints a markdown table."""
    import csv
    import glob
    per = {}
    for d in dirs:
        path = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)[0]
        vals = {}
        for r in csv.DictReader(open(path)):
            kind = next((k2 for frag, k2 in KERNEL_KINDS.items() if frag in r["Kernel_Name"]), None)
            if kind is None:
                continue
            vals.setdefault((kind, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
        for (kind, name), v in vals.items():
            per.setdefault(kind, {})[name] = float(np.mean(v[len(v) // 2:]))
    out = {"workload": workload, "source_hash": kernel_source_hash(), "kernels": per}
    with open(os.path.join(ROOT, "profiles", f"counters_{workload}.json"), "w") as f:
        json.dump(out, f, indent=1)
    names = sorted({n for k in per.values() for n in k})
    print("| kernel | " + " | ".join(names) + " |")
    print("|---" * (len(names) + 1) + "|")
    for kind, k in per.items():
        print(f"| {kind} | " + " | ".join(f"{k.get(n, float('nan')):.4g}" for n in names) + " |")


def load_traffic(workload):
    try:
        with open(traffic_path(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("source_hash") == kernel_source_hash() else None


def time_calls(torch, stream, call, reps):
    """Milliseconds per call over `reps` back-to-back calls on `stream`
    (timing hooks off)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def hooked_pass(torch, B, call, reps):
    """`reps` more calls with the library's per-kernel timing hooks on; the
    tallies are left for flce_timing_read."""
    B.flce_timing_reset()
    B.flce_timing_enable(True)
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    B.flce_timing_enable(False)


def bench_ce(torch, B, reps=200):
    """Standalone CE over bf16 logits [1024, 32768] (one vocabulary shard,
    std 2, 5% ignored), gradient to a separate buffer, mean reduction. Eight
    buffer sets (1 GiB) are rotated so the 256 MB Infinity Cache cannot hold
    the working set. Algorithmic bytes per call: read logits + write grad
    (2 x N x V x 2) + targets 4N + per-row losses 4N."""
    from linear_cross_entropy_03_amd import synth
    N, V = 1024, 32768
    inp = synth.make_ce_inputs(N, V, "bf16", std=2.0, ignore_frac=0.05)
    base = torch.from_numpy(inp["logits"].view(np.int16)).view(torch.bfloat16).cuda()
    y = torch.from_numpy(inp["targets"]).cuda()
    sets = [(base.clone(), torch.empty_like(base)) for _ in range(8)]
    loss = torch.empty(1, device="cuda")
    ws = torch.empty(B.ce_workspace_bytes(N, V), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for i in range(8):
        B.ce_forward_backward(sets[i][0], y, grad_logits=sets[i][1], loss=loss, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # The call, hooks off.
    a.record(stream)
    for r in range(reps):
        lg, g = sets[r % 8]
        B.ce_forward_backward(lg, y, grad_logits=g, loss=loss, workspace=ws, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    call_us = a.elapsed_time(b) / reps * 1e3
    # The row kernel alone: the same call with reduction "none" is that one
    # launch (per-row losses to a [N] output), hooks off. Per-launch event
    # hooks add microseconds to a kernel this short, so they only count the
    # launches of the mean call here.
    loss_rows = torch.empty(N, device="cuda")
    a.record(stream)
    for r in range(reps):
        lg, g = sets[r % 8]
        B.ce_forward_backward(lg, y, reduction="none", grad_logits=g, loss=loss_rows, workspace=ws,
                              stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    kern_us = a.elapsed_time(b) / reps * 1e3
    B.flce_timing_reset()
    B.flce_timing_enable(True)
    for r in range(reps):
        lg, g = sets[r % 8]
        B.ce_forward_backward(lg, y, grad_logits=g, loss=loss, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    B.flce_timing_enable(False)
    _, k_n = B.flce_timing_read("row_ce")
    _, o_n = B.flce_timing_read("other")
    B.flce_timing_reset()
    algo = 2.0 * N * V * 2 + 8.0 * N
    # shard statistics over the same shard (read-only pass)
    m = torch.empty(N, device="cuda"); s_ = torch.empty(N, device="cuda"); t = torch.empty(N, device="cuda")
    a.record(stream)
    for r in range(reps):
        B.ce_shard_stats(sets[r % 8][0], y, 0, 2 * V, out=(m, s_, t), workspace=ws, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    st_us = a.elapsed_time(b) / reps * 1e3
    st_algo = 1.0 * N * V * 2 + 16.0 * N
    # device-to-device copy of 1 GiB as the practical bandwidth reference
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(5):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    copy_GBps = 2.0 * (1 << 30) * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    return {
        "workload": "ce_shard_bf16 (logits [1024, 32768] bf16, mean, grad out of place)",
        "us_per_call": call_us, "launches_per_call": (k_n + o_n) / reps,
        "row_ce_kernel_us": kern_us,
        "row_ce_kernel_timing": "the same calls with reduction none: the row kernel's one launch, hooks off",
        "reduction_launch_us_per_call": call_us - kern_us,
        "frac_hbm_call": algo / (call_us * 1e-6) / PEAK_HBM_BYTES,
        "algorithmic_bytes": algo,
        "achieved_GBps_call": algo / (call_us * 1e-6) / 1e9,
        "achieved_GBps_kernel": algo / (kern_us * 1e-6) / 1e9,
        "frac_hbm_kernel": algo / (kern_us * 1e-6) / PEAK_HBM_BYTES,
        "copy_GBps": copy_GBps,
        "frac_of_copy_kernel": algo / (kern_us * 1e-6) / 1e9 / copy_GBps,
        "shard_stats_us_per_call": st_us,
        "shard_stats_GBps": st_algo / (st_us * 1e-6) / 1e9,
    }


def bench_vocab_parallel(torch, B, X, W, y, cfg, reps=5):
    """The vocabulary-parallel path at a real shard shape: the 8B head split 8
    ways, shard 3 (V_local 16032). One rank's work per step: shard statistics
    (logits GEMM + statistics), the combine of 8 shards' statistics (the same
    statistics replicated, so only the arithmetic is real), then the shard's
    backward (logits GEMM again, dZ from the global lse, grad_X partial and
    grad_W shard). GEMM work per step: 2 x N x H x V_local flop for the
    statistics (every row) and 3 x 2 x L x H x V_local for the backward, L the
    rows it runs over (the non-ignored ones when row packing is on)."""
    N, H, V = cfg["N"], cfg["H"], cfg["V"]
    P = 8
    Vl = V // P
    a = 3 * Vl
    Ws = W[a:a + Vl]
    stream = torch.cuda.current_stream()
    m, s_, t = (torch.empty(N, device="cuda") for _ in range(3))
    ms, ss, ts = (torch.empty(P, N, device="cuda") for _ in range(3))
    lse = torch.empty(N, device="cuda")
    loss = torch.empty(1, device="cuda")
    gX = torch.empty(N, H, device="cuda")
    gW = torch.empty(Vl, H, device="cuda")
    ws = torch.empty(B.flce_workspace_bytes(N, H, Vl, B.BF16), dtype=torch.uint8, device="cuda")
    cws = torch.empty(B.ce_workspace_bytes(N, V), dtype=torch.uint8, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def once(record):
        if record:
            ev[0].record(stream)
        B.flce_shard_stats(X, Ws, y, a, V, out=(m, s_, t), workspace=ws, stream=stream)
        for k in range(P):
            ms[k].copy_(m); ss[k].copy_(s_); ts[k].copy_(t)
        if record:
            ev[1].record(stream)
        B.ce_combine_shard_stats(ms, ss, ts, y, V, reduction=cfg["reduction"], row_lse=lse, loss=loss,
                                 workspace=cws, stream=stream)
        if record:
            ev[2].record(stream)
        B.flce_shard_backward(X, Ws, y, lse, a, V, reduction=cfg["reduction"], grad_X=gX, grad_W=gW,
                              grad_bias=False, workspace=ws, stream=stream)
        if record:
            ev[3].record(stream)

    once(False)
    torch.cuda.synchronize()
    tot = [0.0, 0.0, 0.0]
    for _ in range(reps):
        once(True)
        torch.cuda.synchronize()
        for i in range(3):
            tot[i] += ev[i].elapsed_time(ev[i + 1])
    # Kernel times in a separate pass with the hooks on.
    B.flce_timing_reset()
    B.flce_timing_enable(True)
    for _ in range(reps):
        once(False)
    torch.cuda.synchronize()
    B.flce_timing_enable(False)
    gemm_ms = sum(B.flce_timing_read(k)[0] for k in ("logits_gemm", "grad_x_gemm", "grad_w_gemm"))
    row_ms, row_n = B.flce_timing_read("row_ce")
    B.flce_timing_reset()
    stats_ms, comb_ms, bwd_ms = (x / reps for x in tot)
    step_ms = stats_ms + comb_ms + bwd_ms
    gemm_flops = 2.0 * (N + 3 * rows_through_products(B, y)) * H * Vl
    return {
        "workload": f"llama8b_head_bf16 vocabulary shard 3 of {P} (N {N}, H {H}, V_local {Vl}, "
                    f"V {V}, {cfg['reduction']})",
        "ms_shard_stats": stats_ms, "ms_combine": comb_ms, "ms_shard_backward": bwd_ms,
        "ms_per_step": step_ms, "tokens_per_s": N / (step_ms * 1e-3),
        "gemm_tflops": gemm_flops / (gemm_ms / reps * 1e-3) / 1e12,
        "gemm_frac": gemm_flops / (gemm_ms / reps * 1e-3) / PEAK_BF16_FLOPS,
        "row_kernels_ms_per_step": row_ms / reps, "row_kernel_launches_per_step": row_n / reps,
        "note": "the shard-stats step's 8 statistics copies are replicated on the device; "
                "no collective runs (one GPU)",
    }


def bench_torch_eager(torch, X, W, y, cfg, reps=3):
    """Context, not a target: the materialised computation in plain PyTorch on
    the same GPU and inputs: logits = X W^T in bf16 (the vendor GEMM library),
    upcast to float32, F.cross_entropy (ignore_index, the workload's
    reduction) and autograd for grad_X and grad_W."""
    import torch.nn.functional as F
    Xr = X.detach().clone().requires_grad_(True)
    Wr = W.detach().clone().requires_grad_(True)
    yl = y.long()

    def step():
        Xr.grad = None
        Wr.grad = None
        logits = Xr @ Wr.t()
        loss = F.cross_entropy(logits.float(), yl, ignore_index=-100, reduction=cfg["reduction"])
        loss.backward()
        return loss

    step()
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        loss = step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    out = {"what": "PyTorch eager, materialised logits (bf16 GEMMs, float32 cross_entropy, autograd)",
           "ms_per_step": ms, "tokens_per_s": cfg["N"] / (ms * 1e-3),
           "peak_extra_bytes": torch.cuda.max_memory_allocated() - base, "loss": float(loss.item())}
    del Xr, Wr
    torch.cuda.empty_cache()
    return out


def bench_distill(torch, B, X, W, y, cfg, n_rows=8192, reps=3):
    """Jensen-Shannon distillation at the 8B head's shape on the first n_rows
    token rows: the student is the workload's head, the teacher the same head
    rolled by 11 vocabulary rows over the hidden states rolled by one row (no
    new host draws), temperature 2. Per call: student and teacher logits,
    grad_X and grad_W of the student, 8 x n x H x V flop, plus the row kernel's
    three passes over both chunk logits."""
    N, H, V = n_rows, cfg["H"], cfg["V"]
    Xs = X[:N]
    Xt = torch.roll(X[:N], shifts=1, dims=0).contiguous()
    Wt = torch.roll(W, shifts=11, dims=0).contiguous()
    loss = torch.empty(1, device="cuda")
    gX = torch.empty(N, H, device="cuda")
    gW = torch.empty(V, H, device="cuda")
    ws = torch.empty(B.flce_jsd_workspace_bytes(N, H, V, B.BF16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        B.flce_jsd_forward_backward(Xs, W, Xt, Wt, y[:N], temperature=2.0, reduction=cfg["reduction"],
                                    grad_X=gX, grad_W=gW, loss=loss, workspace=ws, stream=stream)
    call()
    torch.cuda.synchronize()
    ms = time_calls(torch, stream, call, reps)
    hooked_pass(torch, B, call, reps)
    row_ms, row_n = B.flce_timing_read("row_ce")
    gemm_ms = sum(B.flce_timing_read(k)[0] for k in ("logits_gemm", "grad_x_gemm", "grad_w_gemm"))
    B.flce_timing_reset()
    # Two logits GEMMs and the two gradient products over the rows they run on
    # (the non-ignored ones when packed: the teacher here is as wide as the student).
    live = rows_through_products(B, y[:N])
    flops = 8.0 * live * H * V
    out = {
        "workload": f"JSD distillation, llama8b_head_bf16 student and a rolled teacher (N {N}, "
                    f"H {H}, V {V}, T 2, {cfg['reduction']})",
        "ms_per_call": ms, "tokens_per_s": N / (ms * 1e-3),
        "gemm_tflops": flops / (gemm_ms / reps * 1e-3) / 1e12,
        "jsd_row_kernel_ms_per_call": row_ms / reps,
        # bytes moved by the row kernel's three passes: 6 row reads + 1 write per element
        "jsd_row_kernel_GBps": 7.0 * live * ((V + 7) // 8 * 8) * 2 / (row_ms / reps * 1e-3) / 1e9,
        "loss": float(loss.item()),
    }
    del Xt, Wt, gW, ws
    torch.cuda.empty_cache()
    return out


def bench_dpo(torch, B, X, W, y, cfg, n_pairs=4, seq_len=1024, reps=3):
    """DPO at the 8B head's shape: the first 2 * n_pairs * seq_len token rows
    as n_pairs chosen and n_pairs rejected sequences, the first quarter of
    each sequence masked as prompt, synthetic reference log-probabilities
    (about what a uniform model gives the responses), beta 0.1."""
    N, H, V = 2 * n_pairs * seq_len, cfg["H"], cfg["V"]
    Xd = X[:N]
    yd = y[:N].clone()
    for k in range(2 * n_pairs):
        yd[k * seq_len:k * seq_len + seq_len // 4] = -100
    g = torch.Generator(device="cpu").manual_seed(0)
    ref = (torch.randn(2 * n_pairs, generator=g) * 3.0 - (3 * seq_len // 4) * float(np.log(V))).cuda()
    loss = torch.empty(1, device="cuda")
    gX = torch.empty(N, H, device="cuda")
    gW = torch.empty(V, H, device="cuda")
    ws = torch.empty(B.flce_dpo_workspace_bytes(n_pairs, seq_len, H, V, B.BF16), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        B.flce_dpo_forward_backward(Xd, W, yd, n_pairs, seq_len, ref, beta=0.1, grad_X=gX, grad_W=gW,
                                    pair_loss=False, loss=loss, workspace=ws, stream=stream)
    call()
    torch.cuda.synchronize()
    ms = time_calls(torch, stream, call, reps)
    hooked_pass(torch, B, call, reps)
    logit_ms, logit_n = B.flce_timing_read("logits_gemm")
    gemm_ms = logit_ms + sum(B.flce_timing_read(k)[0] for k in ("grad_x_gemm", "grad_w_gemm"))
    B.flce_timing_reset()
    chunk = B.flce_plan(N, H, V, B.BF16)[0]
    n_logits = logit_n / reps                      # logits GEMMs per call (1 or 2 per chunk)
    # Passes over the logits (1 with one chunk, else 2), each over the rows
    # that go through the products.
    flops = (4.0 + 2.0 * n_logits * chunk / N) * rows_through_products(B, yd) * H * V
    out = {
        "workload": f"DPO, {n_pairs} pairs x 2 x {seq_len} tokens over the llama8b_head_bf16 head "
                    f"(N {N}, H {H}, V {V}, beta 0.1, prompt quarter masked)",
        "ms_per_call": ms, "tokens_per_s": N / (ms * 1e-3),
        "logits_gemms_per_call": n_logits,
        "gemm_tflops": flops / (gemm_ms / reps * 1e-3) / 1e12,
        "loss": float(loss.item()),
    }
    del gW, ws
    torch.cuda.empty_cache()
    return out


def scratch_parts(B, N, H, V, dt, chunk_rows=0):
    """Bytes of each region of one FLCE call's workspace, from the library's
    own query: chunk logits / dlogits, grad_X K-split partials (which also
    hold the chunk's gathered hidden states when rows are packed), and the
    O(N) rest (header, per-row losses, packed-row lists)."""
    parts = B.flce_workspace_parts(N, H, V, dt, chunk_rows)
    parts["workspace"] = sum(parts.values())
    return parts


def one_chunk_bound_bytes(parts, N, V):
    """Peak extra memory allowed for one call: one chunk of logits, O((N + V)
    x 16) bytes of per-row and per-vocabulary scratch, and the split-K partials
    of the grad_X product."""
    return parts["chunk_logits"] + (N + V) * 16 + parts["split_partials"]


def rows_through_products(B, y):
    """Rows an FLCE call over targets y runs through its products: the
    non-ignored ones when row packing is on, else all."""
    packing = B.flce_set_row_packing(True)
    B.flce_set_row_packing(packing)
    return int((y != -100).sum().item()) if packing else int(y.numel())


def bench_grad16(torch, B, X, W, y, cfg, reps=5):
    """The same FLCE step with the gradients written in the input's 16-bit type
    (flce_forward_backward_ex): grad_W accumulated chunk by chunk in bf16."""
    N, H, V = cfg["N"], cfg["H"], cfg["V"]
    gX = torch.empty(N, H, dtype=X.dtype, device="cuda")
    gW = torch.empty(V, H, dtype=X.dtype, device="cuda")
    loss = torch.empty(1, device="cuda")
    ws = torch.empty(B.flce_workspace_bytes(N, H, V, B.BF16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        B.flce_forward_backward(X, W, y, reduction=cfg["reduction"], grad_X=gX, grad_W=gW,
                                grad_bias=False, loss=loss, workspace=ws, stream=stream,
                                grad_dtype="input")
    call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    live = rows_through_products(B, y)
    out = {
        "workload": "llama8b_head_bf16 with bf16 grad_X and grad_W",
        "ms_per_step": ms, "tokens_per_s": N / (ms * 1e-3),
        "rows_through_products": live,
        "frac_bf16_peak": 6.0 * live * H * V / (ms * 1e-3) / PEAK_BF16_FLOPS,
        "gradient_output_bytes": (N * H + V * H) * 2, "float32_gradient_output_bytes": (N * H + V * H) * 4,
        "loss": float(loss.item()),
    }
    del gX, gW, ws
    return out


def bench_multihead(torch, B, X, W, y, cfg, K=5, n_rows=None, reps=3):
    """K LM heads over shared hidden states (the liger README's Medusa example:
    5 heads) at the 8B head's shape, on all its token rows by default (the
    headline step's rows, so each head's work matches one headline step).
    Head k's weight is the workload's W rolled by 7k rows and its targets are
    the targets shifted by k positions (a head predicting further ahead); all
    on the device, no new host draws. GEMM work per call: K x 6 x n x H x V
    flop."""
    N, H, V = n_rows or cfg["N"], cfg["H"], cfg["V"]
    Xm = X[:N]
    Wk = torch.stack([torch.roll(W, shifts=7 * k, dims=0) for k in range(K)]).contiguous()
    yk = torch.stack([torch.roll(y[:N], shifts=-k) for k in range(K)]).contiguous()
    loss = torch.empty(K, device="cuda")
    gX = torch.empty(N, H, device="cuda")
    gW = torch.empty(K, V, H, device="cuda")
    ws = torch.empty(B.flce_multihead_workspace_bytes(N, H, V, K, B.BF16), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        B.flce_multihead_forward_backward(Xm, Wk, yk, reduction=cfg["reduction"], grad_X=gX,
                                          grad_W=gW, grad_bias=False, loss=loss, workspace=ws,
                                          stream=stream)
    call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    # Each head runs over its own non-ignored rows (when packing is on).
    flops = sum(rows_through_products(B, yk[k]) for k in range(K)) * 6.0 * H * V
    # The same rows through one head alone (head 0 in a single-head call), for
    # the per-head comparison at this N.
    del ws
    gW1 = gW[0]
    ws1 = torch.empty(B.flce_workspace_bytes(N, H, V, B.BF16), dtype=torch.uint8, device="cuda")
    l1 = torch.empty(1, device="cuda")

    def one():
        B.flce_forward_backward(Xm, Wk[0], yk[0], reduction=cfg["reduction"], grad_X=gX, grad_W=gW1,
                                grad_bias=False, loss=l1, workspace=ws1, stream=stream)
    one()
    torch.cuda.synchronize()
    ms1 = time_calls(torch, stream, one, reps)
    f1 = rows_through_products(B, yk[0]) * 6.0 * H * V
    out = {
        "workload": f"{K} heads over llama8b_head_bf16 hidden states (N {N}, H {H}, V {V}, "
                    f"{cfg['reduction']})",
        "ms_per_call": ms, "tokens_per_s": N / (ms * 1e-3),
        "tflops": flops / (ms * 1e-3) / 1e12, "frac_bf16_peak": flops / (ms * 1e-3) / PEAK_BF16_FLOPS,
        "single_head_same_rows": {"ms_per_call": ms1,
                                  "frac_bf16_peak": f1 / (ms1 * 1e-3) / PEAK_BF16_FLOPS},
        "head_losses": [float(v) for v in loss.cpu()],
    }
    del Wk, gW, ws1
    return out


def kernel_table(B, n_live, H, V, e, steps, step_ms):
    """Per-class kernel times from the library's HIP-event hooks (read after
    `steps` hooked steps): ms per launch, and for the GEMMs and the row CE the
    algorithmic work per launch (2 x rows x H x V flop; 2 x rows x V x e bytes)
    over that time against the MI355X peak."""
    gemm_flops_per_step = 2.0 * n_live * H * V
    kernels = {}
    for kind in ("logits_gemm", "grad_x_gemm", "grad_w_gemm", "row_ce", "other"):
        tot_ms, launches = B.flce_timing_read(kind)
        if launches == 0:
            continue
        entry = {"ms_per_launch": tot_ms / launches, "launches": launches}
        if kind.endswith("gemm"):
            per_launch = gemm_flops_per_step * steps / launches
            entry.update(bound="mfma", unit="TFLOP/s", algorithmic_per_launch=per_launch,
                         achieved=per_launch / (tot_ms / launches * 1e-3) / 1e12,
                         peak=PEAK_BF16_FLOPS / 1e12)
        elif kind == "row_ce":
            per_launch = 2.0 * n_live * V * e * steps / launches
            entry.update(bound="hbm", unit="GB/s", algorithmic_per_launch=per_launch,
                         achieved=per_launch / (tot_ms / launches * 1e-3) / 1e9,
                         peak=PEAK_HBM_BYTES / 1e9)
        if "achieved" in entry:
            entry["frac"] = entry["achieved"] / entry["peak"]
        entry["share_of_step"] = tot_ms / steps / step_ms
        kernels[kind] = entry
    B.flce_timing_reset()
    return kernels


def measure_flce(torch, B, cfg, inp, dev, steps, warmup, chunk_rows=0, packing=True,
                 hook_steps=None):
    """Times `steps` FLCE steps of one workload (inputs resident on the GPU,
    hooks off), then `hook_steps` more with the per-kernel HIP-event hooks on
    (a separate pass, so the hooks' event records stay out of the headline).
    Returns step times, executed-flop fractions, the kernel table, the peak
    extra device memory against the one-chunk bound, and the loss."""
    X, W, bias, y = dev
    N, H, V = cfg["N"], cfg["H"], cfg["V"]
    dt = B.BF16 if cfg["dtype"] == "bf16" else (B.F16 if cfg["dtype"] == "f16" else B.F32)
    e = 4 if dt == B.F32 else 2
    packing = packing and dt != B.F32
    B.flce_set_row_packing(packing)
    chunk, splits = B.flce_plan(N, H, V, dt, chunk_rows)
    n_live = int(np.count_nonzero(inp["targets"] != -100)) if packing else N
    parts = scratch_parts(B, N, H, V, dt, chunk_rows)
    loss = torch.empty((1,), dtype=torch.float32, device="cuda")
    gX = torch.empty((N, H), dtype=torch.float32, device="cuda")
    gW = torch.empty((V, H), dtype=torch.float32, device="cuda")
    gb = torch.empty((V,), dtype=torch.float32, device="cuda") if bias is not None else None
    torch.cuda.synchronize()
    io_bytes = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ws = torch.empty((parts["workspace"],), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        B.flce_forward_backward(X, W, y, bias=bias, reduction=cfg["reduction"], grad_X=gX,
                                grad_W=gW, grad_bias=gb, loss=loss, workspace=ws,
                                chunk_rows=chunk_rows, stream=stream)

    first = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for i in range(warmup):
        if i == 0:
            first[0].record(stream)
        step()
        if i == 0:
            first[1].record(stream)
    torch.cuda.synchronize()
    first_call_ms = first[0].elapsed_time(first[1]) if warmup > 0 else None
    if B.flce_check_device_error(ws) != B.OK:
        sys.exit("device reported an out-of-range target")
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(steps):
        step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = marks[0].elapsed_time(marks[steps]) / steps
    per_step = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
    peak = torch.cuda.max_memory_allocated()
    hook_steps = steps if hook_steps is None else hook_steps
    B.flce_timing_reset()
    B.flce_timing_enable(True)
    hm = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    hm[0].record(stream)
    for _ in range(hook_steps):
        step()
    hm[1].record(stream)
    torch.cuda.synchronize()
    B.flce_timing_enable(False)
    hooked_ms = hm[0].elapsed_time(hm[1]) / hook_steps
    kernels = kernel_table(B, n_live, H, V, e, hook_steps, hooked_ms)
    step_flops = 6.0 * n_live * H * V
    extra = peak - io_bytes
    bound = one_chunk_bound_bytes(parts, N, V)
    out = {
        "N": N, "H": H, "V": V, "reduction": cfg["reduction"], "bias": bias is not None,
        "chunk_rows": chunk, "dx_splits": splits, "row_packing": packing,
        "rows_through_products": n_live,
        "ms_per_step": ms, "tokens_per_s": N / (ms * 1e-3),
        "step_ms_median": float(np.median(per_step)), "step_ms_min": float(np.min(per_step)),
        "first_call_ms": first_call_ms,
        # Executed work: 6 x rows_through_products x H x V flops per step.
        "mfma_frac_step": step_flops / (ms * 1e-3) / PEAK_BF16_FLOPS,
        "step_tflops": step_flops / (ms * 1e-3) / 1e12,
        # 6 N H V over the step time: counts the ignored rows' products, which
        # packing does not run, so it is not a measure of MFMA use.
        "nominal_6NHV_frac_step": 6.0 * N * H * V / (ms * 1e-3) / PEAK_BF16_FLOPS,
        "peak_bytes": peak, "extra_bytes": extra,
        "workspace_parts": parts,
        "chunk_logits_bytes": parts["chunk_logits"],
        "extra_over_chunk_logits": extra / parts["chunk_logits"],
        # one chunk of logits + (N + V) x 16 bytes + the split-K partials
        "extra_bound_bytes": bound,
        "extra_within_bound": extra <= bound,
        "materialised_logits_bytes": N * V * e,
        "hooked_ms_per_step": hooked_ms, "hooked_steps": hook_steps,
        "kernels": kernels,
        "loss": float(loss.item()),
    }
    del ws, gX, gW, gb
    torch.cuda.empty_cache()
    return out


def other_config(torch, B, name, steps=5, warmup=2):
    """One of the other full-size FLCE workloads (its own inputs), timed like
    the headline with fewer steps."""
    from linear_cross_entropy_03_amd import synth
    cfg = dict(synth.WORKLOADS[name])
    t0 = time.time()
    inp = synth.make_workload(name)
    log(f"{name}: inputs ready in {time.time() - t0:.1f}s")
    dev = gpu_inputs(torch, inp)
    out = measure_flce(torch, B, cfg, inp, dev, steps, warmup, hook_steps=3)
    out["workload"] = name
    del dev
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.traffic_from:
        summarise_traffic(args.workload, *args.traffic_from)
        return
    if args.counters_from:
        summarise_counters(args.workload, args.counters_from)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1"}))
        sys.exit(2)

    import torch

    from linear_cross_entropy_03_amd import binding as B
    from linear_cross_entropy_03_amd import synth

    cfg = dict(synth.WORKLOADS[args.workload])
    if cfg["kind"] != "flce":
        sys.exit("bench workload must be an FLCE workload")
    N, H, V = cfg["N"], cfg["H"], cfg["V"]
    dt = B.BF16 if cfg["dtype"] == "bf16" else B.F32
    torch.cuda.set_device(0)
    if args.profile_step:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        torch.empty_like(a).copy_(a)  # 1 GiB read + 1 GiB write: counter calibration
        torch.cuda.synchronize()
        del a
    log(f"generating {args.workload}: N={N} H={H} V={V} {cfg['dtype']}")
    t0 = time.time()
    inp = synth.make_workload(args.workload)
    log(f"inputs ready in {time.time() - t0:.1f}s; uploading")
    X, W, bias, y = gpu_inputs(torch, inp)
    packing = dt != B.F32 and not args.no_packing

    if args.profile_step:
        B.flce_set_row_packing(packing)
        ws = torch.empty((B.flce_workspace_bytes(N, H, V, dt, args.chunk_rows),), dtype=torch.uint8,
                         device="cuda")
        gX = torch.empty((N, H), device="cuda")
        gW = torch.empty((V, H), device="cuda")
        gb = torch.empty((V,), device="cuda") if bias is not None else None
        for _ in range(2):
            B.flce_forward_backward(X, W, y, bias=bias, reduction=cfg["reduction"], grad_X=gX,
                                    grad_W=gW, grad_bias=gb, workspace=ws,
                                    chunk_rows=args.chunk_rows)
        torch.cuda.synchronize()
        log("profile step done")
        return

    chunk, splits = B.flce_plan(N, H, V, dt, args.chunk_rows)
    log(f"plan: chunk_rows={chunk} dx_splits={splits}; {args.warmup} warmup, {args.steps} timed steps")
    head = measure_flce(torch, B, cfg, inp, (X, W, bias, y), args.steps, args.warmup,
                        chunk_rows=args.chunk_rows, packing=packing)
    ms = head["ms_per_step"]
    kernels = head["kernels"]
    dom_kind = max((k for k in kernels if "achieved" in kernels[k]),
                   key=lambda k: kernels[k]["ms_per_launch"] * kernels[k]["launches"])
    dom = kernels[dom_kind]
    traffic = load_traffic(args.workload)
    t_dom = None
    if traffic is not None:
        for kind, entry in kernels.items():
            if kind in traffic["kernels"]:
                entry["traffic_bytes_per_launch"] = traffic["kernels"][kind]["traffic_bytes"]
        t_dom = traffic["kernels"].get(dom_kind, {}).get("traffic_bytes")
    roofline = {"kernel": dom_kind, "bound": dom["bound"], "achieved": dom["achieved"],
                "peak": dom["peak"], "unit": dom["unit"], "frac": dom["frac"], "traffic": t_dom,
                "algorithmic_per_launch": dom["algorithmic_per_launch"],
                "timing": "HIP events around each launch on the library's stream, "
                          f"over {head['hooked_steps']} steps timed after the headline's"}

    unpacked = None
    if packing and not args.no_unpacked:
        log("comparison: row packing off")
        u = measure_flce(torch, B, cfg, inp, (X, W, bias, y), 5, 1, chunk_rows=args.chunk_rows,
                         packing=False, hook_steps=1)
        B.flce_set_row_packing(packing)
        unpacked = {k: u[k] for k in ("ms_per_step", "tokens_per_s", "mfma_frac_step")}
    result = {
        "metric": "FLCE fwd+bwd tokens/s + % bf16 MFMA peak at H4096 V128256; peak HBM bytes",
        "value": head["tokens_per_s"],
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
                   "row_packing": packing,
                   "parallelism": "single GPU"},
        "roofline": roofline,
    }
    for k in ("rows_through_products", "step_ms_median", "step_ms_min", "first_call_ms",
              "mfma_frac_step", "step_tflops", "nominal_6NHV_frac_step", "peak_bytes", "extra_bytes",
              "extra_bound_bytes", "extra_within_bound", "extra_over_chunk_logits",
              "chunk_logits_bytes", "workspace_parts", "materialised_logits_bytes",
              "hooked_ms_per_step", "kernels", "loss"):
        result[k] = head[k]
    result["unpacked"] = unpacked
    if not args.no_vp:
        log("vocabulary-parallel shard")
        result["vocab_parallel"] = bench_vocab_parallel(torch, B, X, W, y, cfg)
    if not args.no_eager:
        log("PyTorch eager context")
        result["torch_eager_context"] = bench_torch_eager(torch, X, W, y, cfg)
    if not args.no_distill:
        log("distillation")
        result["distill"] = bench_distill(torch, B, X, W, y, cfg)
    if not args.no_dpo:
        log("DPO")
        result["dpo"] = bench_dpo(torch, B, X, W, y, cfg)
    if not args.no_g16:
        log("16-bit gradients")
        result["grad16"] = bench_grad16(torch, B, X, W, y, cfg)
    if not args.no_mh:
        log("multi-head")
        result["multihead"] = bench_multihead(torch, B, X, W, y, cfg)
    if not args.no_ce:
        log("standalone CE")
        result["ce"] = bench_ce(torch, B)
    del X, W, bias, y
    torch.cuda.empty_cache()
    if not args.no_configs:
        for key, name in (("c3", "llama1b_head_bf16"), ("c5", "vocab256k_bias_bf16")):
            log(f"full-size workload {name}")
            result[key] = other_config(torch, B, name)
    if not args.no_cpu_baseline:
        log("timing the FP64 oracle on a CPU sample")
        result["cpu_baseline"] = cpu_baseline(inp, cfg, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
