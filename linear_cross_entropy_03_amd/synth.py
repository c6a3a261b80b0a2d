"""Seeded synthetic inputs for FLCE / CE, shared by the tests, the smoke check
and the benchmark.

This module only draws data: it holds none of the loss arithmetic. Values are
drawn in float32 with numpy.random.default_rng(seed) in a fixed order (X, W,
bias, targets, ignored positions) and, for bf16 or fp16, rounded to the nearest
representable value (ties to even). Each array is returned twice: as the
storage the GPU receives (uint16 bit patterns for bf16 and fp16, float32 for
fp32) and as the exact float32 value of that storage, which the oracle upcasts
to float64.

Workload shapes follow the pages' workloads: a Llama-3.2-1B head (H 2048,
V 128256), a Llama-3-8B head at batch 8 x seq 4096 (H 4096, V 128256), a 256k
vocabulary at the same token count (the 16.8 GB logits example of the torchtune
blog, Figure 1), and a CE-only vocabulary shard of 32768 of 65536 at 1024 tokens
(DeepSpeed PR memory profile).
"""

import numpy as np

DTYPES = ("f32", "bf16", "f16")


def f32_to_bf16_bits(a):
    """Round float32 values to bf16, nearest-even; returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact float32 value of bf16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(values_f32, dtype):
    if dtype == "bf16":
        bits = f32_to_bf16_bits(values_f32)
        return bits, bf16_bits_to_f32(bits)
    if dtype == "f16":
        h = np.ascontiguousarray(values_f32, dtype=np.float32).astype(np.float16)  # nearest-even
        return h.view(np.uint16), h.astype(np.float32)
    if dtype == "f32":
        v = np.ascontiguousarray(values_f32, dtype=np.float32)
        return v, v
    raise ValueError(f"dtype must be one of {DTYPES}")


def _targets(rng, N, V, dist, zipf_s):
    if dist == "uniform":
        return rng.integers(0, V, size=N, dtype=np.int64)
    if dist == "zipf":
        # P(rank r) proportional to r**-s for r = 1..V; token id = r - 1,
        # sampled by inverse CDF.
        w = np.arange(1, V + 1, dtype=np.float64) ** (-float(zipf_s))
        cdf = np.cumsum(w)
        cdf /= cdf[-1]
        u = rng.random(N)
        return np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int64)
    raise ValueError("target distribution must be 'uniform' or 'zipf'")


def _ignore(rng, y, frac, ignore_index):
    N = y.shape[0]
    k = int(round(frac * N))
    if k > 0:
        pos = rng.choice(N, k, replace=False)
        y[pos] = ignore_index
    return y.astype(np.int32)


def make_flce_inputs(N, H, V, dtype="bf16", x_std=1.0, w_std=0.02, bias_std=None,
                     target_dist="uniform", zipf_s=1.1, ignore_frac=0.1,
                     ignore_index=-100, seed=0):
    """X [N,H] ~ N(0, x_std), W [V,H] ~ N(0, w_std), optional bias [V] ~
    N(0, bias_std), int32 targets with round(ignore_frac*N) rows ignored."""
    rng = np.random.default_rng(seed)
    X, Xf = _store(rng.standard_normal((N, H), dtype=np.float32) * np.float32(x_std), dtype)
    W, Wf = _store(rng.standard_normal((V, H), dtype=np.float32) * np.float32(w_std), dtype)
    b = bf = None
    if bias_std is not None:
        b, bf = _store(rng.standard_normal(V, dtype=np.float32) * np.float32(bias_std), dtype)
    y = _ignore(rng, _targets(rng, N, V, target_dist, zipf_s), ignore_frac, ignore_index)
    return {"N": N, "H": H, "V": V, "dtype": dtype, "ignore_index": ignore_index,
            "X": X, "X_f32": Xf, "W": W, "W_f32": Wf, "bias": b, "bias_f32": bf,
            "targets": y}


def make_ce_inputs(N, V, dtype="bf16", std=2.0, target_range=None, ignore_frac=0.05,
                   ignore_index=-100, seed=0):
    """Logits [N,V] ~ N(0, std); targets uniform in [0, target_range or V)."""
    rng = np.random.default_rng(seed)
    Z, Zf = _store(rng.standard_normal((N, V), dtype=np.float32) * np.float32(std), dtype)
    y = _ignore(rng, _targets(rng, N, target_range or V, "uniform", 0.0),
                ignore_frac, ignore_index)
    return {"N": N, "V": V, "dtype": dtype, "ignore_index": ignore_index,
            "logits": Z, "logits_f32": Zf, "targets": y}


# Named workloads. "reduction" is the one the workload is quoted with; tests
# run the others too.
WORKLOADS = {
    "tiny_f32": dict(kind="flce", N=256, H=64, V=1024, dtype="f32", reduction="mean",
                     ignore_frac=0.1),
    "ce_shard_bf16": dict(kind="ce", N=1024, V=32768, V_global=65536, dtype="bf16",
                          reduction="mean", std=2.0, ignore_frac=0.05),
    "llama1b_head_bf16": dict(kind="flce", N=8192, H=2048, V=128256, dtype="bf16",
                              reduction="mean", ignore_frac=0.1),
    "llama1b_head_f16": dict(kind="flce", N=8192, H=2048, V=128256, dtype="f16",
                             reduction="mean", ignore_frac=0.1),
    "llama8b_head_bf16": dict(kind="flce", N=32768, H=4096, V=128256, dtype="bf16",
                              reduction="mean", ignore_frac=0.1, target_dist="zipf"),
    "vocab256k_bias_bf16": dict(kind="flce", N=32768, H=4096, V=256000, dtype="bf16",
                                reduction="sum", ignore_frac=0.1, bias_std=0.01),
}


def make_workload(name, seed=0, **overrides):
    """Inputs for a named FLCE workload (overrides may shrink N for sampling)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    if cfg["kind"] != "flce":
        raise ValueError("use make_ce_inputs for the CE workload")
    return make_flce_inputs(cfg["N"], cfg["H"], cfg["V"], cfg["dtype"],
                            bias_std=cfg.get("bias_std"),
                            target_dist=cfg.get("target_dist", "uniform"),
                            ignore_frac=cfg.get("ignore_frac", 0.1), seed=seed)
