"""Writes the FP64 oracle's expected values for the full-size FLCE workloads
into tests/golden/fullsize_<workload>.npz.

Calls only the oracle (oracle/flce_oracle.py) on the seeded synthetic inputs
of linear_cross_entropy_03_amd/synth.py; nothing here comes from the HIP
library. Per workload it stores every row's loss, the reduced loss, grad_X
for 256 token rows and grad_W (and grad_bias) for 64 vocabulary rows, plus a
SHA-256 of each input array so a test can tell that it regenerated the same
inputs.

Workloads (the shapes of the pages' examples: a Llama-3.2-1B head, a
Llama-3-8B head at batch 8 x seq 4096, a 256k vocabulary at the same token
count, the torchtune blog's Figure 1 example):
  llama1b_head_bf16, llama1b_head_f16   N 8192,  H 2048, V 128256, mean
  llama8b_head_bf16                     N 32768, H 4096, V 128256, mean, Zipf targets
  vocab256k_bias_bf16                   N 32768, H 4096, V 256000, sum, bias

Run from the repository root (about 10 minutes on 8 cores, ~20 GB of RAM):
    python tests/golden/make_fullsize_golden.py [workload ...]
"""

import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from linear_cross_entropy_03_amd import synth  # noqa: E402
from oracle import flce_oracle as O  # noqa: E402

WORKLOADS = ["llama1b_head_bf16", "llama1b_head_f16", "llama8b_head_bf16", "vocab256k_bias_bf16"]
N_TOKEN_ROWS = 256
N_VOCAB_ROWS = 64


def input_digest(arr):
    """SHA-256 of an input array's bytes (None for an absent array)."""
    if arr is None:
        return ""
    return hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest()


def sample_rows(inp, seed=2024):
    """Token rows: first, last, two ignored rows, two rows of the most
    frequent target, the rest uniform. Vocabulary rows: the most frequent
    target, a target-free row, the first and last ids, the rest uniform."""
    N, V = inp["N"], inp["V"]
    y = inp["targets"]
    valid = y != inp["ignore_index"]
    counts = np.bincount(y[valid], minlength=V)
    top = int(counts.argmax())
    rng = np.random.default_rng(seed)
    fixed_t = np.unique(np.concatenate([[0, N - 1], np.flatnonzero(~valid)[:2],
                                        np.flatnonzero(y == top)[:2]]))
    rest_t = rng.choice(np.setdiff1d(np.arange(N), fixed_t), N_TOKEN_ROWS - len(fixed_t),
                        replace=False)
    fixed_v = np.unique(np.array([top, int(np.flatnonzero(counts == 0)[0]), 0, V - 1]))
    rest_v = rng.choice(np.setdiff1d(np.arange(V), fixed_v), N_VOCAB_ROWS - len(fixed_v),
                        replace=False)
    return np.sort(np.concatenate([fixed_t, rest_t])), np.sort(np.concatenate([fixed_v, rest_v]))


def make(name):
    cfg = synth.WORKLOADS[name]
    t0 = time.perf_counter()
    inp = synth.make_workload(name)
    trows, vrows = sample_rows(inp)
    f64 = lambda a: None if a is None else np.asarray(a, dtype=np.float64)
    loss, rows, gx, gw, gb, n_valid = O.flce_sampled(
        f64(inp["X_f32"]), f64(inp["W_f32"]), inp["targets"], trows, vrows,
        bias=f64(inp["bias_f32"]), ignore_index=inp["ignore_index"], reduction=cfg["reduction"])
    out = os.path.join(HERE, f"fullsize_{name}.npz")
    np.savez(out, workload=name, reduction=cfg["reduction"], N=inp["N"], H=inp["H"], V=inp["V"],
             loss=np.float64(loss), loss_rows=rows, n_valid=n_valid,
             token_rows=trows, grad_X_rows=gx.astype(np.float32),
             vocab_rows=vrows, grad_W_rows=gw.astype(np.float32),
             grad_bias_rows=(np.zeros(0) if gb is None else gb),
             sha_X=input_digest(inp["X"]), sha_W=input_digest(inp["W"]),
             sha_bias=input_digest(inp["bias"]), sha_targets=input_digest(inp["targets"]))
    print(f"{name}: loss {loss!r}, n_valid {n_valid}, {time.perf_counter() - t0:.0f} s -> {out}",
          flush=True)


if __name__ == "__main__":
    for w in (sys.argv[1:] or WORKLOADS):
        make(w)
