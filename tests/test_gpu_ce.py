"""GPU parity: standalone cross-entropy and vocabulary-shard statistics
(through the C ABI) against the FP64 oracle."""

import numpy as np
import pytest

from gpu_util import TOL, check_max_rel, check_scalar, say, to_dev, to_host, torch_or_skip
from linear_cross_entropy_03_amd import synth
from oracle import flce_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    torch_or_skip()
    from linear_cross_entropy_03_amd import binding
    binding.lib()
    return binding


def _run_ce(B, inp, reduction, mode="out"):
    import torch
    dt = inp["dtype"]
    logits = to_dev(inp["logits"], dt)
    y = to_dev(inp["targets"], "i32")
    before = logits.clone()
    if mode == "inplace":
        loss, g = B.ce_forward_backward(logits, y, reduction=reduction, grad_logits=logits)
    elif mode == "lossonly":
        loss, g = B.ce_forward_backward(logits, y, reduction=reduction, grad_logits=False)
    else:
        loss, g = B.ce_forward_backward(logits, y, reduction=reduction)
    torch.cuda.synchronize()
    unchanged = bool(torch.equal(before.view(torch.int16) if dt == "bf16" else before,
                                 logits.view(torch.int16) if dt == "bf16" else logits))
    return to_host(loss), to_host(g), unchanged, g


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_ce_shard_shape_bf16(B, reduction):
    """[1024, 32768] bf16 logits ~ N(0, 2), 5% ignored (one vocabulary shard's size)."""
    inp = synth.make_ce_inputs(1024, 32768, "bf16", std=2.0, ignore_frac=0.05)
    say("ce bf16 1024x32768", reduction)
    loss, g, unchanged, _ = _run_ce(B, inp, reduction)
    ref_loss, ref_g, info = O.cross_entropy(inp["logits_f32"], inp["targets"], reduction=reduction)
    t = TOL["bf16"]
    if reduction == "none":
        check_max_rel(loss, ref_loss, t["loss"], "loss rows")
        ign = inp["targets"] == -100
        assert np.all(loss[ign] == 0.0)
    else:
        check_scalar(loss, ref_loss, t["loss"])
    check_max_rel(g, ref_g, t["grad"], "grad_logits")
    assert unchanged, "out-of-place CE modified its input logits"
    ign = inp["targets"] == -100
    assert np.all(g[ign] == 0.0)


def test_ce_inplace_equals_out_of_place(B):
    inp = synth.make_ce_inputs(512, 32768, "bf16", std=2.0, seed=3)
    say("ce bf16 in-place vs out-of-place")
    l1, g1, _, _ = _run_ce(B, inp, "mean")
    l2, g2, _, _ = _run_ce(B, inp, "mean", mode="inplace")
    l3, _, unchanged, g3 = _run_ce(B, inp, "mean", mode="lossonly")
    assert g3 is None and unchanged
    assert np.array_equal(l1, l2) and np.array_equal(l1, l3)
    assert np.array_equal(g1, g2)


@pytest.mark.parametrize("N,V", [(37, 1000), (5, 7), (64, 70001)])
def test_ce_f32_ragged(B, N, V):
    """fp32 rows whose starts are not 16-byte aligned (V % 4 != 0)."""
    inp = synth.make_ce_inputs(N, V, "f32", std=3.0, ignore_frac=0.2, seed=N)
    say("ce f32", N, V)
    for red in ("none", "sum", "mean"):
        loss, g, unchanged, _ = _run_ce(B, inp, red)
        ref_loss, ref_g, _ = O.cross_entropy(inp["logits_f32"], inp["targets"], reduction=red)
        t = TOL["f32"]
        if red == "none":
            check_max_rel(loss, ref_loss, t["loss"], "loss rows")
        else:
            check_scalar(loss, ref_loss, t["loss"])
        check_max_rel(g, ref_g, t["grad"], "grad_logits")
        assert unchanged


@pytest.mark.parametrize("V", [1003, 8, 300001])
def test_ce_bf16_ragged_and_streaming(B, V):
    """Odd V (misaligned rows) and V beyond the register-resident limit."""
    N = 24 if V > 100000 else 129
    inp = synth.make_ce_inputs(N, V, "bf16", std=2.0, ignore_frac=0.1, seed=V)
    say("ce bf16", N, V)
    loss, g, _, _ = _run_ce(B, inp, "sum")
    ref_loss, ref_g, _ = O.cross_entropy(inp["logits_f32"], inp["targets"], reduction="sum")
    check_scalar(loss, ref_loss, TOL["bf16"]["loss"])
    check_max_rel(g, ref_g, TOL["bf16"]["grad"], "grad_logits")


@pytest.mark.parametrize("dtype,V", [("bf16", 262147), ("f32", 140003)])
def test_ce_streaming_rows_in_place(B, dtype, V):
    """Rows beyond the register-resident limit (two streaming passes in
    batches of vectors), misaligned row starts, gradient over the logits."""
    N = 40
    inp = synth.make_ce_inputs(N, V, dtype, std=2.0, ignore_frac=0.1, seed=V % 997)
    say("ce streaming in place", dtype, N, V)
    loss, g, _, _ = _run_ce(B, inp, "mean", mode="inplace")
    ref_loss, ref_g, _ = O.cross_entropy(inp["logits_f32"], inp["targets"], reduction="mean")
    check_scalar(loss, ref_loss, TOL[dtype]["loss"])
    check_max_rel(g, ref_g, TOL[dtype]["grad"], "grad_logits")


@pytest.mark.parametrize("V", [1003, 300001])
def test_ce_f16(B, V):
    """Half-precision logits: register-resident and streaming rows."""
    N = 24 if V > 100000 else 129
    inp = synth.make_ce_inputs(N, V, "f16", std=2.0, ignore_frac=0.1, seed=V + 1)
    say("ce f16", N, V)
    loss, g, _, _ = _run_ce(B, inp, "mean")
    ref_loss, ref_g, _ = O.cross_entropy(inp["logits_f32"], inp["targets"], reduction="mean")
    check_scalar(loss, ref_loss, TOL["f16"]["loss"])
    check_max_rel(g, ref_g, TOL["f16"]["grad"], "grad_logits")


@pytest.mark.parametrize("dtype,N,V,mode,reduction", [
    ("bf16", 1023, 16389, "out", "mean"),      # odd rows (a last workgroup with one row), misaligned rows
    ("f16", 2047, 16384, "inplace", "none"),   # 4 vectors per lane, every target counted in-kernel
    ("bf16", 2048, 32768, "inplace", "sum")])  # the self-count limit, 8 vectors per lane
def test_ce_two_rows_per_workgroup(B, dtype, N, V, mode, reduction):
    """Standalone calls of up to 2048 rows of 16384-32768 16-bit logits run
    two rows per workgroup: odd row counts, rows that do not start on 16
    bytes, bad targets in the last two rows (one of them alone in its
    workgroup when N is odd) and ignored rows, in place and out of place,
    against the oracle; the device error report sees the bad targets."""
    import torch
    inp = synth.make_ce_inputs(N, V, dtype, std=2.0, ignore_frac=0.1, seed=N + V)
    y = inp["targets"].copy()
    y[N - 1] = V
    y[N - 2] = -7
    inp = dict(inp, targets=y)
    ws = torch.zeros(B.ce_workspace_bytes(N, V), dtype=torch.uint8, device="cuda")
    logits = to_dev(inp["logits"], dtype)
    say("ce two rows per workgroup", dtype, N, V, mode, reduction)
    g_arg = logits if mode == "inplace" else True
    loss, g = B.ce_forward_backward(logits, to_dev(y, "i32"), reduction=reduction, grad_logits=g_arg,
                                    workspace=ws)
    assert B.flce_check_device_error(ws) == B.E_TARGET
    ref_loss, ref_g, info = O.cross_entropy(inp["logits_f32"], y, reduction=reduction)
    assert info["n_bad"] == 2
    t = TOL[dtype]
    if reduction == "none":
        l = to_host(loss)
        assert l[N - 1] == 0.0 and l[N - 2] == 0.0
        check_max_rel(l, ref_loss, t["loss"], "loss rows")
    else:
        check_scalar(to_host(loss), ref_loss, t["loss"])
    gh = to_host(g)
    assert np.all(gh[N - 1] == 0.0) and np.all(gh[N - 2] == 0.0)
    assert np.all(gh[y == -100] == 0.0)
    check_max_rel(gh, ref_g, t["grad"], "grad")


def test_ce_all_ignored_and_empty(B):
    import torch
    inp = synth.make_ce_inputs(16, 100, "f32", ignore_frac=1.0)
    say("ce all ignored")
    loss, g, _, _ = _run_ce(B, inp, "mean")
    assert float(loss[0]) == 0.0 and np.all(g == 0.0)
    z = torch.empty((0, 100), dtype=torch.float32, device="cuda")
    y = torch.empty((0,), dtype=torch.int32, device="cuda")
    for red in ("sum", "mean"):
        l0, _ = B.ce_forward_backward(z, y, reduction=red, grad_logits=False)
        torch.cuda.synchronize()
        assert float(l0.item()) == 0.0


def test_ce_bad_target_is_reported_and_ignored(B):
    import torch
    inp = synth.make_ce_inputs(32, 500, "f32", ignore_frac=0.0, seed=9)
    y = inp["targets"].copy()
    y[3] = 500
    y[7] = -5
    logits = to_dev(inp["logits"], "f32")
    ws = torch.zeros(B.ce_workspace_bytes(32, 500), dtype=torch.uint8, device="cuda")
    say("ce bad targets")
    loss, g = B.ce_forward_backward(logits, to_dev(y, "i32"), reduction="none", workspace=ws)
    assert B.flce_check_device_error(ws) == B.E_TARGET
    ref_loss, ref_g, info = O.cross_entropy(inp["logits_f32"], y, reduction="none")
    assert info["n_bad"] == 2
    l = to_host(loss)
    assert l[3] == 0.0 and l[7] == 0.0
    check_max_rel(l, ref_loss, TOL["f32"]["loss"], "loss rows")
    check_max_rel(to_host(g), ref_g, TOL["f32"]["grad"], "grad")
    # A clean call on the same workspace clears the report.
    B.ce_forward_backward(logits, to_dev(inp["targets"], "i32"), reduction="none", workspace=ws)
    assert B.flce_check_device_error(ws) == B.OK


@pytest.mark.parametrize("N", [2048, 2049])
def test_ce_target_count_paths(B, N):
    """Calls of up to 2048 rows count their targets inside the row kernel,
    larger ones in a separate launch: both give the mean over valid rows and
    report a bad target."""
    import torch
    inp = synth.make_ce_inputs(N, 777, "bf16", std=2.0, ignore_frac=0.3, seed=N)
    y = inp["targets"].copy()
    y[N - 1] = 777
    ws = torch.zeros(B.ce_workspace_bytes(N, 777), dtype=torch.uint8, device="cuda")
    say("ce count paths", N)
    loss, g = B.ce_forward_backward(to_dev(inp["logits"], "bf16"), to_dev(y, "i32"),
                                    reduction="mean", workspace=ws)
    assert B.flce_check_device_error(ws) == B.E_TARGET
    ref_loss, ref_g, info = O.cross_entropy(inp["logits_f32"], y, reduction="mean")
    assert info["n_bad"] == 1
    check_scalar(to_host(loss), ref_loss, TOL["bf16"]["loss"])
    check_max_rel(to_host(g), ref_g, TOL["bf16"]["grad"], "grad")


@pytest.mark.parametrize("N,Vl,dtype", [(64, 1000, "bf16"), (2049, 1000, "f32"), (8, 70001, "f16"),
                                        (8, 140001, "bf16")])
def test_shard_stats_bad_target_and_paths(B, N, Vl, dtype):
    """Shard statistics of shard [1000, 1000 + Vl) of a 3 * Vl vocabulary:
    register-resident (with the target count in the same launch up to 2048
    rows, a separate count above) and streaming rows; a target outside the
    global vocabulary is reported and a clean call clears the report."""
    import torch
    V = 3 * Vl
    inp = synth.make_ce_inputs(N, Vl, dtype, std=2.0, ignore_frac=0.2, seed=Vl + N)
    rng = np.random.default_rng(N)
    y = rng.integers(0, V, size=N).astype(np.int32)
    y[inp["targets"] == -100] = -100
    y[0] = V
    y[1] = 1000 + Vl // 2
    ws = torch.zeros(B.ce_workspace_bytes(N, V), dtype=torch.uint8, device="cuda")
    say("shard stats paths", N, Vl, dtype)
    m, s, t = B.ce_shard_stats(to_dev(inp["logits"], dtype), to_dev(y, "i32"), 1000, V, workspace=ws)
    assert B.flce_check_device_error(ws) == B.E_TARGET
    rm, rs, rt = O.shard_stats(inp["logits_f32"], y, 1000, V)
    assert np.array_equal(to_host(m), rm), "row max must be exact"
    check_max_rel(to_host(s), rs, 1e-5, "sumexp")
    assert np.array_equal(to_host(t), rt), "target logit must be exact"
    y[0] = -100
    B.ce_shard_stats(to_dev(inp["logits"], dtype), to_dev(y, "i32"), 1000, V, workspace=ws)
    assert B.flce_check_device_error(ws) == B.OK


def test_shard_stats_two_halves_combine(B):
    """[1024, 65536] bf16 logits split into vocabulary shards [0, 32768) and
    [32768, 65536); the host combination of the two shards' statistics equals
    the full-vocabulary logsumexp and target logit."""
    import torch
    inp = synth.make_ce_inputs(1024, 65536, "bf16", std=2.0, ignore_frac=0.05)
    full = to_dev(inp["logits"], "bf16")
    y = to_dev(inp["targets"], "i32")
    parts = []
    for v0 in (0, 32768):
        say("shard stats", v0)
        shard = full[:, v0:v0 + 32768].contiguous()
        m, s, t = B.ce_shard_stats(shard, y, v0, 65536)
        torch.cuda.synchronize()
        m, s, t = to_host(m), to_host(s), to_host(t)
        rm, rs, rt = O.shard_stats(inp["logits_f32"][:, v0:v0 + 32768], inp["targets"], v0, 65536)
        assert np.array_equal(m, rm), "row max must be exact"
        check_max_rel(s, rs, 1e-5, "sumexp")
        assert np.array_equal(t, rt), "target logit must be exact"
        parts.append((m, s, t))
    lse, zt = O.combine_shard_stats(parts)
    ref_lse = O.logsumexp_rows(inp["logits_f32"])
    check_max_rel(lse, ref_lse, 1e-6, "combined lse")
    valid = inp["targets"] != -100
    assert np.array_equal(zt[valid], inp["logits_f32"][np.arange(1024)[valid], inp["targets"][valid]])


@pytest.mark.parametrize("dtype,V,mode", [("bf16", 100003, "out"), ("f16", 100003, "inplace"),
                                          ("f32", 40001, "out"), ("bf16", 131072, "inplace")])
def test_ce_long_rows_persistent(B, dtype, V, mode):
    """Rows of 8193..16384 16-byte vectors with more rows than CUs take the
    persistent kernel that streams each workgroup's next row into LDS while
    the current one is reduced; odd V gives misaligned rows (head and tail
    elements) on every other row."""
    N = 600
    inp = synth.make_ce_inputs(N, V, dtype, std=2.0, ignore_frac=0.1, seed=V % 1000)
    say("ce long rows", dtype, N, V, mode)
    loss, g, unchanged, _ = _run_ce(B, inp, "mean", mode=mode)
    ref_loss, ref_g, _ = O.cross_entropy(inp["logits_f32"], inp["targets"], reduction="mean")
    check_scalar(loss, ref_loss, TOL[dtype]["loss"])
    check_max_rel(g, ref_g, TOL[dtype]["grad"], "grad_logits")
    if mode == "out":
        assert unchanged
