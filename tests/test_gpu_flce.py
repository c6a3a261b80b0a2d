"""GPU parity: fused linear cross-entropy (through the C ABI) against the FP64
oracle, element by element at sizes the oracle finishes in seconds (several
tiles, several chunks, ragged tails), plus invariants."""

import numpy as np
import pytest

from gpu_util import (TOL, check_max_rel, check_scalar, oracle_inputs, say, to_dev, to_host,
                      torch_or_skip)
from linear_cross_entropy_03_amd import synth
from oracle import flce_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    torch_or_skip()
    from linear_cross_entropy_03_amd import binding
    binding.lib()
    return binding


def run_flce(B, inp, reduction, chunk_rows=0, want=("X", "W", "bias")):
    import torch
    dt = inp["dtype"]
    X, W = to_dev(inp["X"], dt), to_dev(inp["W"], dt)
    b = to_dev(inp["bias"], dt)
    y = to_dev(inp["targets"], "i32")
    loss, gX, gW, gb = B.flce_forward_backward(
        X, W, y, bias=b, reduction=reduction, chunk_rows=chunk_rows,
        grad_X="X" in want, grad_W="W" in want, grad_bias=(b is not None and "bias" in want))
    torch.cuda.synchronize()
    return to_host(loss), to_host(gX), to_host(gW), to_host(gb)


def check_against_oracle(inp, reduction, got, want=("X", "W", "bias")):
    X, W, b, y = oracle_inputs(inp)
    ref_loss, ref_g, info = O.flce(X, W, y, bias=b, reduction=reduction)
    t = TOL[inp["dtype"]]
    loss, gX, gW, gb = got
    if reduction == "none":
        check_max_rel(loss, ref_loss, t["loss"], "loss rows")
        assert np.all(loss[y == -100] == 0.0), "ignored rows must have exact zero loss"
    else:
        check_scalar(loss, ref_loss, t["loss"])
    if "X" in want:
        check_max_rel(gX, ref_g["X"], t["grad"], "grad_X")
        assert np.all(gX[y == -100] == 0.0), "ignored rows must have exact zero grad_X"
    if "W" in want:
        check_max_rel(gW, ref_g["W"], t["grad"], "grad_W")
    if b is not None and "bias" in want:
        check_max_rel(gb, ref_g["bias"], t["grad"], "grad_bias")
    return ref_loss, ref_g


@pytest.mark.parametrize("reduction", ["mean", "none", "sum"])
def test_tiny_f32(B, reduction):
    """N 256, H 64, V 1024, fp32, 10% ignored."""
    inp = synth.make_flce_inputs(256, 64, 1024, "f32", ignore_frac=0.1)
    say("flce tiny f32", reduction)
    check_against_oracle(inp, reduction, run_flce(B, inp, reduction))


@pytest.mark.parametrize("chunk", [32, 64, 0])
def test_tiny_f32_forced_chunks(B, chunk):
    inp = synth.make_flce_inputs(256, 64, 1024, "f32", ignore_frac=0.1)
    say("flce tiny f32 chunk", chunk)
    check_against_oracle(inp, "mean", run_flce(B, inp, "mean", chunk_rows=chunk))


def test_f32_ragged_with_bias(B):
    inp = synth.make_flce_inputs(300, 72, 1000, "f32", bias_std=0.5, ignore_frac=0.15, seed=5)
    say("flce f32 ragged bias")
    check_against_oracle(inp, "sum", run_flce(B, inp, "sum", chunk_rows=128))


@pytest.mark.parametrize("chunk", [0, 256, 160])
@pytest.mark.parametrize("reduction", ["mean", "sum", "none"])
def test_bf16_ragged_tiles(B, reduction, chunk):
    """bf16, N 600 (3 row tiles), H 136 (K tail), V 1000 (V % 8 != 0), bias."""
    inp = synth.make_flce_inputs(600, 136, 1000, "bf16", bias_std=0.1, ignore_frac=0.1, seed=11)
    say("flce bf16 ragged", reduction, chunk)
    check_against_oracle(inp, reduction, run_flce(B, inp, reduction, chunk_rows=chunk))


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_f16_ragged_tiles_and_chunks(B, reduction):
    """IEEE half inputs (the fp16 MFMA path): N 600, H 136, V 1000, bias, 3
    chunks of 256/256/88 rows."""
    inp = synth.make_flce_inputs(600, 136, 1000, "f16", bias_std=0.1, ignore_frac=0.1, seed=14)
    say("flce f16 ragged", reduction)
    check_against_oracle(inp, reduction, run_flce(B, inp, reduction, chunk_rows=256))


@pytest.mark.parametrize("dtype,N,H,V,chunk", [
    ("bf16", 1000, 136, 4099, 256),      # 4 chunks: grad_W / grad_bias rounded at each add
    ("f16", 600, 136, 1000, 0),
    ("bf16", 512, 2048, 16384, 0)])      # split-K grad_X reduced in fp32, rounded once
def test_gradients_in_the_input_type(B, dtype, N, H, V, chunk):
    """flce_forward_backward_ex with 16-bit gradient outputs, against the
    oracle at the 16-bit bar, and against the float32-gradient call: each
    16-bit gradient is within a few roundings of the float32 one."""
    import torch
    inp = synth.make_flce_inputs(N, H, V, dtype, bias_std=0.1, ignore_frac=0.1, seed=N + V)
    X, W = to_dev(inp["X"], dtype), to_dev(inp["W"], dtype)
    b, y = to_dev(inp["bias"], dtype), to_dev(inp["targets"], "i32")
    say("flce 16-bit gradients", dtype, N, H, V, chunk)
    l16, gX16, gW16, gb16 = B.flce_forward_backward(X, W, y, bias=b, chunk_rows=chunk, grad_dtype="input")
    l32, gX32, gW32, gb32 = B.flce_forward_backward(X, W, y, bias=b, chunk_rows=chunk)
    torch.cuda.synchronize()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    assert gX16.dtype == tdt and gW16.dtype == tdt and gb16.dtype == tdt
    assert float(l16[0]) == float(l32[0])
    got = (to_host(l16), gX16.float().cpu().numpy(), gW16.float().cpu().numpy(),
           gb16.float().cpu().numpy())
    check_against_oracle(inp, "mean", got)
    chunks = -(-N // (chunk or B.flce_plan(N, H, V, B.BF16 if dtype == "bf16" else B.F16)[0]))
    ulp = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -11
    for g16, g32, name in ((gX16, gX32, "grad_X"), (gW16, gW32, "grad_W"), (gb16, gb32, "grad_bias")):
        a, r = g16.double().cpu().numpy(), g32.double().cpu().numpy()
        rounds = 1 if name == "grad_X" else chunks
        assert np.abs(a - r).max() <= rounds * ulp * np.abs(r).max() + 1e-30, name


def test_multihead_gradients_in_the_input_type(B):
    """Three bf16 heads with 16-bit gradients against the float32-gradient
    call: grad_X is summed over the heads in bf16 (one rounding per head),
    grad_W per head rounded once per chunk."""
    import torch
    K, N, H, V = 3, 700, 136, 1500
    inp = synth.make_flce_inputs(N, H, K * V, "bf16", ignore_frac=0.1, seed=33)
    X = to_dev(inp["X"], "bf16")
    W = to_dev(inp["W"], "bf16").reshape(K, V, H).contiguous()
    rng = np.random.default_rng(34)
    yk = rng.integers(0, V, size=(K, N)).astype(np.int32)
    yk[:, ::7] = -100
    y = to_dev(yk, "i32")
    say("multihead 16-bit gradients", K, N, H, V)
    l16, gX16, gW16, _ = B.flce_multihead_forward_backward(X, W, y, chunk_rows=256, grad_dtype="input")
    l32, gX32, gW32, _ = B.flce_multihead_forward_backward(X, W, y, chunk_rows=256)
    torch.cuda.synchronize()
    assert gX16.dtype == torch.bfloat16 and gW16.dtype == torch.bfloat16
    assert torch.equal(l16, l32)
    ulp = 2.0 ** -8
    for g16, g32, rounds in ((gX16, gX32, K), (gW16, gW32, 3)):
        a, r = g16.double().cpu().numpy(), g32.double().cpu().numpy()
        assert np.abs(a - r).max() <= rounds * ulp * np.abs(r).max()


def test_multihead_bad_target_reported(B):
    """A target outside [0, V) in the second of three heads is reported by
    flce_check_device_error for the multi-head call (its row is treated as
    ignored, so the losses match the oracle with that row ignored); the next
    call on the same workspace with clean targets reports OK."""
    import torch
    K, N, H, V = 3, 300, 64, 700
    inp = synth.make_flce_inputs(N, H, K * V, "bf16", ignore_frac=0.0, seed=37)
    X = to_dev(inp["X"], "bf16")
    W = to_dev(inp["W"], "bf16").reshape(K, V, H).contiguous()
    rng = np.random.default_rng(38)
    yk = rng.integers(0, V, size=(K, N)).astype(np.int32)
    bad = yk.copy()
    bad[1, 17] = V + 5
    ws = torch.empty(B.flce_multihead_workspace_bytes(N, H, V, K, B.BF16), dtype=torch.uint8,
                     device="cuda")
    ws.fill_(0xAB)  # stale contents must not leak into the report
    say("multihead bad target in head 1")
    loss, _, _, _ = B.flce_multihead_forward_backward(X, W, to_dev(bad, "i32"), workspace=ws,
                                                      reduction="sum")
    assert B.flce_check_device_error(ws) == B.E_TARGET
    Xf = np.asarray(inp["X_f32"], np.float64)
    Wf = np.asarray(inp["W_f32"], np.float64).reshape(K, V, H)
    ref, _ = O.flce_multihead(Xf, list(Wf), list(bad), reduction="sum")
    check_max_rel(to_host(loss), ref, TOL["bf16"]["loss"], "losses with a bad target")
    say("multihead clean targets, same workspace")
    B.flce_multihead_forward_backward(X, W, to_dev(yk, "i32"), workspace=ws, reduction="sum")
    assert B.flce_check_device_error(ws) == B.OK


def test_bf16_multi_chunk_mid(B):
    """N 1024 in 4 chunks, H 512, V 4099: the grad_W read-modify-write path."""
    inp = synth.make_flce_inputs(1024, 512, 4099, "bf16", ignore_frac=0.1, seed=12)
    say("flce bf16 mid 4 chunks")
    check_against_oracle(inp, "mean", run_flce(B, inp, "mean", chunk_rows=256))


def test_bf16_split_k_grad_x(B):
    """N 512, H 2048, V 16384: the planner splits grad_X's K over V."""
    c, s = B.flce_plan(512, 2048, 16384, B.BF16)
    assert s > 1
    inp = synth.make_flce_inputs(512, 2048, 16384, "bf16", ignore_frac=0.1, seed=13)
    say("flce bf16 split-K", c, s)
    check_against_oracle(inp, "mean", run_flce(B, inp, "mean"))


def test_bf16_zipf_targets_with_skipped_grads(B):
    inp = synth.make_flce_inputs(768, 256, 3000, "bf16", target_dist="zipf", seed=14)
    say("flce bf16 zipf, grad_X only")
    got = run_flce(B, inp, "mean", chunk_rows=256, want=("X",))
    assert got[2] is None
    check_against_oracle(inp, "mean", got, want=("X",))
    say("flce bf16 zipf, grad_W only")
    got = run_flce(B, inp, "mean", chunk_rows=256, want=("W",))
    check_against_oracle(inp, "mean", got, want=("W",))
    say("flce bf16 zipf, loss only")
    got = run_flce(B, inp, "mean", want=())
    check_against_oracle(inp, "mean", got, want=())


@pytest.mark.parametrize("pack", [True, False])
def test_loss_bitwise_independent_of_chunking_and_deterministic(packing, pack):
    """Per-row losses (hence the loss) are bitwise independent of the chunk
    size, with row packing on or off; unpacked, grad_X is bitwise equal
    whenever the grad_X K-split is the same (a different split only changes
    its rounding order; packed, the last chunk may split its K in two);
    repeated calls are bitwise identical."""
    B = packing
    B.flce_set_row_packing(pack)
    inp = synth.make_flce_inputs(1000, 256, 5000, "bf16", bias_std=0.02, seed=15)
    say("flce chunk independence, packing", pack)
    chunks = (0, 256, 512, 1000)
    runs = {c: run_flce(B, inp, "none", chunk_rows=c) for c in chunks}
    splits = {c: B.flce_plan(1000, 256, 5000, B.BF16, c)[1] for c in chunks}
    base = runs[1000]
    for c, r in runs.items():
        assert np.array_equal(r[0], base[0]), f"loss rows differ at chunk {c}"
        if splits[c] == splits[1000] and not pack:
            assert np.array_equal(r[1], base[1]), f"grad_X differs at chunk {c}"
        else:
            check_max_rel(r[1], base[1], 1e-5, f"grad_X chunk {c} vs 1000")
        check_max_rel(r[2], base[2], 1e-5, f"grad_W chunk {c} vs 1000")
        check_max_rel(r[3], base[3], 1e-5, f"grad_bias chunk {c} vs 1000")
    again = run_flce(B, inp, "none", chunk_rows=256)
    for a, b in zip(again, runs[256]):
        assert np.array_equal(a, b), "two identical calls differ"


def test_gradient_invariants_f32(B):
    """Each dlogits row sums to zero, so sum_v grad_W[v, :] = 0 and
    sum_v grad_bias[v] = 0 (fp32: up to fp32 rounding)."""
    inp = synth.make_flce_inputs(512, 128, 2048, "f32", bias_std=0.05, seed=16)
    say("flce invariants f32")
    loss, gX, gW, gb = run_flce(B, inp, "sum")
    assert np.abs(gW.sum(axis=0)).max() <= 1e-5 * np.abs(gW).max() * 2048 ** 0.5
    assert abs(gb.sum()) <= 1e-5 * np.abs(gb).max() * 2048 ** 0.5


def test_gradient_invariants_bf16(B):
    """With dlogits stored in bf16 each row sum is off by at most the rounding
    of its entries: at most 2**-9 for the target entry (|p - 1| < 1) plus
    2**-9 * sum_v p_v for the rest, i.e. 2**-8 per valid row in total."""
    inp = synth.make_flce_inputs(512, 128, 2048, "bf16", bias_std=0.05, seed=16)
    say("flce invariants bf16")
    loss, gX, gW, gb = run_flce(B, inp, "sum")
    n_valid = int((inp["targets"] != -100).sum())
    assert abs(gb.sum()) <= n_valid * 2.0 ** -8
    xmax = np.abs(np.asarray(inp["X_f32"], dtype=np.float64)).max()
    assert np.abs(gW.sum(axis=0)).max() <= n_valid * 2.0 ** -8 * xmax


def test_all_ignored_and_empty(B):
    import torch
    inp = synth.make_flce_inputs(64, 32, 100, "f32", ignore_frac=1.0)
    say("flce all ignored")
    loss, gX, gW, _ = run_flce(B, inp, "mean")
    assert float(loss[0]) == 0.0 and np.all(gX == 0) and np.all(gW == 0)
    X = torch.empty((0, 32), dtype=torch.float32, device="cuda")
    W = torch.randn((100, 32), dtype=torch.float32, device="cuda")
    y = torch.empty((0,), dtype=torch.int32, device="cuda")
    gW0 = torch.full((100, 32), 7.0, device="cuda")
    say("flce empty batch")
    l0, _, gW0, _ = B.flce_forward_backward(X, W, y, reduction="sum", grad_X=False, grad_W=gW0)
    torch.cuda.synchronize()
    assert float(l0.item()) == 0.0 and bool((gW0 == 0).all())


def test_bad_target_reported(B):
    import torch
    inp = synth.make_flce_inputs(40, 16, 50, "f32", ignore_frac=0.0, seed=17)
    y = inp["targets"].copy()
    y[5] = 77
    inp2 = dict(inp, targets=y)
    ws = torch.zeros(B.flce_workspace_bytes(40, 16, 50, B.F32), dtype=torch.uint8, device="cuda")
    say("flce bad target")
    loss, gX, gW, _ = B.flce_forward_backward(
        to_dev(inp["X"], "f32"), to_dev(inp["W"], "f32"), to_dev(y, "i32"), reduction="none",
        workspace=ws)
    assert B.flce_check_device_error(ws) == B.E_TARGET
    check_against_oracle(inp2, "none", (to_host(loss), to_host(gX), to_host(gW), None))


@pytest.fixture
def packing(B):
    """Restores the row-packing switch after a test that flips it."""
    was = B.flce_set_row_packing(True)
    yield B
    B.flce_set_row_packing(was)


def _flce_dev(B, inp, reduction, chunk, grad_dtype=None):
    import torch
    dt = inp["dtype"]
    X, W = to_dev(inp["X"], dt), to_dev(inp["W"], dt)
    b, y = to_dev(inp["bias"], dt), to_dev(inp["targets"], "i32")
    kw = {} if grad_dtype is None else {"grad_dtype": grad_dtype}
    out = B.flce_forward_backward(X, W, y, bias=b, reduction=reduction, chunk_rows=chunk, **kw)
    torch.cuda.synchronize()
    return tuple(None if t is None else t.double().cpu().numpy() for t in out)


@pytest.mark.parametrize("dtype,N,H,V,chunk,ignore,reduction,bias", [
    ("bf16", 1024, 136, 1000, 256, 0.6, "mean", True),   # packed rows fill 2 of 4 chunks
    ("bf16", 600, 136, 1000, 0, 0.1, "none", True),      # one chunk, ragged tiles
    ("bf16", 1000, 264, 4099, 128, 0.35, "sum", False),  # 8 chunks, a partial live tile
    ("f16", 700, 136, 1500, 256, 0.5, "mean", True),
    ("bf16", 512, 2048, 16384, 0, 0.3, "mean", False),   # split-K grad_X reduced through the map
])
def test_row_packing_against_oracle_and_unpacked(packing, dtype, N, H, V, chunk, ignore, reduction,
                                                 bias):
    """Packed chunk loop (ignored rows listed out on the device) against the
    FP64 oracle, and against the same call with packing off: the loss (every
    row for none) is bitwise equal, and so is grad_X outside the last chunk;
    the rest differ only in float32 summation order (the last chunk's K
    split, where chunk boundaries fall in the grad_W and grad_bias sums)."""
    B = packing
    inp = synth.make_flce_inputs(N, H, V, dtype, bias_std=0.1 if bias else 0.0,
                                 ignore_frac=ignore, seed=N + H)
    say("flce row packing", dtype, N, H, V, chunk, ignore, reduction)
    packed = _flce_dev(B, inp, reduction, chunk)
    check_against_oracle(inp, reduction, packed)
    B.flce_set_row_packing(False)
    say("flce row packing off", dtype, N, H, V, chunk, ignore, reduction)
    plain = _flce_dev(B, inp, reduction, chunk)
    B.flce_set_row_packing(True)
    assert np.array_equal(packed[0], plain[0]), "loss differs with packing"
    # grad_X rows are bitwise equal, except those packed into the last chunk,
    # whose K may be split in two (only the summation order differs).
    c = chunk or B.flce_plan(N, H, V, B.BF16 if dtype == "bf16" else B.F16)[0]
    last0 = (-(-N // c) - 1) * c
    live_rows = np.flatnonzero(inp["targets"] != -100)
    tail = live_rows[last0:]
    same = np.ones(N, dtype=bool)
    same[tail] = False
    assert np.array_equal(packed[1][same], plain[1][same]), "grad_X differs with packing"
    check_max_rel(packed[1], plain[1], 1e-6, "grad_X packed vs plain")
    check_max_rel(packed[2], plain[2], 1e-5, "grad_W packed vs plain")
    if bias:
        check_max_rel(packed[3], plain[3], 1e-5, "grad_bias packed vs plain")


def test_row_packing_16bit_gradients(packing):
    """flce_forward_backward_ex (bf16 gradient outputs) through the packed
    loop: grad_X rows rounded once, so bitwise equal to the unpacked call;
    zero rows for the ignored targets."""
    B = packing
    inp = synth.make_flce_inputs(900, 136, 2000, "bf16", bias_std=0.1, ignore_frac=0.4, seed=41)
    say("flce row packing, bf16 gradients")
    packed = _flce_dev(B, inp, "mean", 256, grad_dtype="input")
    B.flce_set_row_packing(False)
    plain = _flce_dev(B, inp, "mean", 256, grad_dtype="input")
    B.flce_set_row_packing(True)
    assert np.array_equal(packed[0], plain[0]) and np.array_equal(packed[1], plain[1])
    assert np.all(packed[1][inp["targets"] == -100] == 0.0)
    check_against_oracle(inp, "mean", packed)


def test_row_packing_multihead(packing):
    """Multi-head call with every head packed over its own targets (heads
    after the first add their grad_X rows through the partial buffer): the
    head losses are bitwise those of the unpacked call, the gradients equal
    up to float32 summation order."""
    import torch
    B = packing
    K, N, H, V = 3, 900, 136, 2100
    inp = synth.make_flce_inputs(N, H, K * V, "bf16", ignore_frac=0.0, seed=44)
    X = to_dev(inp["X"], "bf16")
    W = to_dev(inp["W"], "bf16").reshape(K, V, H).contiguous()
    rng = np.random.default_rng(45)
    yk = rng.integers(0, V, size=(K, N)).astype(np.int32)
    for k in range(K):  # different ignored rows per head, 10% to 50%
        yk[k, rng.choice(N, int(N * (0.1 + 0.2 * k)), replace=False)] = -100
    y = to_dev(yk, "i32")
    out = {}
    for pack in (True, False):
        B.flce_set_row_packing(pack)
        say("multihead packing", pack, K, N, H, V)
        res = B.flce_multihead_forward_backward(X, W, y, reduction="none", chunk_rows=256)
        torch.cuda.synchronize()
        out[pack] = [None if t is None else t.double().cpu().numpy() for t in res]
    B.flce_set_row_packing(True)
    assert np.array_equal(out[True][0], out[False][0]), "head losses differ with packing"
    check_max_rel(out[True][1], out[False][1], 1e-6, "grad_X packed vs plain")
    check_max_rel(out[True][2], out[False][2], 1e-5, "grad_W packed vs plain")
    assert np.all(out[True][1][(yk == -100).all(axis=0)] == 0.0)


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_ignore_index_inside_vocabulary_bf16(B, reduction):
    """ignore_index 7, a legal class id: rows with target 7 are ignored (and
    packed out), the other rows keep their targets; against the oracle with
    the same ignore_index."""
    import torch
    N, H, V = 700, 136, 1500
    inp = synth.make_flce_inputs(N, H, V, "bf16", bias_std=0.1, ignore_frac=0.0, seed=46)
    y = inp["targets"].copy()
    y[np.random.default_rng(47).choice(N, 120, replace=False)] = 7
    X, W, b, _ = oracle_inputs(inp)
    ref_loss, ref_g, _ = O.flce(X, W, y, bias=b, ignore_index=7, reduction=reduction)
    say("flce bf16 ignore_index 7", reduction)
    loss, gX, gW, gb = B.flce_forward_backward(
        to_dev(inp["X"], "bf16"), to_dev(inp["W"], "bf16"), to_dev(y, "i32"),
        bias=to_dev(inp["bias"], "bf16"), ignore_index=7, reduction=reduction, chunk_rows=256)
    torch.cuda.synchronize()
    t = TOL["bf16"]
    if reduction == "none":
        check_max_rel(to_host(loss), ref_loss, t["loss"], "loss rows")
        assert np.all(to_host(loss)[y == 7] == 0.0)
    else:
        check_scalar(to_host(loss), ref_loss, t["loss"])
    check_max_rel(to_host(gX), ref_g["X"], t["grad"], "grad_X")
    assert np.all(to_host(gX)[y == 7] == 0.0)
    check_max_rel(to_host(gW), ref_g["W"], t["grad"], "grad_W")
    check_max_rel(to_host(gb), ref_g["bias"], t["grad"], "grad_bias")


def test_row_packing_all_ignored_and_bad_targets_bf16(B):
    """16-bit inputs take the packed loop: with every row ignored no row is
    live (loss 0, all gradients 0, including grad_W's first-chunk store);
    an out-of-range target is reported and its row is left out like an
    ignored one."""
    import torch
    inp = synth.make_flce_inputs(300, 64, 500, "bf16", bias_std=0.1, ignore_frac=1.0, seed=42)
    say("flce bf16 all ignored (packed)")
    for red in ("mean", "sum", "none"):
        loss, gX, gW, gb = run_flce(B, inp, red, chunk_rows=128)
        assert np.all(loss == 0.0) and np.all(gX == 0) and np.all(gW == 0) and np.all(gb == 0)
    inp = synth.make_flce_inputs(300, 64, 500, "bf16", ignore_frac=0.2, seed=43)
    y = inp["targets"].copy()
    y[7], y[200] = 500, -5
    ws = torch.zeros(B.flce_workspace_bytes(300, 64, 500, B.BF16, 128), dtype=torch.uint8, device="cuda")
    say("flce bf16 bad targets (packed)")
    loss, gX, gW, _ = B.flce_forward_backward(
        to_dev(inp["X"], "bf16"), to_dev(inp["W"], "bf16"), to_dev(y, "i32"), reduction="none",
        chunk_rows=128, workspace=ws)
    assert B.flce_check_device_error(ws) == B.E_TARGET
    got = (to_host(loss), to_host(gX), to_host(gW), None)
    assert got[0][7] == 0.0 and got[0][200] == 0.0
    assert np.all(got[1][[7, 200]] == 0.0)
    check_against_oracle(dict(inp, targets=y), "none", got)


def test_shard_stats_of_projection(B):
    """flce_shard_stats on W[v0:v0+Vl] equals the oracle's statistics of the
    materialised shard logits."""
    import torch
    inp = synth.make_flce_inputs(700, 256, 3000, "bf16", bias_std=0.1, seed=18)
    X, W, b, y = oracle_inputs(inp)
    v0, Vl = 1000, 1200
    say("flce shard stats")
    m, s, t = B.flce_shard_stats(to_dev(inp["X"], "bf16"),
                                 to_dev(np.ascontiguousarray(inp["W"][v0:v0 + Vl]), "bf16"),
                                 to_dev(inp["targets"], "i32"), v0, 3000,
                                 bias_shard=to_dev(np.ascontiguousarray(inp["bias"][v0:v0 + Vl]), "bf16"),
                                 chunk_rows=256)
    torch.cuda.synchronize()
    rm, rs, rt = O.flce_shard_stats(X, W[v0:v0 + Vl], y, v0, 3000, bias_shard=b[v0:v0 + Vl])
    # The statistics are taken over bf16-rounded logits: the shard's
    # log-sum-exp (max + ln sumexp, what the combine step uses) is held to the
    # loss bar; the raw max and target logit to bf16's rounding (2^-8 relative).
    glse = to_host(m) + np.log(to_host(s))
    check_max_rel(glse, rm + np.log(rs), TOL["bf16"]["loss"], "shard lse")
    check_max_rel(to_host(m), rm, 2.0 ** -8, "row max")
    check_max_rel(to_host(t), rt, 2.0 ** -8, "target logit")
    assert np.all(to_host(t)[(inp["targets"] < v0) | (inp["targets"] >= v0 + Vl)] == 0.0)


def test_shift_labels_bit_exact(B):
    """Integer work: bit-exact against the oracle, including S = 1."""
    import torch
    rng = np.random.default_rng(41)
    for Bn, S in ((7, 513), (3, 1), (1, 4096)):
        lab = rng.integers(0, 128256, (Bn, S)).astype(np.int32)
        say("shift labels", Bn, S)
        got = B.flce_shift_labels(torch.from_numpy(lab).cuda())
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), O.shift_labels(lab))


def _run_multihead(B, inps, reduction, chunk_rows=0):
    import torch
    dt = inps[0]["dtype"]
    X = to_dev(inps[0]["X"], dt)
    W = torch.stack([to_dev(i["W"], dt) for i in inps]).contiguous()
    has_b = inps[0]["bias"] is not None
    b = torch.stack([to_dev(i["bias"], dt) for i in inps]).contiguous() if has_b else None
    y = torch.stack([to_dev(i["targets"], "i32") for i in inps]).contiguous()
    loss, gX, gW, gb = B.flce_multihead_forward_backward(X, W, y, bias=b, reduction=reduction,
                                                         chunk_rows=chunk_rows)
    torch.cuda.synchronize()
    return to_host(loss), to_host(gX), to_host(gW), to_host(gb)


@pytest.mark.parametrize("dtype,K,reduction,chunk,shape", [
    ("bf16", 3, "mean", 256, (600, 136, 1000)),
    ("f32", 2, "none", 0, (300, 64, 900)),
    ("bf16", 2, "sum", 0, (512, 2048, 16384)),   # grad_X split over K: accumulating reduce
])
def test_multihead_against_oracle(B, dtype, K, reduction, chunk, shape):
    """K heads over shared hidden states: per-head losses, summed grad_X,
    per-head grad_W / grad_bias."""
    N, H, V = shape
    base = synth.make_flce_inputs(N, H, V, dtype, bias_std=0.05 if N < 1000 else None,
                                  ignore_frac=0.1, seed=50)
    inps = [base] + [synth.make_flce_inputs(N, H, V, dtype, bias_std=0.05 if N < 1000 else None,
                                            ignore_frac=0.1, seed=51 + k) for k in range(K - 1)]
    for i in inps[1:]:                      # the heads share the hidden states
        i["X"], i["X_f32"] = base["X"], base["X_f32"]
    say("multihead", dtype, K, reduction, chunk, shape, B.flce_plan(N, H, V, B.BF16))
    loss, gX, gW, gb = _run_multihead(B, inps, reduction, chunk)
    X = np.asarray(base["X_f32"], np.float64)
    Ws = [np.asarray(i["W_f32"], np.float64) for i in inps]
    bs = None if base["bias"] is None else [np.asarray(i["bias_f32"], np.float64) for i in inps]
    ys = [i["targets"] for i in inps]
    ref_loss, ref_g = O.flce_multihead(X, Ws, ys, biases=bs, reduction=reduction)
    t = TOL[dtype]
    check_max_rel(loss, ref_loss, t["loss"], "head losses")
    check_max_rel(gX, ref_g["X"], t["grad"], "grad_X (sum over heads)")
    for k in range(K):
        check_max_rel(gW[k], ref_g["W"][k], t["grad"], f"grad_W head {k}")
        if bs is not None:
            check_max_rel(gb[k], ref_g["bias"][k], t["grad"], f"grad_bias head {k}")


def _run_jsd(B, s_inp, t_inp, temperature, reduction, chunk_rows=0):
    import torch
    dt = s_inp["dtype"]
    loss, gX, gW = B.flce_jsd_forward_backward(
        to_dev(s_inp["X"], dt), to_dev(s_inp["W"], dt), to_dev(t_inp["X"], dt), to_dev(t_inp["W"], dt),
        to_dev(s_inp["targets"], "i32"), temperature=temperature, reduction=reduction,
        chunk_rows=chunk_rows)
    torch.cuda.synchronize()
    return to_host(loss), to_host(gX), to_host(gW)


@pytest.mark.parametrize("dtype,reduction,temperature,chunk", [
    ("bf16", "mean", 1.0, 256), ("f32", "none", 2.0, 0), ("f16", "sum", 1.5, 0),
    ("f16", "mean", 0.5, 256)])
def test_jsd_distillation_against_oracle(B, dtype, reduction, temperature, chunk):
    """Student (H 136) distilled towards a teacher with another hidden size
    (H 72) over a ragged vocabulary (V 1000); 10% of rows masked."""
    N, Hs, Ht, V = 600, 136, 72, 1000
    s_inp = synth.make_flce_inputs(N, Hs, V, dtype, w_std=0.08, ignore_frac=0.1, seed=60)
    t_inp = synth.make_flce_inputs(N, Ht, V, dtype, w_std=0.12, ignore_frac=0.0, seed=61)
    say("jsd", dtype, reduction, temperature, chunk)
    loss, gX, gW = _run_jsd(B, s_inp, t_inp, temperature, reduction, chunk)
    f = lambda a: np.asarray(a, np.float64)
    ref_loss, ref_g, info = O.flce_jsd(f(s_inp["X_f32"]), f(s_inp["W_f32"]), f(t_inp["X_f32"]),
                                       f(t_inp["W_f32"]), s_inp["targets"], temperature=temperature,
                                       reduction=reduction)
    t = TOL[dtype]
    if reduction == "none":
        check_max_rel(loss, ref_loss, t["loss"], "JSD rows")
    else:
        check_scalar(loss, ref_loss, t["loss"], "JSD")
    check_max_rel(gX, ref_g["X"], t["grad"], "grad_X student")
    check_max_rel(gW, ref_g["W"], t["grad"], "grad_W student")
    masked = s_inp["targets"] == -100
    assert np.all(gX[masked] == 0.0)


def test_jsd_wide_teacher_bf16(B):
    """A teacher much wider than the student (H 520 against 64): its gathered
    rows do not fit the student's split-K buffer, so the call runs unpacked;
    against the oracle."""
    N, Hs, Ht, V = 300, 64, 520, 900
    s_inp = synth.make_flce_inputs(N, Hs, V, "bf16", w_std=0.08, ignore_frac=0.2, seed=62)
    t_inp = synth.make_flce_inputs(N, Ht, V, "bf16", w_std=0.05, ignore_frac=0.0, seed=63)
    say("jsd wide teacher")
    loss, gX, gW = _run_jsd(B, s_inp, t_inp, 1.0, "mean", 128)
    f = lambda a: np.asarray(a, np.float64)
    ref_loss, ref_g, _ = O.flce_jsd(f(s_inp["X_f32"]), f(s_inp["W_f32"]), f(t_inp["X_f32"]),
                                    f(t_inp["W_f32"]), s_inp["targets"], temperature=1.0,
                                    reduction="mean")
    t = TOL["bf16"]
    check_scalar(loss, ref_loss, t["loss"], "JSD")
    check_max_rel(gX, ref_g["X"], t["grad"], "grad_X student")
    check_max_rel(gW, ref_g["W"], t["grad"], "grad_W student")
    assert np.all(gX[s_inp["targets"] == -100] == 0.0)


def test_jsd_teacher_equal_to_student_is_exactly_zero(B):
    """Identical heads give identical logits on both sides: the divergence and
    every gradient are exactly zero."""
    inp = synth.make_flce_inputs(512, 64, 3000, "bf16", w_std=0.1, ignore_frac=0.05, seed=62)
    say("jsd identical heads")
    loss, gX, gW = _run_jsd(B, inp, inp, 1.0, "sum")
    assert float(loss[0]) == 0.0
    assert np.all(gX == 0.0) and np.all(gW == 0.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("N,H,V", [(1, 8, 1), (2, 8, 3), (257, 8, 9), (3, 16, 70001)])
def test_degenerate_shapes(B, dtype, N, H, V):
    """One row, one class (loss and gradients exactly 0), the smallest bf16
    hidden size, a ragged single row tile, and a long row over very few rows."""
    inp = synth.make_flce_inputs(N, H, V, dtype, w_std=0.3, ignore_frac=0.0, seed=N + V)
    say("flce degenerate", dtype, N, H, V)
    got = run_flce(B, inp, "mean")
    if V == 1:
        assert float(got[0][0]) == 0.0
        assert np.all(got[1] == 0.0) and np.all(got[2] == 0.0)
    else:
        check_against_oracle(inp, "mean", got, want=("X", "W"))


@pytest.mark.parametrize("N,H,V", [(32, 8, (1 << 22) - 8), (8, (1 << 22) - 8, 8)])
def test_maximum_strides_bf16(B, N, H, V):
    """The largest row strides the 16-bit path accepts (H and the chunk buffer's
    row stride below 2^22 elements): a GEMM tile's byte offsets reach
    255 * 2 * (2^22 - 8), just inside 32 bits; the long rows also take the
    streaming row kernel and split-K for grad_X."""
    inp = synth.make_flce_inputs(N, H, V, "bf16", w_std=0.05, ignore_frac=0.1, seed=5)
    say("flce maximum strides", N, H, V, B.flce_plan(N, H, V, B.BF16))
    check_against_oracle(inp, "mean", run_flce(B, inp, "mean"), want=("X", "W"))


def _dpo_inputs(P, S, H, V, dtype, seed):
    inp = synth.make_flce_inputs(2 * P * S, H, V, dtype, w_std=0.08, ignore_frac=0.0, seed=seed)
    y = inp["targets"]
    for k in range(2 * P):                 # the first S // 4 rows of every sequence are prompt
        y[k * S:k * S + S // 4] = -100
    rng = np.random.default_rng(seed + 1)
    ref = (rng.standard_normal(2 * P) * 3.0 - (3 * S // 4) * np.log(V)).astype(np.float32)
    return inp, ref


@pytest.mark.parametrize("dtype,P,S,H,V,chunk", [
    ("bf16", 3, 200, 136, 1000, 0),        # one chunk: no recompute
    ("bf16", 2, 300, 64, 3001, 256),       # four chunks: logits recomputed
    ("f32", 3, 64, 64, 900, 128),
    ("f16", 2, 300, 64, 3001, 256)])       # fp16: per-row factors with a power-of-two shift
def test_dpo_against_oracle(B, dtype, P, S, H, V, chunk):
    import torch
    inp, ref = _dpo_inputs(P, S, H, V, dtype, seed=70 + P)
    say("dpo", dtype, P, S, H, V, chunk)
    loss, pl, gX, gW = B.flce_dpo_forward_backward(
        to_dev(inp["X"], dtype), to_dev(inp["W"], dtype), to_dev(inp["targets"], "i32"), P, S,
        torch.from_numpy(ref).cuda(), beta=0.2, chunk_rows=chunk)
    torch.cuda.synchronize()
    X, W, _, y = oracle_inputs(inp)
    ref_loss, ref_g, info = O.flce_dpo(X, W, y, P, S, ref.astype(np.float64), beta=0.2)
    t = TOL[dtype]
    check_scalar(to_host(loss), ref_loss, t["loss"], "DPO loss")
    check_max_rel(to_host(pl), info["pair_loss"], t["loss"], "pair losses")
    check_max_rel(to_host(gX), ref_g["X"], t["grad"], "grad_X")
    check_max_rel(to_host(gW), ref_g["W"], t["grad"], "grad_W")
    assert np.all(to_host(gX)[y == -100] == 0.0)


def _rounds_ok(g16, g32, rounds, ulp, name):
    a, r = g16.double().cpu().numpy(), g32.double().cpu().numpy()
    err = np.abs(a - r).max()
    assert err <= rounds * ulp * np.abs(r).max() + 1e-30, f"{name}: {err} > {rounds} ulp"


def test_jsd_and_dpo_gradients_in_the_input_type(B):
    """flce_jsd_forward_backward_ex and flce_dpo_forward_backward_ex with bf16
    gradient outputs: the same loss as the float32-gradient calls, grad_X within
    one bf16 rounding of theirs, grad_W within one rounding per chunk, and the
    oracle's bar."""
    import torch
    ulp = 2.0 ** -8
    N, Hs, Ht, V, chunk = 600, 136, 72, 1000, 256
    s_inp = synth.make_flce_inputs(N, Hs, V, "bf16", w_std=0.08, ignore_frac=0.1, seed=80)
    t_inp = synth.make_flce_inputs(N, Ht, V, "bf16", w_std=0.12, ignore_frac=0.0, seed=81)
    args = (to_dev(s_inp["X"], "bf16"), to_dev(s_inp["W"], "bf16"), to_dev(t_inp["X"], "bf16"),
            to_dev(t_inp["W"], "bf16"), to_dev(s_inp["targets"], "i32"))
    say("jsd 16-bit gradients")
    l16, gX16, gW16 = B.flce_jsd_forward_backward(*args, temperature=1.5, chunk_rows=chunk,
                                                  grad_dtype="input")
    l32, gX32, gW32 = B.flce_jsd_forward_backward(*args, temperature=1.5, chunk_rows=chunk)
    torch.cuda.synchronize()
    assert gX16.dtype == torch.bfloat16 and gW16.dtype == torch.bfloat16
    assert torch.equal(l16, l32)
    _rounds_ok(gX16, gX32, 1, ulp, "JSD grad_X")
    _rounds_ok(gW16, gW32, -(-N // chunk), ulp, "JSD grad_W")
    f = lambda a: np.asarray(a, np.float64)
    _, ref_g, _ = O.flce_jsd(f(s_inp["X_f32"]), f(s_inp["W_f32"]), f(t_inp["X_f32"]),
                             f(t_inp["W_f32"]), s_inp["targets"], temperature=1.5)
    check_max_rel(gX16.float().cpu().numpy(), ref_g["X"], TOL["bf16"]["grad"], "JSD grad_X bf16")
    check_max_rel(gW16.float().cpu().numpy(), ref_g["W"], TOL["bf16"]["grad"], "JSD grad_W bf16")

    P, S, H, V = 2, 300, 64, 3001
    inp, ref = _dpo_inputs(P, S, H, V, "bf16", seed=82)
    args = (to_dev(inp["X"], "bf16"), to_dev(inp["W"], "bf16"), to_dev(inp["targets"], "i32"), P, S,
            torch.from_numpy(ref).cuda())
    say("dpo 16-bit gradients")
    l16, _, gX16, gW16 = B.flce_dpo_forward_backward(*args, beta=0.2, chunk_rows=256, grad_dtype="input")
    l32, _, gX32, gW32 = B.flce_dpo_forward_backward(*args, beta=0.2, chunk_rows=256)
    torch.cuda.synchronize()
    assert gX16.dtype == torch.bfloat16 and torch.equal(l16, l32)
    _rounds_ok(gX16, gX32, 1, ulp, "DPO grad_X")
    _rounds_ok(gW16, gW32, -(-(2 * P * S) // 256), ulp, "DPO grad_W")
    X, W, _, y = oracle_inputs(inp)
    _, ref_g, _ = O.flce_dpo(X, W, y, P, S, ref.astype(np.float64), beta=0.2)
    check_max_rel(gX16.float().cpu().numpy(), ref_g["X"], TOL["bf16"]["grad"], "DPO grad_X bf16")
    check_max_rel(gW16.float().cpu().numpy(), ref_g["W"], TOL["bf16"]["grad"], "DPO grad_W bf16")


@pytest.mark.timeout(300)
def test_row_packing_over_a_thousand_pack_blocks(packing):
    """4.2 million rows (H 8, V 64, 30% ignored): the packing kernels' block
    prefix runs over more than 1024 blocks of 4096 rows (several rounds of its
    single-workgroup scan). Against the unpacked call: per-row losses bitwise,
    grad_X and grad_W to float32 summation order; sampled rows' losses against
    the oracle."""
    import torch
    B = packing
    N, H, V = 1024 * 4096 + 3001, 8, 64
    inp = synth.make_flce_inputs(N, H, V, "bf16", ignore_frac=0.3, seed=90)
    X, W, y = to_dev(inp["X"], "bf16"), to_dev(inp["W"], "bf16"), to_dev(inp["targets"], "i32")
    out = {}
    for pack in (True, False):
        B.flce_set_row_packing(pack)
        say("flce 4.2M rows, packing", pack)
        out[pack] = B.flce_forward_backward(X, W, y, reduction="none")
        torch.cuda.synchronize()
    B.flce_set_row_packing(True)
    (l1, gx1, gw1, _), (l0, gx0, gw0, _) = out[True], out[False]
    assert torch.equal(l1, l0), "per-row losses differ with packing"
    # grad_X rows sum 64 products: float32 order only. grad_W entries are
    # float32 sums over ~2.9 million rows, split into chunks at different rows
    # by the two paths; each sum carries a rounding error of order
    # sqrt(n) * 2^-24 of its magnitude (~1e-4 here), so the two may differ by
    # about twice that.
    for a, r, name, tol in ((gx1, gx0, "grad_X", 1e-5), (gw1, gw0, "grad_W", 2e-4)):
        err = float((a - r).abs().max())
        assert err <= tol * float(r.abs().max()), f"{name}: {err}"
    assert float(gx1[y == -100].abs().max()) == 0.0
    rows = np.random.default_rng(91).choice(N, 64, replace=False)
    Xs, Ws, _, ys = oracle_inputs(inp)
    ref_rows, _, _ = O.flce(Xs[rows], Ws, ys[rows], reduction="none", want_grads=False)
    check_max_rel(l1.cpu().numpy()[rows], ref_rows, TOL["bf16"]["loss"], "sampled row losses")


def _guarded_workspace(n, guard=1 << 13):
    """A workspace of exactly n bytes followed by `guard` bytes of 0x5A."""
    import torch
    buf = torch.full((n + guard,), 0x5A, dtype=torch.uint8, device="cuda")
    return buf, buf[:n]


def _guard_intact(buf, n):
    import torch
    torch.cuda.synchronize()
    assert bool((buf[n:] == 0x5A).all()), "a call wrote past the workspace it was given"


@pytest.mark.parametrize("chunk", [256, 160])
def test_calls_stay_inside_the_workspace(B, chunk):
    """Each FLCE-family call (FLCE, multi-head, distillation, DPO), given a
    workspace of exactly its queried size, leaves the bytes after it alone and
    still matches the oracle. Chunks of 256 rows hold the packed chunk's rows
    and their transpose in the split-K partial buffer; chunks of 160 rows
    (a transpose stride of 192) hold the rows only."""
    import torch
    N, H, V = 600, 136, 1000
    inp = synth.make_flce_inputs(N, H, V, "bf16", bias_std=0.1, ignore_frac=0.1, seed=81)
    X, W, b = (to_dev(inp[k], "bf16") for k in ("X", "W", "bias"))
    y = to_dev(inp["targets"], "i32")
    say("workspace bounds, chunk", chunk)
    n = B.flce_workspace_bytes(N, H, V, B.BF16, chunk)
    buf, ws = _guarded_workspace(n)
    got = B.flce_forward_backward(X, W, y, bias=b, reduction="mean", chunk_rows=chunk,
                                  grad_bias=True, workspace=ws)
    _guard_intact(buf, n)
    check_against_oracle(inp, "mean", tuple(None if t is None else to_host(t) for t in got))

    K = 2
    Wk = torch.stack([W, torch.roll(W, 3, dims=0)]).contiguous()
    yk = torch.stack([y, torch.roll(y, -1)]).contiguous()
    n = B.flce_multihead_workspace_bytes(N, H, V, K, B.BF16, chunk)
    buf, ws = _guarded_workspace(n)
    B.flce_multihead_forward_backward(X, Wk, yk, reduction="mean", chunk_rows=chunk, workspace=ws)
    _guard_intact(buf, n)

    n = B.flce_jsd_workspace_bytes(N, H, V, B.BF16, chunk)
    buf, ws = _guarded_workspace(n)
    B.flce_jsd_forward_backward(X, W, torch.roll(X, 1, dims=0).contiguous(), Wk[1], y,
                                temperature=1.5, chunk_rows=chunk, workspace=ws)
    _guard_intact(buf, n)

    P, S = 2, N // 4
    n = B.flce_dpo_workspace_bytes(P, S, H, V, B.BF16, chunk)
    buf, ws = _guarded_workspace(n)
    ref = torch.full((2 * P,), -float(S) * 7.0, device="cuda")
    B.flce_dpo_forward_backward(X, W, y, P, S, ref, beta=0.2, chunk_rows=chunk, workspace=ws)
    _guard_intact(buf, n)
