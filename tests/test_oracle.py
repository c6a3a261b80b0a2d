"""Pins for the FP64 oracle, independent of the oracle's own formulas.

Each test checks the oracle against something it does not compute itself:
closed forms of special cases, hand-worked values, central finite differences,
a brute-force pure-Python evaluation, PyTorch's CPU cross-entropy (the pages
define CE by PyTorch's CrossEntropyLoss), invariants that any correct result
satisfies, and the one number the pages print for this path (16.8 GB of logits).
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import flce_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(rng, N=7, H=5, V=9, bias=True, n_ignored=2, ignore_index=-100):
    X = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H)) * 0.7
    b = rng.standard_normal(V) * 0.3 if bias else None
    y = rng.integers(0, V, size=N)
    if n_ignored:
        y[rng.choice(N, n_ignored, replace=False)] = ignore_index
    return X, W, b, y


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_zero_weight_gives_log_vocab(reduction):
    rng = np.random.default_rng(1)
    N, H, V = 11, 6, 13
    X = rng.standard_normal((N, H))
    W = np.zeros((V, H))
    y = rng.integers(0, V, size=N)
    y[[2, 5]] = -100
    valid = y != -100
    nv = int(valid.sum())
    loss, g, info = O.flce(X, W, y, reduction=reduction)
    lnV = math.log(V)
    if reduction == "none":
        np.testing.assert_allclose(loss, np.where(valid, lnV, 0.0), rtol=0, atol=1e-14)
    elif reduction == "sum":
        assert abs(loss - nv * lnV) < 1e-12
    else:
        assert abs(loss - lnV) < 1e-14
    s = 1.0 / nv if reduction == "mean" else 1.0
    # With W = 0 every softmax is uniform: dZ[n] = s (1/V - e_{y_n}) for valid n.
    assert np.all(g["X"] == 0.0)
    expect_gW = np.zeros((V, H))
    for n in range(N):
        if valid[n]:
            expect_gW += s * X[n][None, :] / V
            expect_gW[y[n]] -= s * X[n]
    np.testing.assert_allclose(g["W"], expect_gW, rtol=0, atol=1e-13)


def test_zero_input_reduces_to_bias_softmax():
    """X = 0 makes every logit row equal to the bias: loss_n = lse(b) - b_y,
    grad_W = 0, grad_bias = s (N_valid softmax(b) - counts), grad_X_n =
    s (softmax(b) - e_y) W. softmax / logsumexp come from scipy here."""
    from scipy.special import logsumexp, softmax

    rng = np.random.default_rng(2)
    N, H, V = 9, 4, 17
    X = np.zeros((N, H))
    W = rng.standard_normal((V, H))
    b = rng.standard_normal(V) * 2
    y = rng.integers(0, V, size=N)
    y[3] = -100
    valid = y != -100
    nv = int(valid.sum())
    loss, g, _ = O.flce(X, W, y, bias=b, reduction="mean")
    lse = logsumexp(b)
    assert abs(loss - np.mean(lse - b[y[valid]])) < 1e-13
    assert np.all(g["W"] == 0.0)
    counts = np.bincount(y[valid], minlength=V)
    p = softmax(b)
    np.testing.assert_allclose(g["bias"], (nv * p - counts) / nv, atol=1e-14)
    for n in range(N):
        e = np.zeros(V)
        if valid[n]:
            e[y[n]] = 1.0
            np.testing.assert_allclose(g["X"][n], (p - e) @ W / nv, atol=1e-14)
        else:
            assert np.all(g["X"][n] == 0.0)


def test_two_classes_is_softplus():
    """With V = 2 the loss is softplus(z_other - z_target) and its gradient
    w.r.t. z_target is -sigmoid(z_other - z_target)."""
    rng = np.random.default_rng(3)
    Z = rng.standard_normal((20, 2)) * 3
    y = rng.integers(0, 2, size=20)
    loss, dZ, _ = O.cross_entropy(Z, y, reduction="none")
    d = Z[np.arange(20), 1 - y] - Z[np.arange(20), y]
    np.testing.assert_allclose(loss, np.logaddexp(0.0, d), rtol=1e-11, atol=1e-15)
    sig = 1.0 / (1.0 + np.exp(-d))
    np.testing.assert_allclose(dZ[np.arange(20), y], -sig, rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(dZ[np.arange(20), 1 - y], sig, rtol=1e-11, atol=1e-15)


def test_hand_worked_examples():
    with open(os.path.join(GOLDEN, "ce_hand_example.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        z = np.array([c["logits"]])
        loss, dZ, _ = O.cross_entropy(z, [c["target"]], reduction="sum")
        assert abs(loss - c["loss"]) < 1e-14
        np.testing.assert_allclose(dZ[0], c["grad"], atol=1e-15)


def test_materialised_logits_bytes_matches_page():
    with open(os.path.join(GOLDEN, "logits_bytes.json")) as f:
        g = json.load(f)
    nbytes = O.materialised_logits_bytes(g["batch"] * g["seq"], g["vocab"], g["elem_bytes"])
    assert round(nbytes / 1e9, 1) == g["printed_gb"]


# ------------------------------------------------------- independent evaluators

def _brute_force_ce(Z, y, ignore_index, reduction):
    """Pure-Python loops with math.exp / math.log, no max subtraction."""
    total = 0.0
    rows = []
    nv = 0
    for n in range(len(Z)):
        if y[n] == ignore_index:
            rows.append(0.0)
            continue
        nv += 1
        s = 0.0
        for z in Z[n]:
            s += math.exp(z)
        li = math.log(s) - Z[n][y[n]]
        rows.append(li)
        total += li
    if reduction == "none":
        return rows
    if reduction == "sum":
        return total
    return total / nv


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_brute_force_tiny(reduction):
    rng = np.random.default_rng(4)
    X, W, b, y = _rand_problem(rng, N=6, H=3, V=5)
    loss, _, _ = O.flce(X, W, y, bias=b, reduction=reduction)
    Z = [[sum(X[n][h] * W[v][h] for h in range(3)) + b[v] for v in range(5)] for n in range(6)]
    ref = _brute_force_ce(Z, list(y), -100, reduction)
    np.testing.assert_allclose(loss, ref, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_finite_differences(reduction):
    """Central differences of the scalar objective (sum of per-row losses for
    'none') agree with the oracle's analytic gradients."""
    rng = np.random.default_rng(5)
    X, W, b, y = _rand_problem(rng, N=6, H=4, V=7)

    def obj(X_, W_, b_):
        loss, _, _ = O.flce(X_, W_, y, bias=b_, reduction=reduction, want_grads=False)
        return float(np.sum(loss))

    _, g, _ = O.flce(X, W, y, bias=b, reduction=reduction)
    eps = 1e-6
    for name, arr, grad in (("X", X, g["X"]), ("W", W, g["W"]), ("bias", b, g["bias"])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = arr[idx]
            arr[idx] = old + eps
            fp = obj(X, W, b)
            arr[idx] = old - eps
            fm = obj(X, W, b)
            arr[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        scale = max(1.0, float(np.abs(grad).max()))
        assert np.abs(num - grad).max() <= 1e-7 * scale, name


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_against_torch_cpu_float64(reduction):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(6)
    X, W, b, y = _rand_problem(rng, N=40, H=16, V=33, n_ignored=5)
    loss, g, _ = O.flce(X, W, y, bias=b, reduction=reduction, row_block=7)
    tX = torch.tensor(X, requires_grad=True)
    tW = torch.tensor(W, requires_grad=True)
    tb = torch.tensor(b, requires_grad=True)
    ty = torch.tensor(y)
    tl = F.cross_entropy(F.linear(tX, tW, tb), ty, ignore_index=-100, reduction=reduction)
    tl.sum().backward()
    np.testing.assert_allclose(loss, tl.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["X"], tX.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(g["W"], tW.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(g["bias"], tb.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_ce_against_torch_cpu_float64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    Z = rng.standard_normal((30, 50)) * 4
    y = rng.integers(0, 50, size=30)
    y[[0, 7, 9]] = -100
    for red in ("none", "sum", "mean"):
        loss, dZ, _ = O.cross_entropy(Z, y, reduction=red)
        tZ = torch.tensor(Z, requires_grad=True)
        tl = torch.nn.functional.cross_entropy(tZ, torch.tensor(y), reduction=red)
        tl.sum().backward()
        np.testing.assert_allclose(loss, tl.detach().numpy(), rtol=1e-12)
        np.testing.assert_allclose(dZ, tZ.grad.numpy(), rtol=1e-11, atol=1e-15)


# ------------------------------------------------------------------ invariants

def test_reduction_identities():
    rng = np.random.default_rng(8)
    X, W, b, y = _rand_problem(rng, N=25, H=6, V=11, n_ignored=4)
    ln, gn, info = O.flce(X, W, y, bias=b, reduction="none")
    ls, gs, _ = O.flce(X, W, y, bias=b, reduction="sum")
    lm, gm, _ = O.flce(X, W, y, bias=b, reduction="mean")
    nv = info["n_valid"]
    assert nv == 21
    assert abs(ls - ln.sum()) < 1e-12
    assert abs(lm - ls / nv) < 1e-13
    for k in ("X", "W", "bias"):
        np.testing.assert_allclose(gn[k], gs[k], atol=0)
        np.testing.assert_allclose(gm[k], gs[k] / nv, rtol=1e-13, atol=1e-16)


def test_gradient_row_sums_vanish():
    rng = np.random.default_rng(9)
    X, W, b, y = _rand_problem(rng, N=20, H=5, V=12)
    _, dZ, _ = O.cross_entropy(X @ W.T + b, y, reduction="sum")
    np.testing.assert_allclose(dZ.sum(axis=1), 0.0, atol=1e-14)
    _, g, _ = O.flce(X, W, y, bias=b, reduction="sum")
    np.testing.assert_allclose(g["W"].sum(axis=0), 0.0, atol=1e-12)
    assert abs(g["bias"].sum()) < 1e-12


def test_bias_shift_invariance():
    rng = np.random.default_rng(10)
    X, W, b, y = _rand_problem(rng, N=15, H=5, V=8)
    l1, g1, _ = O.flce(X, W, y, bias=b, reduction="mean")
    l2, g2, _ = O.flce(X, W, y, bias=b + 3.25, reduction="mean")
    assert abs(l1 - l2) < 1e-13
    for k in ("X", "W", "bias"):
        np.testing.assert_allclose(g1[k], g2[k], atol=1e-14)


def test_row_permutation_equivariance():
    rng = np.random.default_rng(11)
    X, W, b, y = _rand_problem(rng, N=18, H=5, V=8)
    perm = rng.permutation(18)
    ln, g, _ = O.flce(X, W, y, bias=b, reduction="none")
    lp, gp, _ = O.flce(X[perm], W, y[perm], bias=b, reduction="none")
    np.testing.assert_allclose(lp, ln[perm], atol=1e-15)
    np.testing.assert_allclose(gp["X"], g["X"][perm], atol=1e-15)
    np.testing.assert_allclose(gp["W"], g["W"], atol=1e-13)


def test_row_blocking_does_not_change_results():
    rng = np.random.default_rng(12)
    X, W, b, y = _rand_problem(rng, N=23, H=6, V=10)
    l1, g1, _ = O.flce(X, W, y, bias=b, reduction="mean", row_block=1024)
    l2, g2, _ = O.flce(X, W, y, bias=b, reduction="mean", row_block=4)
    assert abs(l1 - l2) < 1e-14
    for k in ("X", "W", "bias"):
        np.testing.assert_allclose(g1[k], g2[k], atol=1e-14)


def test_ignored_and_bad_rows_are_exact_zeros():
    rng = np.random.default_rng(13)
    X, W, b, y = _rand_problem(rng, N=12, H=4, V=6, n_ignored=3)
    y[0] = 6      # out of range -> bad
    y[1] = -7     # negative, not the ignore index -> bad
    loss, g, info = O.flce(X, W, y, bias=b, reduction="none")
    assert info["n_bad"] == 2
    dead = (y == -100) | (y == 6) | (y == -7)
    assert np.all(loss[dead] == 0.0)
    assert np.all(g["X"][dead] == 0.0)
    assert np.all(loss[~dead] > 0.0)


def test_mean_with_no_valid_rows_is_zero():
    X = np.ones((4, 3))
    W = np.ones((5, 3))
    y = np.full(4, -100)
    loss, g, info = O.flce(X, W, y, reduction="mean")
    assert loss == 0.0 and info["n_valid"] == 0
    assert np.all(g["X"] == 0) and np.all(g["W"] == 0)


def test_ignore_index_inside_vocab_range():
    """A row is ignored iff its target equals ignore_index, even when that value
    is a legal class id."""
    rng = np.random.default_rng(14)
    Z = rng.standard_normal((6, 5))
    y = np.array([0, 1, 2, 3, 4, 2])
    loss, dZ, info = O.cross_entropy(Z, y, ignore_index=2, reduction="none")
    assert info["n_valid"] == 4
    assert loss[2] == 0.0 and loss[5] == 0.0
    assert np.all(dZ[[2, 5]] == 0.0)


# ----------------------------------------------------------------- shard stats

def test_shard_stats_combine_to_full_vocab():
    rng = np.random.default_rng(15)
    N, V = 64, 96
    Z = rng.standard_normal((N, V)) * 2
    y = rng.integers(0, V, size=N)
    y[[1, 4, 9]] = -100
    parts = [O.shard_stats(Z[:, a:a + 32], y, a, V) for a in (0, 32, 64)]
    lse, zt = O.combine_shard_stats(parts)
    full_lse = np.array([math.log(sum(math.exp(v) for v in row)) for row in Z])
    np.testing.assert_allclose(lse, full_lse, rtol=1e-14)
    valid = y != -100
    np.testing.assert_allclose(zt[valid], Z[np.arange(N)[valid], y[valid]], rtol=0, atol=0)
    assert np.all(zt[~valid] == 0.0)
    for m, s, t in parts:
        assert np.all(s >= 1.0)   # the shard maximum contributes exp(0) = 1


def test_flce_shard_stats_matches_materialised():
    rng = np.random.default_rng(16)
    X, W, b, y = _rand_problem(rng, N=30, H=6, V=20)
    Ws, bs = W[8:15], b[8:15]
    m, s, t = O.flce_shard_stats(X, Ws, y, 8, 20, bias_shard=bs, row_block=7)
    m2, s2, t2 = O.shard_stats(X @ Ws.T + bs, y, 8, 20)
    np.testing.assert_allclose(m, m2, atol=1e-15)
    np.testing.assert_allclose(s, s2, rtol=1e-14)
    np.testing.assert_allclose(t, t2, atol=1e-15)


def test_sampled_helpers_agree_with_full():
    rng = np.random.default_rng(17)
    X, W, b, y = _rand_problem(rng, N=26, H=5, V=14, n_ignored=3)
    loss, g, info = O.flce(X, W, y, bias=b, reduction="mean")
    rows = np.array([0, 5, 25, 11])
    lr, gx = O.flce_rows(X, W, y, rows, bias=b, reduction="mean")
    np.testing.assert_allclose(lr, info["loss_rows"][rows], atol=1e-15)
    np.testing.assert_allclose(gx, g["X"][rows], atol=1e-15)
    vr = np.array([13, 0, 7])
    gw, gb = O.flce_grad_w_rows(X, W, y, vr, bias=b, reduction="mean", row_block=5)
    np.testing.assert_allclose(gw, g["W"][vr], atol=1e-14)
    np.testing.assert_allclose(gb, g["bias"][vr], atol=1e-14)


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_one_pass_sampled_flce_agrees_with_full(reduction):
    """flce_sampled (the full-size golden values) keeps exactly the rows the
    full oracle computes: every loss row, the reduction, and the selected
    grad_X / grad_W / grad_bias rows, across several row blocks."""
    rng = np.random.default_rng(18)
    X, W, b, y = _rand_problem(rng, N=37, H=6, V=15, n_ignored=5)
    y[3] = 40  # out of range: treated as ignored
    loss, g, info = O.flce(X, W, y, bias=b, reduction=reduction, row_block=8)
    tr, vr = np.array([0, 7, 8, 36, 3]), np.array([14, 0, 6])
    l2, rows, gx, gw, gb, nv = O.flce_sampled(X, W, y, tr, vr, bias=b, reduction=reduction,
                                              row_block=8)
    np.testing.assert_allclose(np.asarray(l2), np.asarray(loss), rtol=1e-15, atol=0)
    np.testing.assert_array_equal(rows, info["loss_rows"])
    assert nv == info["n_valid"]
    np.testing.assert_allclose(gx, g["X"][tr], atol=1e-15)
    np.testing.assert_allclose(gw, g["W"][vr], atol=1e-14)
    np.testing.assert_allclose(gb, g["bias"][vr], atol=1e-14)
    assert np.all(gx[4] == 0.0)
    _, _, _, _, gb0, _ = O.flce_sampled(X, W, y, tr, vr, reduction=reduction)
    assert gb0 is None


# ------------------------------------------------- vocabulary-shard backward

def _lse_by_loops(Z):
    return np.array([math.log(sum(math.exp(v) for v in row)) for row in Z])


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_shard_backward_with_one_shard_is_flce(reduction):
    rng = np.random.default_rng(18)
    X, W, b, y = _rand_problem(rng, N=23, H=6, V=17, n_ignored=4)
    y[3] = 17  # bad target: treated as ignored on both sides
    _, g, _ = O.flce(X, W, y, bias=b, reduction=reduction)
    lse = _lse_by_loops(X @ W.T + b)
    gx, gw, gb = O.flce_shard_backward(X, W, y, 0, 17, lse, bias_shard=b, reduction=reduction,
                                       row_block=5)
    np.testing.assert_allclose(gx, g["X"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gw, g["W"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(gb, g["bias"], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_vocab_parallel_pipeline_is_flce(reduction):
    """Shard stats -> combine -> loss, then each shard's backward: the loss,
    the sum of the grad_X partials and the concatenated grad_W / grad_bias
    shards equal the unsharded FLCE."""
    rng = np.random.default_rng(19)
    V = 29
    X, W, b, y = _rand_problem(rng, N=31, H=7, V=V, n_ignored=5)
    y[0] = -3   # bad target
    loss, g, info = O.flce(X, W, y, bias=b, reduction=reduction)
    bounds = [0, 5, 18, V]   # uneven shards
    stats = [O.flce_shard_stats(X, W[a:c], y, a, V, bias_shard=b[a:c], row_block=8)
             for a, c in zip(bounds[:-1], bounds[1:])]
    lse, zt = O.combine_shard_stats(stats)
    sl, rows, n_valid = O.shard_loss(lse, zt, y, V, reduction=reduction)
    assert n_valid == info["n_valid"]
    np.testing.assert_allclose(rows, info["loss_rows"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sl, loss, rtol=1e-12, atol=1e-14)
    parts = [O.flce_shard_backward(X, W[a:c], y, a, V, lse, bias_shard=b[a:c], reduction=reduction)
             for a, c in zip(bounds[:-1], bounds[1:])]
    np.testing.assert_allclose(sum(p[0] for p in parts), g["X"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.concatenate([p[1] for p in parts]), g["W"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(np.concatenate([p[2] for p in parts]), g["bias"], rtol=1e-12, atol=1e-14)


def test_shard_backward_finite_differences():
    """grad_W_shard is the derivative of the global mean loss w.r.t. the
    shard's head rows (central differences through the unsharded loss)."""
    rng = np.random.default_rng(20)
    V = 11
    X, W, b, y = _rand_problem(rng, N=9, H=4, V=V, n_ignored=2)
    a, c = 4, 9
    lse = _lse_by_loops(X @ W.T + b)
    gx, gw, gb = O.flce_shard_backward(X, W[a:c], y, a, V, lse, bias_shard=b[a:c])
    h = 1e-6
    for (i, j) in [(0, 0), (2, 3), (4, 1)]:
        Wp, Wm = W.copy(), W.copy()
        Wp[a + i, j] += h
        Wm[a + i, j] -= h
        lp, _, _ = O.flce(X, Wp, y, bias=b, want_grads=False)
        lm, _, _ = O.flce(X, Wm, y, bias=b, want_grads=False)
        assert abs((lp - lm) / (2 * h) - gw[i, j]) < 1e-8
    # grad_X partials: the other shards' columns are missing, so compare the
    # sum over a full partition instead.
    rest = [O.flce_shard_backward(X, W[p:q], y, p, V, lse, bias_shard=b[p:q])[0]
            for p, q in ((0, a), (c, V))]
    Xp = X.copy()
    Xp[1, 2] += h
    Xm = X.copy()
    Xm[1, 2] -= h
    lp, _, _ = O.flce(Xp, W, y, bias=b, want_grads=False)
    lm, _, _ = O.flce(Xm, W, y, bias=b, want_grads=False)
    assert abs((lp - lm) / (2 * h) - (gx + rest[0] + rest[1])[1, 2]) < 1e-8


def test_shift_labels_hand_example():
    """Position s predicts token s + 1; each sequence's last position has no target."""
    lab = np.array([[5, 6, 7], [1, 2, 3]])
    np.testing.assert_array_equal(O.shift_labels(lab), [6, 7, -100, 2, 3, -100])
    np.testing.assert_array_equal(O.shift_labels(np.array([[9], [4]]), ignore_index=-1), [-1, -1])


# --------------------------------------------------------------- multi-head

def test_multihead_single_head_is_flce():
    rng = np.random.default_rng(21)
    X, W, b, y = _rand_problem(rng, N=13, H=5, V=9)
    losses, g = O.flce_multihead(X, [W], [y], biases=[b], reduction="sum")
    loss, g1, _ = O.flce(X, W, y, bias=b, reduction="sum")
    assert losses.shape == (1,) and losses[0] == loss
    np.testing.assert_array_equal(g["X"], g1["X"])
    np.testing.assert_array_equal(g["W"][0], g1["W"])


def test_multihead_finite_differences():
    """grad_X of the multi-head call is the derivative of the summed head
    losses (each head's mean over its own valid rows)."""
    rng = np.random.default_rng(22)
    N, H, V, K = 8, 4, 7, 3
    X = rng.standard_normal((N, H))
    Ws = [rng.standard_normal((V, H)) * 0.5 for _ in range(K)]
    ys = [rng.integers(0, V, N) for _ in range(K)]
    ys[1][[0, 3]] = -100
    _, g = O.flce_multihead(X, Ws, ys, reduction="mean")

    def total(Xp):
        return sum(O.flce(Xp, Ws[k], ys[k], want_grads=False)[0] for k in range(K))
    h = 1e-6
    for (i, j) in [(0, 0), (3, 2), (7, 1)]:
        Xp, Xm = X.copy(), X.copy()
        Xp[i, j] += h
        Xm[i, j] -= h
        assert abs((total(Xp) - total(Xm)) / (2 * h) - g["X"][i, j]) < 1e-8


# ------------------------------------------------------------ distillation

def _jsd_brute(zs, zt, T):
    """Pure-Python Jensen-Shannon divergence of one row (no shifts)."""
    es = [math.exp(v / T) for v in zs]
    et = [math.exp(v / T) for v in zt]
    p = [v / sum(es) for v in es]
    q = [v / sum(et) for v in et]
    m = [(a + b) / 2 for a, b in zip(p, q)]
    return 0.5 * sum(a * math.log(a / c) for a, c in zip(p, m)) + \
        0.5 * sum(b * math.log(b / c) for b, c in zip(q, m))


def test_jsd_brute_force_and_bounds():
    rng = np.random.default_rng(23)
    Zs, Zt = rng.standard_normal((6, 9)) * 2, rng.standard_normal((6, 9)) * 2
    for T in (1.0, 2.5):
        jsd, _ = O.jsd_rows(Zs, Zt, T)
        ref = [_jsd_brute(Zs[i], Zt[i], T) for i in range(6)]
        np.testing.assert_allclose(jsd, ref, rtol=1e-12)
        assert np.all(jsd >= 0) and np.all(jsd <= math.log(2))
    # identical distributions: zero divergence and zero gradient
    jsd, dZ = O.jsd_rows(Zs, Zs + 3.0, 1.0)   # a shift leaves softmax unchanged
    assert np.abs(jsd).max() < 1e-15 and np.abs(dZ).max() < 1e-15
    # symmetric in its two distributions
    np.testing.assert_allclose(O.jsd_rows(Zs, Zt)[0], O.jsd_rows(Zt, Zs)[0], rtol=1e-13)
    # disjoint one-hot limits approach ln 2
    big = np.full((1, 4), -60.0)
    a, b = big.copy(), big.copy()
    a[0, 0] = 60.0
    b[0, 3] = 60.0
    assert abs(O.jsd_rows(a, b)[0][0] - math.log(2)) < 1e-12


def test_jsd_gradient_finite_differences():
    rng = np.random.default_rng(24)
    Zs, Zt = rng.standard_normal((3, 7)), rng.standard_normal((3, 7))
    for T in (1.0, 1.7):
        _, dZ = O.jsd_rows(Zs, Zt, T)
        h = 1e-6
        for (i, j) in [(0, 0), (1, 4), (2, 6)]:
            Zp, Zm = Zs.copy(), Zs.copy()
            Zp[i, j] += h
            Zm[i, j] -= h
            fd = (O.jsd_rows(Zp, Zt, T)[0][i] - O.jsd_rows(Zm, Zt, T)[0][i]) / (2 * h)
            assert abs(fd - dZ[i, j]) < 1e-8


@pytest.mark.parametrize("reduction", ["none", "sum", "mean"])
def test_flce_jsd_finite_differences_and_masking(reduction):
    rng = np.random.default_rng(25)
    N, Hs, Ht, V = 9, 5, 3, 8
    Xs, Ws = rng.standard_normal((N, Hs)), rng.standard_normal((V, Hs)) * 0.6
    Xt, Wt = rng.standard_normal((N, Ht)), rng.standard_normal((V, Ht)) * 0.6
    y = rng.integers(0, V, N)
    y[[2, 5]] = -100
    loss, g, info = O.flce_jsd(Xs, Ws, Xt, Wt, y, temperature=1.5, reduction=reduction, row_block=4)
    assert np.all(info["loss_rows"][[2, 5]] == 0.0) and np.all(g["X"][[2, 5]] == 0.0)

    def total(Xs_, Ws_):
        return float(np.sum(O.flce_jsd(Xs_, Ws_, Xt, Wt, y, temperature=1.5, reduction=reduction)[0]))
    h = 1e-6
    for (i, j) in [(0, 0), (4, 3)]:
        Xp, Xm = Xs.copy(), Xs.copy()
        Xp[i, j] += h
        Xm[i, j] -= h
        assert abs((total(Xp, Ws) - total(Xm, Ws)) / (2 * h) - g["X"][i, j]) < 1e-7
    for (i, j) in [(1, 2), (7, 4)]:
        Wp, Wm = Ws.copy(), Ws.copy()
        Wp[i, j] += h
        Wm[i, j] -= h
        assert abs((total(Xs, Wp) - total(Xs, Wm)) / (2 * h) - g["W"][i, j]) < 1e-7


# -------------------------------------------------------------------- DPO

def _dpo_problem(rng, P=3, S=5, H=4, V=7):
    X = rng.standard_normal((2 * P * S, H))
    W = rng.standard_normal((V, H)) * 0.7
    y = rng.integers(0, V, 2 * P * S)
    y[[0, 1, P * S, P * S + 1]] = -100       # prompt tokens of two sequences
    ref = rng.standard_normal(2 * P) - 10.0
    return X, W, y, ref


def test_dpo_logps_and_closed_form():
    rng = np.random.default_rng(26)
    P, S = 3, 5
    X, W, y, ref = _dpo_problem(rng, P, S)
    loss, g, info = O.flce_dpo(X, W, y, P, S, ref, beta=0.3)
    # sequence log-probabilities by brute force
    for k in range(2 * P):
        lp = 0.0
        for r in range(k * S, (k + 1) * S):
            if y[r] == -100:
                continue
            z = X[r] @ W.T
            lp += z[y[r]] - math.log(sum(math.exp(v) for v in z))
        assert abs(info["logps"][k] - lp) < 1e-12
    d = 0.3 * ((info["logps"][:P] - ref[:P]) - (info["logps"][P:] - ref[P:]))
    ref_loss = np.mean([-math.log(1.0 / (1.0 + math.exp(-v))) for v in d])
    assert abs(loss - ref_loss) < 1e-12
    # swapping chosen and rejected turns d into -d
    Xs = np.concatenate([X[P * S:], X[:P * S]])
    ys = np.concatenate([y[P * S:], y[:P * S]])
    refs = np.concatenate([ref[P:], ref[:P]])
    _, _, info2 = O.flce_dpo(Xs, W, ys, P, S, refs, beta=0.3)
    np.testing.assert_allclose(info2["d"], -info["d"], rtol=1e-12)


def test_dpo_finite_differences():
    rng = np.random.default_rng(27)
    P, S = 2, 4
    X, W, y, ref = _dpo_problem(rng, P, S, H=3, V=5)
    loss, g, _ = O.flce_dpo(X, W, y, P, S, ref, beta=0.5)
    h = 1e-6
    for (i, j) in [(2, 0), (9, 2)]:
        Xp, Xm = X.copy(), X.copy()
        Xp[i, j] += h
        Xm[i, j] -= h
        fd = (O.flce_dpo(Xp, W, y, P, S, ref, beta=0.5)[0] - O.flce_dpo(Xm, W, y, P, S, ref, beta=0.5)[0]) / (2 * h)
        assert abs(fd - g["X"][i, j]) < 1e-8
    for (i, j) in [(0, 1), (4, 2)]:
        Wp, Wm = W.copy(), W.copy()
        Wp[i, j] += h
        Wm[i, j] -= h
        fd = (O.flce_dpo(X, Wp, y, P, S, ref, beta=0.5)[0] - O.flce_dpo(X, Wm, y, P, S, ref, beta=0.5)[0]) / (2 * h)
        assert abs(fd - g["W"][i, j]) < 1e-8
    assert np.all(g["X"][[0, 1, P * S, P * S + 1]] == 0.0)   # ignored tokens get no gradient
