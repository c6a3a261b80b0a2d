"""FP64 CPU oracle for fused linear cross-entropy (FLCE), standalone
cross-entropy (CE) and per-shard vocabulary statistics.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module. The HIP library never
calls it, and it shares no code with the HIP library: it is plain NumPy in
float64, written from the definitions, so a reader can check it by eye.

Sources (web pages in the reference set):
  * "liger-kernel 0.0.1 -> 0.1.1" package diff, README section "Kernels":
    CrossEntropy is PyTorch's CrossEntropyLoss (linked there as the definition),
    computed together with its gradient; FusedLinearCrossEntropy fuses the model
    head with that loss and chunks the input rows; "Key Features": the
    computation is exact, with no approximation.
  * "Peak performance, minimized memory" (torchtune + Liger blog), text under
    Figure 1 "Fused Linear Cross Entropy": flatten [B, S, H] to [B*S, H], apply
    the head on row chunks, take each chunk's loss and logits gradient, then
    derive the hidden-state gradient and accumulate the head gradient.
  * DeepSpeed PR "opt-in Liger vocab-parallel CE backend", sections "Changes"
    and "Real-device validation": reductions none/sum/mean, ignored targets,
    vocabulary shards across tensor-parallel ranks.

Readings where the pages say nothing (each is also listed in the design notes):
  * loss_n = logsumexp(z_n) - z_n[y_n]; a row is ignored iff y_n == ignore_index;
    a row whose target is not ignored but lies outside [0, V) is "bad": it is
    treated as ignored and reported.
  * mean divides by the number of rows that are neither ignored nor bad; with
    no such row the loss and every gradient are 0 (PyTorch would give NaN).
  * reduction "none" returns per-row losses; its gradients are those of their
    sum (an all-ones upstream gradient).
  * the optional head bias b enters as z = x W^T + b; its gradient is the
    column sum of dZ.
  * shard statistics are taken relative to the shard's own maximum; the target
    logit is 0 when the target is outside the shard or the row is ignored.
  * distillation loss: the standard Jensen-Shannon divergence (equal weights,
    M = (P + Q) / 2) between softmax(student / T) and softmax(teacher / T), no
    T^2 factor; the teacher is frozen; target ids only mask rows.
  * DPO: the standard sigmoid preference loss on sequence log-probabilities
    summed over non-ignored target tokens, reference log-probabilities given
    as inputs, mean over pairs.
  * a shard's backward takes the global per-row lse as input (the pages
    exchange the statistics, not the gradient); validity and the mean's
    N_valid are judged against the whole vocabulary.

Every function here evaluates the plain definition. The only partition is the
row blocking of `flce`, which the FLCE description itself prescribes (rows are
independent, so blocking changes nothing but the order of the grad_W sum); for
inputs of at most `row_block` rows there is no blocking at all.
"""

import numpy as np

REDUCTIONS = ("none", "sum", "mean")


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def target_masks(targets, V, ignore_index):
    """Row classification for targets y (any integer array).

    valid[n]: y_n != ignore_index and 0 <= y_n < V (the row contributes).
    bad[n]:   y_n != ignore_index and y_n outside [0, V) (reported, then
              treated like an ignored row).
    """
    y = np.asarray(targets).astype(np.int64)
    not_ignored = y != int(ignore_index)
    in_range = (y >= 0) & (y < V)
    return not_ignored & in_range, not_ignored & ~in_range


def reduction_scale(n_valid, reduction):
    """Factor applied to each row's loss gradient: 1/N_valid for mean (0 when
    N_valid is 0), else 1 (sum, and none whose gradient is that of the sum)."""
    if reduction not in REDUCTIONS:
        raise ValueError(f"unknown reduction {reduction!r}")
    if reduction == "mean":
        return 1.0 / n_valid if n_valid > 0 else 0.0
    return 1.0


def logsumexp_rows(Z):
    """lse_n = M_n + ln sum_v exp(Z[n, v] - M_n) with M_n = max_v Z[n, v]."""
    Z = _f64(Z)
    M = Z.max(axis=1)
    return M + np.log(np.exp(Z - M[:, None]).sum(axis=1))


def _rows_loss_and_dlogits(Z, y, valid, scale):
    """Per-row CE loss and the gradient of scale * sum(loss) w.r.t. Z.

    loss_n = lse_n - Z[n, y_n] for valid rows, 0 otherwise;
    dZ[n, :] = scale * (softmax(Z[n, :]) - onehot(y_n)) for valid rows, 0 otherwise.
    """
    Z = _f64(Z)
    n_rows = Z.shape[0]
    lse = logsumexp_rows(Z)
    rows = np.arange(n_rows)
    ysafe = np.where(valid, y, 0)
    z_target = Z[rows, ysafe]
    loss = np.where(valid, lse - z_target, 0.0)
    P = np.exp(Z - lse[:, None])
    P[rows[valid], ysafe[valid]] -= 1.0
    dZ = scale * P * valid[:, None]
    return loss, dZ


def _reduce(loss_rows, n_valid, reduction):
    if reduction == "none":
        return loss_rows.copy()
    total = float(loss_rows.sum())
    if reduction == "sum":
        return total
    return total / n_valid if n_valid > 0 else 0.0


def cross_entropy(logits, targets, ignore_index=-100, reduction="mean"):
    """Cross-entropy over given logits [N, V] and its gradient.

    Returns (loss, grad_logits, info): loss is a float (sum/mean) or an [N]
    array (none); grad_logits is [N, V] float64; info holds n_valid, n_bad and
    the per-row losses.
    """
    Z = _f64(logits)
    N, V = Z.shape
    y = np.asarray(targets).astype(np.int64)
    valid, bad = target_masks(y, V, ignore_index)
    n_valid = int(valid.sum())
    scale = reduction_scale(n_valid, reduction)
    loss_rows, dZ = _rows_loss_and_dlogits(Z, y, valid, scale)
    info = {"n_valid": n_valid, "n_bad": int(bad.sum()), "loss_rows": loss_rows}
    return _reduce(loss_rows, n_valid, reduction), dZ, info


def flce(X, W, targets, bias=None, ignore_index=-100, reduction="mean",
         row_block=1024, want_grads=True):
    """Fused linear cross-entropy: loss of CE(X W^T + b, y) and its gradients.

    X [N, H], W [V, H] (lm_head weight, nn.Linear layout), bias [V] or None,
    targets [N]. Logits are materialised one row block at a time, in float64.
    Returns (loss, grads, info) with grads = {"X": [N, H], "W": [V, H],
    "bias": [V] or None} (None entries when want_grads is False).
    """
    X = _f64(X)
    W = _f64(W)
    N, H = X.shape
    V = W.shape[0]
    if W.shape[1] != H:
        raise ValueError("X and W disagree on H")
    b = None if bias is None else _f64(bias)
    y = np.asarray(targets).astype(np.int64)
    valid, bad = target_masks(y, V, ignore_index)
    n_valid = int(valid.sum())
    scale = reduction_scale(n_valid, reduction)

    loss_rows = np.zeros(N)
    gX = np.zeros((N, H)) if want_grads else None
    gW = np.zeros((V, H)) if want_grads else None
    gb = (np.zeros(V) if b is not None else None) if want_grads else None
    for r0 in range(0, N, max(1, int(row_block))):
        r1 = min(N, r0 + int(row_block))
        Xb = X[r0:r1]
        Z = Xb @ W.T
        if b is not None:
            Z = Z + b[None, :]
        lr, dZ = _rows_loss_and_dlogits(Z, y[r0:r1], valid[r0:r1], scale)
        loss_rows[r0:r1] = lr
        if want_grads:
            gX[r0:r1] = dZ @ W
            gW += dZ.T @ Xb
            if gb is not None:
                gb += dZ.sum(axis=0)
    info = {"n_valid": n_valid, "n_bad": int(bad.sum()), "loss_rows": loss_rows}
    return _reduce(loss_rows, n_valid, reduction), {"X": gX, "W": gW, "bias": gb}, info


def flce_rows(X, W, targets, rows, bias=None, ignore_index=-100, reduction="mean"):
    """Loss and grad_X for selected rows only (grad_X of a row needs only that
    row), with the reduction scale of the whole batch. Used to check sampled
    rows of large problems. Returns (loss_rows [R], grad_X [R, H])."""
    X = _f64(X)
    W = _f64(W)
    V = W.shape[0]
    y = np.asarray(targets).astype(np.int64)
    valid, _ = target_masks(y, V, ignore_index)
    scale = reduction_scale(int(valid.sum()), reduction)
    rows = np.asarray(rows, dtype=np.int64)
    Z = X[rows] @ W.T
    if bias is not None:
        Z = Z + _f64(bias)[None, :]
    lr, dZ = _rows_loss_and_dlogits(Z, y[rows], valid[rows], scale)
    return lr, dZ @ W


def flce_sampled(X, W, targets, token_rows, vocab_rows, bias=None, ignore_index=-100,
                 reduction="mean", row_block=1024):
    """`flce` for shapes whose full gradients are too large to keep: the loss
    of every row and the reduced loss, with grad_X only for the listed token
    rows and grad_W / grad_bias only for the listed vocabulary rows. The same
    definition and row blocking as `flce`, in one pass over the row blocks:
    each block's logits are materialised, its loss rows and dlogits taken,
    and only the requested gradient rows kept.

    Returns (loss, loss_rows [N], grad_X_rows [R, H], grad_W_rows [Q, H],
    grad_bias_rows [Q] or None, n_valid)."""
    X = _f64(X)
    W = _f64(W)
    N, H = X.shape
    V = W.shape[0]
    b = None if bias is None else _f64(bias)
    y = np.asarray(targets).astype(np.int64)
    valid, _ = target_masks(y, V, ignore_index)
    n_valid = int(valid.sum())
    scale = reduction_scale(n_valid, reduction)
    tr = np.asarray(token_rows, dtype=np.int64)
    vr = np.asarray(vocab_rows, dtype=np.int64)
    loss_rows = np.zeros(N)
    gX = np.zeros((len(tr), H))
    gW = np.zeros((len(vr), H))
    gb = np.zeros(len(vr)) if b is not None else None
    for r0 in range(0, N, max(1, int(row_block))):
        r1 = min(N, r0 + int(row_block))
        Xb = X[r0:r1]
        Z = Xb @ W.T
        if b is not None:
            Z = Z + b[None, :]
        lr, dZ = _rows_loss_and_dlogits(Z, y[r0:r1], valid[r0:r1], scale)
        loss_rows[r0:r1] = lr
        here = np.flatnonzero((tr >= r0) & (tr < r1))
        if len(here):
            gX[here] = dZ[tr[here] - r0] @ W
        gW += dZ[:, vr].T @ Xb
        if gb is not None:
            gb += dZ[:, vr].sum(axis=0)
    return _reduce(loss_rows, n_valid, reduction), loss_rows, gX, gW, gb, n_valid


def flce_grad_w_rows(X, W, targets, vocab_rows, bias=None, ignore_index=-100,
                     reduction="mean", row_block=1024):
    """grad_W[v, :] and grad_bias[v] for selected vocabulary rows v, summed over
    every token row (dZ[:, v] needs each token row's full logsumexp). Returns
    (grad_W_rows [R, H], grad_bias_rows [R])."""
    X = _f64(X)
    W = _f64(W)
    N, H = X.shape
    V = W.shape[0]
    y = np.asarray(targets).astype(np.int64)
    valid, _ = target_masks(y, V, ignore_index)
    scale = reduction_scale(int(valid.sum()), reduction)
    vr = np.asarray(vocab_rows, dtype=np.int64)
    b = None if bias is None else _f64(bias)
    gW = np.zeros((len(vr), H))
    gb = np.zeros(len(vr))
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        Z = X[r0:r1] @ W.T
        if b is not None:
            Z = Z + b[None, :]
        _, dZ = _rows_loss_and_dlogits(Z, y[r0:r1], valid[r0:r1], scale)
        gW += dZ[:, vr].T @ X[r0:r1]
        gb += dZ[:, vr].sum(axis=0)
    return gW, gb


def shard_stats(logits_shard, targets, vocab_start, V_global, ignore_index=-100):
    """Per-row statistics of one vocabulary shard [N, V_local] covering global
    ids [vocab_start, vocab_start + V_local).

    m_n = max over the shard; s_n = sum over the shard of exp(z - m_n);
    t_n = z[n, y_n - vocab_start] if row n is valid (w.r.t. V_global) and its
    target falls in the shard, else 0.
    """
    Z = _f64(logits_shard)
    N, Vl = Z.shape
    y = np.asarray(targets).astype(np.int64)
    valid, _ = target_masks(y, V_global, ignore_index)
    m = Z.max(axis=1)
    s = np.exp(Z - m[:, None]).sum(axis=1)
    local = y - int(vocab_start)
    here = valid & (local >= 0) & (local < Vl)
    t = np.where(here, Z[np.arange(N), np.where(here, local, 0)], 0.0)
    return m, s, t


def combine_shard_stats(stats):
    """Combine per-shard (m, s, t) into (lse, target logit) per row:
    M = max_k m_k, S = sum_k s_k exp(m_k - M), lse = M + ln S, z_y = sum_k t_k."""
    ms = np.stack([_f64(st[0]) for st in stats])
    ss = np.stack([_f64(st[1]) for st in stats])
    ts = np.stack([_f64(st[2]) for st in stats])
    M = ms.max(axis=0)
    S = (ss * np.exp(ms - M[None, :])).sum(axis=0)
    return M + np.log(S), ts.sum(axis=0)


def flce_shard_stats(X, W_shard, targets, vocab_start, V_global, bias_shard=None,
                     ignore_index=-100, row_block=1024):
    """Shard statistics of the logits X W_shard^T (+ bias_shard), materialised
    one row block at a time."""
    X = _f64(X)
    Ws = _f64(W_shard)
    y = np.asarray(targets).astype(np.int64)
    N = X.shape[0]
    out = [np.zeros(N), np.zeros(N), np.zeros(N)]
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        Z = X[r0:r1] @ Ws.T
        if bias_shard is not None:
            Z = Z + _f64(bias_shard)[None, :]
        m, s, t = shard_stats(Z, y[r0:r1], vocab_start, V_global, ignore_index)
        out[0][r0:r1], out[1][r0:r1], out[2][r0:r1] = m, s, t
    return tuple(out)


def shard_loss(lse, z_target, targets, V_global, ignore_index=-100, reduction="mean"):
    """The global loss from combined shard statistics: loss_n = lse_n - z_y for
    rows valid w.r.t. the whole vocabulary, 0 otherwise, then reduced.
    Returns (loss, loss_rows, n_valid)."""
    y = np.asarray(targets).astype(np.int64)
    valid, _ = target_masks(y, V_global, ignore_index)
    n_valid = int(valid.sum())
    rows = np.where(valid, _f64(lse) - _f64(z_target), 0.0)
    return _reduce(rows, n_valid, reduction), rows, n_valid


def flce_shard_backward(X, W_shard, targets, vocab_start, V_global, lse, bias_shard=None,
                        ignore_index=-100, reduction="mean", row_block=1024):
    """The part of the global FLCE gradients that one vocabulary shard owns
    (DeepSpeed vocab-parallel CE page: each rank holds the head rows of its
    vocabulary range; the per-row normaliser is global).

    With z = X W_shard^T (+ b_shard) over global ids [vocab_start,
    vocab_start + V_local) and the global lse_n of every row:
      dZ[n, j] = scale * (exp(z[n, j] - lse_n) - [vocab_start + j == y_n])
    for rows valid w.r.t. V_global (0 for the others), scale = 1/N_valid
    (mean) or 1; then
      grad_X partial = dZ W_shard   (the shards' partials sum to grad_X),
      grad_W_shard   = dZ^T X       (rows [vocab_start, ...) of grad_W),
      grad_b_shard   = column sums of dZ.
    Returns (grad_X_partial, grad_W_shard, grad_b_shard or None).
    """
    X = _f64(X)
    Ws = _f64(W_shard)
    lse = _f64(lse)
    y = np.asarray(targets).astype(np.int64)
    N = X.shape[0]
    Vl = Ws.shape[0]
    valid, _ = target_masks(y, V_global, ignore_index)
    scale = reduction_scale(int(valid.sum()), reduction)
    gX = np.zeros_like(X)
    gW = np.zeros_like(Ws)
    gb = np.zeros(Vl) if bias_shard is not None else None
    cols = int(vocab_start) + np.arange(Vl)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        Z = X[r0:r1] @ Ws.T
        if bias_shard is not None:
            Z = Z + _f64(bias_shard)[None, :]
        onehot = (cols[None, :] == y[r0:r1, None]).astype(np.float64)
        dZ = scale * (np.exp(Z - lse[r0:r1, None]) - onehot)
        dZ[~valid[r0:r1]] = 0.0
        gX[r0:r1] = dZ @ Ws
        gW += dZ.T @ X[r0:r1]
        if gb is not None:
            gb += dZ.sum(axis=0)
    return gX, gW, gb


def flce_multihead(X, Ws, targets, biases=None, ignore_index=-100, reduction="mean",
                   row_block=1024):
    """K LM heads over the same hidden states (the Medusa example of the liger
    README): head k is an FLCE of X with its own weight Ws[k], bias and
    targets[k]; the objective is the sum of the K head losses, so grad_X is
    the sum of the heads' grad_X. Returns (losses [K] or [K, N],
    {"X", "W" [K, V, H], "bias" [K, V] or None})."""
    K = len(Ws)
    losses, gX, gW, gb = [], None, [], []
    for k in range(K):
        b = None if biases is None else biases[k]
        loss, g, _ = flce(X, Ws[k], targets[k], bias=b, ignore_index=ignore_index,
                          reduction=reduction, row_block=row_block)
        losses.append(loss)
        gX = g["X"] if gX is None else gX + g["X"]
        gW.append(g["W"])
        gb.append(g["bias"])
    return np.array(losses), {"X": gX, "W": np.stack(gW),
                              "bias": None if biases is None else np.stack(gb)}


def _log_softmax_rows(Z):
    Z = _f64(Z)
    return Z - logsumexp_rows(Z)[:, None]


def jsd_rows(Zs, Zt, temperature=1.0):
    """Per-row Jensen-Shannon divergence between the student and teacher
    distributions P = softmax(Zs / T), Q = softmax(Zt / T):
    JSD = 1/2 KL(P || M) + 1/2 KL(Q || M) with M = (P + Q) / 2, and its
    gradient w.r.t. the student logits Zs:
    dJSD/dZs = (1/T) P * (g - sum_v P g),  g = 1/2 ln(P / M)
    (d/dP of the divergence is 1/2 ln(P/M); the softmax Jacobian gives the rest).
    Returns (jsd [n], dZs [n, V])."""
    T = float(temperature)
    lp = _log_softmax_rows(_f64(Zs) / T)
    lq = _log_softmax_rows(_f64(Zt) / T)
    P, Q = np.exp(lp), np.exp(lq)
    mx = np.maximum(lp, lq)
    lm = mx + np.log(0.5 * (np.exp(lp - mx) + np.exp(lq - mx)))   # ln M, without underflow
    jsd = 0.5 * (P * (lp - lm)).sum(axis=1) + 0.5 * (Q * (lq - lm)).sum(axis=1)
    g = 0.5 * (lp - lm)
    dZ = (P * (g - (P * g).sum(axis=1, keepdims=True))) / T
    return jsd, dZ


def flce_jsd(Xs, Ws, Xt, Wt, targets, temperature=1.0, ignore_index=-100, reduction="mean",
             row_block=1024):
    """Fused linear Jensen-Shannon distillation loss (the knowledge-distillation
    member of the chunked-loss family the Megatron integration page lists): the
    student head Zs = Xs Ws^T and the frozen teacher head Zt = Xt Wt^T over the
    same vocabulary; loss rows are the JSD of the tempered distributions, rows
    whose target is ignore_index (or outside [0, V)) are masked out, reduced
    like CE. Returns (loss, {"X": grad_Xs, "W": grad_Ws}, info)."""
    Xs, Ws, Xt, Wt = _f64(Xs), _f64(Ws), _f64(Xt), _f64(Wt)
    y = np.asarray(targets).astype(np.int64)
    N = Xs.shape[0]
    V = Ws.shape[0]
    valid, _ = target_masks(y, V, ignore_index)
    n_valid = int(valid.sum())
    scale = reduction_scale(n_valid, reduction)
    rows = np.zeros(N)
    gX = np.zeros_like(Xs)
    gW = np.zeros_like(Ws)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        jsd, dZ = jsd_rows(Xs[r0:r1] @ Ws.T, Xt[r0:r1] @ Wt.T, temperature)
        v = valid[r0:r1]
        rows[r0:r1] = np.where(v, jsd, 0.0)
        dZ = scale * dZ * v[:, None]
        gX[r0:r1] = dZ @ Ws
        gW += dZ.T @ Xs[r0:r1]
    return _reduce(rows, n_valid, reduction), {"X": gX, "W": gW}, {"n_valid": n_valid, "loss_rows": rows}


def flce_dpo(X, W, targets, n_pairs, seq_len, ref_logps, beta=0.1, ignore_index=-100,
             row_block=1024):
    """Fused linear DPO loss (the alignment member of the chunked-loss family
    on the Megatron integration page; the torchtune blog plans its recipe):
    X holds 2 * n_pairs sequences of seq_len token rows, the n_pairs chosen
    sequences first, then the rejected ones in the same pair order. A
    sequence's log-probability is the sum over its non-ignored rows of
    log softmax(x W^T)[target] = -(CE row loss); with the reference model's
    sequence log-probabilities ref_logps [2 * n_pairs] (same order),
      d_b = beta * ((logp_w - ref_w) - (logp_l - ref_l)),
      loss = mean_b softplus(-d_b)  (= -log sigmoid(d_b)).
    Gradients: each token row of pair b gets dZ = s (softmax - onehot) with
    s = +beta sigmoid(-d_b) / n_pairs on chosen rows and the negative on
    rejected rows. Returns (loss, {"X", "W"}, {"logps", "d", "pair_loss"})."""
    X, W = _f64(X), _f64(W)
    y = np.asarray(targets).astype(np.int64)
    N = X.shape[0]
    assert N == 2 * n_pairs * seq_len
    V = W.shape[0]
    valid, _ = target_masks(y, V, ignore_index)
    loss_rows = np.zeros(N)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        lr, _ = _rows_loss_and_dlogits(X[r0:r1] @ W.T, y[r0:r1], valid[r0:r1], 1.0)
        loss_rows[r0:r1] = lr
    logps = -loss_rows.reshape(2 * n_pairs, seq_len).sum(axis=1)
    ref = _f64(ref_logps)
    d = beta * ((logps[:n_pairs] - ref[:n_pairs]) - (logps[n_pairs:] - ref[n_pairs:]))
    pair_loss = np.logaddexp(0.0, -d)
    sig = 1.0 / (1.0 + np.exp(d))                      # sigmoid(-d)
    coef = np.concatenate([beta * sig, -beta * sig]) / n_pairs
    row_scale = np.repeat(coef, seq_len)
    gX = np.zeros_like(X)
    gW = np.zeros_like(W)
    for r0 in range(0, N, row_block):
        r1 = min(N, r0 + row_block)
        _, dZ = _rows_loss_and_dlogits(X[r0:r1] @ W.T, y[r0:r1], valid[r0:r1], 1.0)
        dZ = dZ * row_scale[r0:r1, None]
        gX[r0:r1] = dZ @ W
        gW += dZ.T @ X[r0:r1]
    return float(pair_loss.mean()), {"X": gX, "W": gW}, {"logps": logps, "d": d,
                                                         "pair_loss": pair_loss}


def shift_labels(labels, ignore_index=-100):
    """Causal-LM targets from labels [B, S]: position s of sequence b predicts
    token s + 1, so targets[b, s] = labels[b, s + 1] and the last position of
    each sequence has no target (ignore_index). Returns int32 [B * S]
    (DeepSpeed vocab-parallel CE page, "Changes": the loss keeps the label
    shift of causal language modelling)."""
    lab = np.asarray(labels)
    B, S = lab.shape
    out = np.full((B, S), ignore_index, dtype=np.int64)
    out[:, :-1] = lab[:, 1:]
    return out.reshape(B * S).astype(np.int32)


def materialised_logits_bytes(n_tokens, vocab, elem_bytes):
    """Bytes of a full [tokens, vocab] logits tensor: what FLCE avoids holding."""
    return int(n_tokens) * int(vocab) * int(elem_bytes)
