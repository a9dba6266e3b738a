"""Pins for the fp64 oracle, checked against facts that do not come from the
oracle itself: Gibbs' inequality, closed forms, library routines (torch CPU
fp64 cross_entropy / kl_div / autograd), finite differences, a scalar-loop
evaluation and exhaustive enumeration on a tiny vocabulary."""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import (kl_dense, kl_sparse, kl_chunked, kl_loops, kl_logits, topk_rows,
                    teacher_distribution)


def rand_case(T, H, V, K, seed, tau=1.0, mask_frac=0.0, distinct=True, scale=2.0):
    r = np.random.default_rng(seed)
    h = r.standard_normal((T, H))
    W = r.standard_normal((V, H)) * scale / math.sqrt(H)
    if distinct:
        idx = np.stack([r.choice(V, size=K, replace=False) for _ in range(T)]).astype(np.int32)
    else:
        idx = r.integers(0, V, size=(T, K)).astype(np.int32)
    logit = r.standard_normal((T, K)) * 2.0
    mask = (r.random(T) >= mask_frac).astype(np.uint8)
    return h, W, idx, logit, mask


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


# ---------------------------------------------------------------- sign / bound
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_kl_nonnegative_with_support_bound(seed):
    """Per row KL(P||q) = KL(P||q~) - log Q_S >= -log Q_S >= 0, where Q_S is the
    student mass on the teacher's support and q~ its renormalisation."""
    h, W, idx, logit, mask = rand_case(16, 12, 50, 6, seed, tau=1.3)
    out = kl_dense(h, W, idx, logit, None, tau=1.3, grads=False)
    S = h @ W.T / 1.3
    q = np.exp(S - S.max(1, keepdims=True))
    q /= q.sum(1, keepdims=True)
    QS = np.take_along_axis(q, idx.astype(np.int64), 1).sum(1)
    assert np.all(out["kl"] >= -np.log(QS) - 1e-12)
    assert np.all(-np.log(QS) > 0)


# ------------------------------------------------------------- zero cases
@pytest.mark.parametrize("tau", [1.0, 2.0, 0.7])
def test_zero_when_teacher_is_student_full_vocab(tau):
    """K = V and teacher logits equal to the student's (any slot permutation,
    any per-row shift): loss and both gradients vanish."""
    T, H, V = 6, 10, 24
    r = np.random.default_rng(7)
    h = r.standard_normal((T, H))
    W = r.standard_normal((V, H))
    S = h @ W.T
    idx = np.stack([r.permutation(V) for _ in range(T)]).astype(np.int32)
    logit = np.take_along_axis(S, idx.astype(np.int64), 1) + r.standard_normal((T, 1)) * 5
    out = kl_dense(h, W, idx, logit, None, tau=tau)
    assert abs(out["loss"]) < 1e-12
    assert np.max(np.abs(out["dH"])) < 1e-12
    assert np.max(np.abs(out["dW"])) < 1e-12


def test_no_mask_means_zero():
    h, W, idx, logit, _ = rand_case(5, 8, 30, 4, 3)
    out = kl_dense(h, W, idx, logit, np.zeros(5, np.uint8), tau=1.0)
    assert out["loss"] == 0.0 and out["N"] == 0
    assert not np.any(out["dH"]) and not np.any(out["dW"])


# ------------------------------------------------------------- library pins
@pytest.mark.parametrize("tau", [1.0, 2.5])
def test_k1_is_cross_entropy(tau):
    """K = 1: the teacher is one-hot, KL reduces to the cross-entropy of the
    student at the teacher's token (torch CPU fp64 cross_entropy + autograd)."""
    T, H, V = 9, 7, 33
    h, W, idx, logit, mask = rand_case(T, H, V, 1, 11)
    mask[[2, 5]] = 0
    out = kl_dense(h, W, idx, logit, mask, tau=tau)
    th = torch.tensor(h, requires_grad=True)
    tW = torch.tensor(W, requires_grad=True)
    tgt = torch.tensor(idx[:, 0].astype(np.int64))
    tgt[torch.tensor(mask == 0)] = -100
    loss = torch.nn.functional.cross_entropy(th @ tW.T / tau, tgt, ignore_index=-100,
                                             reduction="mean")
    loss.backward()
    assert abs(out["loss"] - loss.item()) < 1e-12 * max(1.0, abs(loss.item()))
    assert rel(out["dH"], th.grad.numpy()) < 1e-12
    assert rel(out["dW"], tW.grad.numpy()) < 1e-12


@pytest.mark.parametrize("tau,K", [(1.0, 5), (2.0, 12), (0.5, 40)])
def test_matches_torch_kl_div_and_autograd(tau, K):
    """General K: torch fp64 log_softmax + kl_div (x log x with 0 log 0 = 0)
    and autograd gradients."""
    T, H, V = 11, 9, 40
    h, W, idx, logit, mask = rand_case(T, H, V, K, 5 + K, tau=tau)
    mask[0] = 0
    out = kl_dense(h, W, idx, logit, mask, tau=tau)
    th = torch.tensor(h, requires_grad=True)
    tW = torch.tensor(W, requires_grad=True)
    logq = torch.log_softmax(th @ tW.T / tau, dim=1)
    p = torch.softmax(torch.tensor(logit) / tau, dim=1)
    P = torch.zeros(T, V, dtype=torch.float64).scatter_add_(1, torch.tensor(idx.astype(np.int64)), p)
    per_row = torch.nn.functional.kl_div(logq, P, reduction="none").sum(1)
    m = torch.tensor(mask.astype(np.float64))
    loss = (per_row * m).sum() / m.sum()
    loss.backward()
    assert abs(out["loss"] - loss.item()) < 1e-12
    assert rel(out["dH"], th.grad.numpy()) < 1e-11
    assert rel(out["dW"], tW.grad.numpy()) < 1e-11


# ------------------------------------------------------------- closed forms
def test_uniform_student_closed_form():
    """W = 0: q is uniform.  With equal teacher logits p = 1/K, so
    KL_t = log(V/K); dH = 0; dW[v] = sum_t (1/V - [v in S_t]/K) h_t / (N tau)."""
    T, H, V, K, tau = 7, 5, 20, 4, 1.7
    r = np.random.default_rng(2)
    h = r.standard_normal((T, H))
    W = np.zeros((V, H))
    idx = np.stack([r.choice(V, K, replace=False) for _ in range(T)]).astype(np.int32)
    logit = np.full((T, K), 3.25)
    mask = np.ones(T, np.uint8)
    mask[3] = 0
    N = T - 1
    out = kl_dense(h, W, idx, logit, mask, tau=tau)
    assert abs(out["loss"] - math.log(V / K)) < 1e-13
    assert np.max(np.abs(out["dH"])) == 0.0
    dW = np.zeros((V, H))
    for t in range(T):
        if not mask[t]:
            continue
        for v in range(V):
            dW[v] += (1.0 / V - (1.0 / K if v in set(idx[t].tolist()) else 0.0)) * h[t] / (N * tau)
    assert rel(out["dW"], dW) < 1e-13


def test_duplicate_indices_merge():
    """Two cached slots on the same token with equal logits: the teacher puts
    mass 1 on that token, so KL = -log q[v]."""
    h, W, _, _, _ = rand_case(1, 6, 10, 2, 9)
    idx = np.array([[4, 4]], np.int32)
    logit = np.array([[0.3, 0.3]])
    out = kl_dense(h, W, idx, logit, None, tau=1.0)
    S = (h @ W.T)[0]
    logq4 = S[4] - (S.max() + math.log(np.exp(S - S.max()).sum()))
    assert abs(out["loss"] + logq4) < 1e-13
    # sparse / chunked / loop evaluations agree on duplicates
    h, W, idx, logit, mask = rand_case(6, 5, 9, 6, 4, distinct=False)
    a = kl_dense(h, W, idx, logit, mask, tau=1.2)
    assert abs(kl_sparse(h, W, idx, logit, mask, tau=1.2)["loss"] - a["loss"]) < 1e-12
    c = kl_chunked(h, W, idx, logit, mask, tau=1.2, chunk_v=4, chunk_t=2)
    assert abs(c["loss"] - a["loss"]) < 1e-12
    assert rel(c["dH"], a["dH"]) < 1e-12 and rel(c["dW"], a["dW"]) < 1e-12
    lp = kl_loops(h, W, idx, logit, mask, tau=1.2)
    assert abs(lp["loss"] - a["loss"]) < 1e-12
    assert rel(lp["dW"], a["dW"]) < 1e-12


def test_temperature_scaling_identity():
    """L(tau; tau*h, W, tau*u) = L(1; h, W, u) and dH_1(h) = tau*dH_tau(tau*h)."""
    h, W, idx, logit, mask = rand_case(8, 6, 25, 5, 21)
    tau = 2.75
    a = kl_dense(h, W, idx, logit, mask, tau=1.0)
    b = kl_dense(tau * h, W, idx, tau * logit, mask, tau=tau)
    assert abs(a["loss"] - b["loss"]) < 1e-12
    assert rel(a["dH"], tau * b["dH"]) < 1e-12
    assert rel(a["dW"], b["dW"]) < 1e-12


# ------------------------------------------------------------- finite differences
@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_central_finite_differences(tau):
    T, H, V, K = 4, 8, 16, 4
    h, W, idx, logit, mask = rand_case(T, H, V, K, 31)
    mask[2] = 0
    out = kl_dense(h, W, idx, logit, mask, tau=tau)
    eps = 1e-5

    def f(hh, WW):
        return kl_dense(hh, WW, idx, logit, mask, tau=tau, grads=False)["loss"]

    fd_h = np.zeros_like(h)
    for i in range(T):
        for j in range(H):
            hp = h.copy(); hp[i, j] += eps
            hm = h.copy(); hm[i, j] -= eps
            fd_h[i, j] = (f(hp, W) - f(hm, W)) / (2 * eps)
    fd_W = np.zeros_like(W)
    for i in range(V):
        for j in range(H):
            Wp = W.copy(); Wp[i, j] += eps
            Wm = W.copy(); Wm[i, j] -= eps
            fd_W[i, j] = (f(h, Wp) - f(h, Wm)) / (2 * eps)
    assert rel(out["dH"], fd_h) < 1e-7
    assert rel(out["dW"], fd_W) < 1e-7
    assert np.all(out["dH"][2] == 0.0)


# ------------------------------------------------------------- brute force
@pytest.mark.parametrize("tau", [1.0, 1.6])
def test_scalar_loops_match_dense(tau):
    h, W, idx, logit, mask = rand_case(3, 5, 11, 4, 17, tau=tau)
    mask[1] = 0
    a = kl_dense(h, W, idx, logit, mask, tau=tau)
    b = kl_loops(h, W, idx, logit, mask, tau=tau)
    assert abs(a["loss"] - b["loss"]) < 1e-13
    assert rel(a["dH"], b["dH"]) < 1e-12
    assert rel(a["dW"], b["dW"]) < 1e-12
    assert np.allclose(a["row_loss"], b["row_loss"], atol=1e-13, rtol=0)


def test_exhaustive_support_and_chunking_v8():
    """Every K-subset of an 8-token vocabulary (K = 1..3) under every chunk
    size 1..8: the chunked two-pass evaluation equals the dense one.  This
    places teacher tokens at every position relative to a chunk boundary."""
    V, H = 8, 3
    r = np.random.default_rng(123)
    h = r.standard_normal((2, H))
    W = r.standard_normal((V, H))
    for K in (1, 2, 3):
        for sub in itertools.combinations(range(V), K):
            idx = np.array([list(sub), list(reversed(sub))], np.int32)
            logit = r.standard_normal((2, K))
            ref = kl_dense(h, W, idx, logit, None, tau=1.3)
            lp = kl_loops(h, W, idx, logit, None, tau=1.3)
            assert abs(lp["loss"] - ref["loss"]) < 1e-13
            for cv in range(1, V + 1):
                c = kl_chunked(h, W, idx, logit, None, tau=1.3, chunk_v=cv, chunk_t=1)
                assert abs(c["loss"] - ref["loss"]) < 1e-13
                assert rel(c["dH"], ref["dH"]) < 1e-12
                assert rel(c["dW"], ref["dW"]) < 1e-12


# ------------------------------------------------------------- chunk invariance
@pytest.mark.parametrize("cv,ct", [(1, 5), (7, 3), (1000, 64), (1024, 17), (3000, 1)])
def test_chunk_invariance(cv, ct):
    T, H, V, K = 24, 16, 3000, 8
    h, W, idx, logit, mask = rand_case(T, H, V, K, 41, tau=1.0, mask_frac=0.2)
    if cv == 1:      # keep the per-chunk Python loop short
        T = 6
        h, idx, logit, mask = h[:T], idx[:T], logit[:T], mask[:T]
    ref = kl_dense(h, W, idx, logit, mask, tau=1.5)
    c = kl_chunked(h, W, idx, logit, mask, tau=1.5, chunk_v=cv, chunk_t=ct)
    assert abs(c["loss"] - ref["loss"]) <= 1e-12 * abs(ref["loss"])
    assert np.allclose(c["lse"], ref["lse"], rtol=1e-13, atol=0)
    assert rel(c["dH"], ref["dH"]) < 1e-12
    assert rel(c["dW"], ref["dW"]) < 1e-12


# ------------------------------------------------------------- invariances
def test_invariances():
    h, W, idx, logit, mask = rand_case(10, 7, 60, 9, 55, mask_frac=0.3)
    ref = kl_dense(h, W, idx, logit, mask, tau=1.1)
    r = np.random.default_rng(0)
    # permuting the K slots
    perm = r.permutation(9)
    a = kl_dense(h, W, idx[:, perm], logit[:, perm], mask, tau=1.1)
    assert abs(a["loss"] - ref["loss"]) < 1e-13 and rel(a["dW"], ref["dW"]) < 1e-13
    # permuting rows together with the mask
    rp = r.permutation(10)
    b = kl_dense(h[rp], W, idx[rp], logit[rp], mask[rp], tau=1.1)
    assert abs(b["loss"] - ref["loss"]) < 1e-13
    assert rel(b["dH"], ref["dH"][rp]) < 1e-13 and rel(b["dW"], ref["dW"]) < 1e-12
    # adding a per-row constant to the cached teacher logits
    c = kl_dense(h, W, idx, logit + r.standard_normal((10, 1)) * 4, mask, tau=1.1)
    assert abs(c["loss"] - ref["loss"]) < 1e-12 and rel(c["dH"], ref["dH"]) < 1e-12


def test_gradient_structure():
    """Each row of the logit gradient sums to zero (both distributions sum to
    one), hence sum_v dW[v,:] = 0; masked rows get dH = 0."""
    h, W, idx, logit, mask = rand_case(12, 8, 70, 6, 77, mask_frac=0.25)
    out = kl_dense(h, W, idx, logit, mask, tau=0.9)
    assert np.max(np.abs(out["dW"].sum(0))) < 1e-13 * max(1.0, np.abs(out["dW"]).max() * 70)
    assert np.all(out["dH"][mask == 0] == 0.0)
    assert np.all(np.isfinite(out["dH"]))


def test_masked_rows_ignore_their_teacher_data():
    h, W, idx, logit, mask = rand_case(6, 5, 20, 3, 8)
    mask[4] = 0
    ref = kl_dense(h, W, idx, logit, mask)
    logit2 = logit.copy()
    logit2[4] = np.nan
    a = kl_dense(h, W, idx, logit2, mask)
    assert a["loss"] == ref["loss"]
    assert np.array_equal(a["dW"], ref["dW"])


def test_teacher_distribution_softmax_library():
    """Teacher renormalisation over K equals torch.softmax (fp64) and sums to 1;
    -inf cached logits carry no mass."""
    r = np.random.default_rng(3)
    u = r.standard_normal((5, 7)) * 3
    u[1, 2] = -np.inf
    p = teacher_distribution(u, 1.7)
    ref = torch.softmax(torch.tensor(u) / 1.7, dim=1).numpy()
    assert np.max(np.abs(p - ref)) < 1e-15
    assert np.allclose(p.sum(1), 1.0, atol=1e-15)
    assert p[1, 2] == 0.0


# ------------------------------------------------ forward-chunked (given logits)
@pytest.mark.parametrize("tau,K", [(1.0, 5), (2.5, 17)])
def test_kl_logits_matches_torch_kl_div_and_autograd(tau, K):
    """Loss on given student logits Z against torch fp64 log_softmax + kl_div,
    and dZ against torch autograd with respect to Z."""
    T, V = 9, 60
    r = np.random.default_rng(40 + K)
    Z = r.standard_normal((T, V)) * 3.0
    idx = np.stack([r.choice(V, K, replace=False) for _ in range(T)]).astype(np.int32)
    logit = r.standard_normal((T, K)) * 2.0
    mask = np.ones(T, np.uint8)
    mask[[2, 7]] = 0
    out = kl_logits(Z, idx, logit, mask, tau=tau)
    tZ = torch.tensor(Z, requires_grad=True)
    logq = torch.log_softmax(tZ / tau, dim=1)
    p = torch.softmax(torch.tensor(logit) / tau, dim=1)
    P = torch.zeros(T, V, dtype=torch.float64).scatter_add_(1, torch.tensor(idx.astype(np.int64)), p)
    per_row = torch.nn.functional.kl_div(logq, P, reduction="none").sum(1)
    m = torch.tensor(mask.astype(np.float64))
    loss = (per_row * m).sum() / m.sum()
    loss.backward()
    assert abs(out["loss"] - loss.item()) < 1e-12
    assert rel(out["dZ"], tZ.grad.numpy()) < 1e-11
    assert np.all(out["dZ"][[2, 7]] == 0.0)


def test_kl_logits_closed_forms_and_invariances():
    """Z = 0 (uniform student): KL_t = sum_k p log p + log V and
    dZ = (1/V - P)/(N tau); a per-row constant added to Z changes nothing;
    every row of dZ sums to zero."""
    T, V, K, tau = 6, 25, 4, 1.3
    r = np.random.default_rng(3)
    idx = np.stack([r.choice(V, K, replace=False) for _ in range(T)]).astype(np.int32)
    logit = r.standard_normal((T, K))
    out = kl_logits(np.zeros((T, V)), idx, logit, None, tau=tau)
    u = logit / tau
    p = np.exp(u - u.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    kl = np.sum(p * np.log(p), axis=1) + math.log(V)
    assert np.max(np.abs(out["kl"] - kl)) < 1e-13
    dz = np.full((T, V), 1.0 / V)
    for t in range(T):
        dz[t, idx[t]] -= p[t]
    assert rel(out["dZ"], dz / (T * tau)) < 1e-13
    Z = r.standard_normal((T, V)) * 2
    a = kl_logits(Z, idx, logit, None, tau=tau)
    b = kl_logits(Z + r.standard_normal((T, 1)) * 50, idx, logit, None, tau=tau)
    assert abs(a["loss"] - b["loss"]) < 1e-11
    assert rel(a["dZ"], b["dZ"]) < 1e-11
    assert np.max(np.abs(a["dZ"].sum(1))) < 1e-15


def test_kl_logits_finite_differences():
    T, V, K, tau = 3, 12, 3, 1.7
    r = np.random.default_rng(8)
    Z = r.standard_normal((T, V))
    idx = np.stack([r.choice(V, K, replace=False) for _ in range(T)]).astype(np.int32)
    logit = r.standard_normal((T, K))
    mask = np.array([1, 0, 1], np.uint8)
    out = kl_logits(Z, idx, logit, mask, tau=tau)
    eps = 1e-5
    fd = np.zeros_like(Z)
    for i in range(T):
        for j in range(V):
            zp = Z.copy(); zp[i, j] += eps
            zm = Z.copy(); zm[i, j] -= eps
            fd[i, j] = (kl_logits(zp, idx, logit, mask, tau, grads=False)["loss"]
                        - kl_logits(zm, idx, logit, mask, tau, grads=False)["loss"]) / (2 * eps)
    assert rel(out["dZ"], fd) < 1e-7


# ------------------------------------------------------------ top-K selection
def test_topk_rows_brute_force_with_ties():
    """Against a pure-Python sort of (value, id) pairs, on rows full of ties."""
    r = np.random.default_rng(9)
    X = r.integers(-3, 4, size=(7, 23)).astype(np.float32)
    X[2] = 1.0                      # a row of one value: ids 0..K-1
    for K in (1, 5, 23):
        idx, vals = topk_rows(X, K)
        for t in range(X.shape[0]):
            ref = sorted(range(X.shape[1]), key=lambda v: (-float(X[t, v]), v))[:K]
            assert idx[t].tolist() == ref
            assert vals[t].tolist() == [float(X[t, v]) for v in ref]
    assert topk_rows(X, 4)[0][2].tolist() == [0, 1, 2, 3]


def test_topk_rows_distinct_values_match_library_selection():
    r = np.random.default_rng(10)
    X = r.standard_normal((5, 1000))
    idx, vals = topk_rows(X, 64)
    for t in range(5):
        top = np.argpartition(-X[t], 64)[:64]
        assert set(top.tolist()) == set(idx[t].tolist())
        assert np.all(np.diff(vals[t]) < 0)
