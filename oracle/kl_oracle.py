"""fp64 CPU oracle for the fused chunked top-K KL distillation loss.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only tests/, __graft_entry__.smoke() and the cpu_baseline leg
of bench.py use it.  It shares no code with the HIP library and does not
import it.

What is computed (sources: page "Making Knowledge Distillation Cheap Enough to
Run at Scale", section "Two systems changes", the three loss variants; page
"Efficient Knowledge Distillation for LLMs: Offline Top-K Logits and a Fused
Chunked KL Loss", abstract):

  inputs   h[T,H] hidden states, W[V,H] output-head weight, the teacher's cached
           top-K per position: teacher_idx[T,K] (vocabulary ids) and
           teacher_logit[T,K]; mask[T] (1 = position counts); temperature tau.
  student  S = h W^T (the output projection), log q = log_softmax(S/tau) over
           the whole vocabulary (the student's dense grid of log-probabilities
           that the Dense KL variant compares against).
  teacher  p[t,k] = softmax_k(teacher_logit[t,k]/tau): the teacher distribution
           is rebuilt from the cached top-K logits alone, so it is renormalised
           over those K entries (the dropped tail carries no mass).  On the
           vocabulary, P[t,v] = sum_k p[t,k] [teacher_idx[t,k] == v].
  loss     KL_t = sum_v P[t,v] (log P[t,v] - log q[t,v]), with 0 log 0 = 0;
           loss = (1/N) sum_t mask_t KL_t, N = sum_t mask_t (loss = 0 if N = 0).
  grads    G[t,v] = mask_t/(N tau) (q[t,v] - P[t,v]);  dH = G W;  dW = G^T h.

Readings where the pages say nothing (each listed in the design notes):
  * tau divides both teacher and student logits; no tau^2 factor.
  * forward KL(teacher || student) with the entropy term kept (a true KL).
  * mean over unmasked positions; masked rows contribute exactly 0 to loss and
    gradients (their teacher data is not used).
  * duplicate teacher indices in a row add their probabilities (scatter-add).

The pages state that the dense, forward-chunked and fused chunked variants are
mathematically equal; kl_dense is the dense variant written out, kl_sparse
keeps the teacher sparse, kl_chunked walks vocabulary and sequence chunks with
an online log-sum-exp and recomputes each chunk for the gradients, and
kl_loops is a scalar, math.fsum implementation for tiny shapes.
"""
from __future__ import annotations

import math
import numpy as np

__all__ = ["teacher_distribution", "teacher_on_vocab", "student_log_softmax",
           "kl_dense", "kl_sparse", "kl_chunked", "kl_loops", "kl_logits", "topk_rows"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _mask(mask, T):
    if mask is None:
        return np.ones(T, dtype=bool)
    return np.asarray(mask).reshape(T) != 0


def teacher_distribution(teacher_logit, tau):
    """p[t,k]: softmax over the K cached logits of row t at temperature tau
    (teacher rebuilt from its cached top-K logits; page "Making Knowledge
    Distillation Cheap Enough to Run at Scale", "Two systems changes")."""
    u = _f64(teacher_logit) / float(tau)
    if u.shape[1] == 0:
        return u
    mx = np.max(u, axis=1, keepdims=True)
    e = np.exp(u - mx)
    return e / np.sum(e, axis=1, keepdims=True)


def teacher_on_vocab(teacher_idx, p, V):
    """Dense teacher grid P[T,V] = scatter-add of p at teacher_idx."""
    T = p.shape[0]
    P = np.zeros((T, V), dtype=np.float64)
    rows = np.repeat(np.arange(T), p.shape[1])
    np.add.at(P, (rows, np.asarray(teacher_idx).reshape(-1)), p.reshape(-1))
    return P


def student_log_softmax(S, tau):
    """log q = S/tau - logsumexp_v(S/tau), row-wise over the full vocabulary."""
    z = _f64(S) / float(tau)
    mx = np.max(z, axis=1, keepdims=True)
    lse = mx + np.log(np.sum(np.exp(z - mx), axis=1, keepdims=True))
    return z - lse, lse[:, 0]


def kl_dense(h, W, teacher_idx, teacher_logit, mask=None, tau=1.0, grads=True):
    """Dense KL: materialise S, the student log-probabilities and the dense
    teacher grid, then compare them (the pages' correctness baseline).

    Returns a dict with loss, row_loss (mask_t * KL_t, not divided by N),
    kl (KL_t for every row), lse (natural-log LSE of S/tau), N and, if grads,
    dH [T,H] and dW [V,H] (all float64)."""
    h = _f64(h)
    W = _f64(W)
    T, V = h.shape[0], W.shape[0]
    m = _mask(mask, T)
    N = int(np.sum(m))
    S = h @ W.T
    logq, lse = student_log_softmax(S, tau)
    p = teacher_distribution(teacher_logit, tau)
    P = teacher_on_vocab(teacher_idx, p, V)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(P > 0, P * np.log(np.where(P > 0, P, 1.0)), 0.0)
    kl = np.sum(plogp, axis=1) - np.sum(P * logq, axis=1)
    row_loss = np.where(m, kl, 0.0)
    loss = float(np.sum(row_loss) / N) if N > 0 else 0.0
    out = dict(loss=loss, row_loss=row_loss, kl=kl, lse=lse, N=N)
    if grads:
        coef = np.where(m, 1.0 / (N * float(tau)) if N > 0 else 0.0, 0.0)
        G = coef[:, None] * (np.exp(logq) - P)
        G[~m] = 0.0
        out["dH"] = G @ W
        out["dW"] = G.T @ h
    return out


def kl_sparse(h, W, teacher_idx, teacher_logit, mask=None, tau=1.0):
    """Forward-chunked-style loss with the teacher kept sparse: per row,
    KL_t = sum_k p_k log Pm_k - sum_k p_k log q[t, idx_k], where Pm_k is the
    total teacher mass on idx_k (equals p_k when indices are distinct)."""
    h = _f64(h)
    W = _f64(W)
    T = h.shape[0]
    m = _mask(mask, T)
    N = int(np.sum(m))
    logq, lse = student_log_softmax(h @ W.T, tau)
    p = teacher_distribution(teacher_logit, tau)
    idx = np.asarray(teacher_idx)
    kl = np.zeros(T)
    for t in range(T):
        pm = np.array([p[t][idx[t] == idx[t, k]].sum() for k in range(idx.shape[1])])
        with np.errstate(divide="ignore", invalid="ignore"):
            ent = np.where(p[t] > 0, p[t] * np.log(np.where(pm > 0, pm, 1.0)), 0.0)
        kl[t] = ent.sum() - np.sum(p[t] * logq[t, idx[t]])
    row_loss = np.where(m, kl, 0.0)
    loss = float(np.sum(row_loss) / N) if N > 0 else 0.0
    return dict(loss=loss, row_loss=row_loss, kl=kl, lse=lse, N=N)


def kl_chunked(h, W, teacher_idx, teacher_logit, mask=None, tau=1.0,
               chunk_v=1024, chunk_t=None, grads=True):
    """Two-pass chunked evaluation (fused chunked KL, page "Making Knowledge
    Distillation Cheap Enough to Run at Scale", "Two systems changes"): the
    logits of one (sequence chunk, vocabulary chunk) block are projected,
    folded into a running max / sum-of-exponentials per row and discarded;
    the gradient pass recomputes every block from h and W.  No [T,V] array
    is ever held."""
    h = _f64(h)
    W = _f64(W)
    T, H = h.shape
    V = W.shape[0]
    tau = float(tau)
    chunk_t = T if not chunk_t else int(chunk_t)
    chunk_v = int(chunk_v)
    m = _mask(mask, T)
    N = int(np.sum(m))
    idx = np.asarray(teacher_idx)
    p = teacher_distribution(teacher_logit, tau)
    K = idx.shape[1]
    # teacher entropy term with duplicate indices merged
    negent = np.zeros(T)
    for t in range(T):
        for k in range(K):
            if p[t, k] > 0:
                negent[t] += p[t, k] * math.log(p[t][idx[t] == idx[t, k]].sum())
    run_max = np.full(T, -np.inf)
    run_sum = np.zeros(T)
    gath = np.zeros(T)          # sum_k p_k S[t, idx_k]
    # pass 1: online log-sum-exp and gather, block by block
    for t0 in range(0, T, chunk_t):
        t1 = min(T, t0 + chunk_t)
        for v0 in range(0, V, chunk_v):
            v1 = min(V, v0 + chunk_v)
            Sb = h[t0:t1] @ W[v0:v1].T
            zb = Sb / tau
            bmax = np.max(zb, axis=1)
            new_max = np.maximum(run_max[t0:t1], bmax)
            run_sum[t0:t1] = (run_sum[t0:t1] * np.exp(run_max[t0:t1] - new_max)
                              + np.sum(np.exp(zb - new_max[:, None]), axis=1))
            run_max[t0:t1] = new_max
            for t in range(t0, t1):
                for k in range(K):
                    if v0 <= idx[t, k] < v1:
                        gath[t] += p[t, k] * Sb[t - t0, idx[t, k] - v0]
    lse = run_max + np.log(run_sum)
    kl = negent - gath / tau + lse
    row_loss = np.where(m, kl, 0.0)
    loss = float(np.sum(row_loss) / N) if N > 0 else 0.0
    out = dict(loss=loss, row_loss=row_loss, kl=kl, lse=lse, N=N)
    if not grads:
        return out
    # pass 2: recompute each block, form its logit gradient, contract it away
    coef = np.where(m, 1.0 / (N * tau) if N > 0 else 0.0, 0.0)
    dH = np.zeros((T, H))
    dW = np.zeros((V, H))
    for t0 in range(0, T, chunk_t):
        t1 = min(T, t0 + chunk_t)
        for v0 in range(0, V, chunk_v):
            v1 = min(V, v0 + chunk_v)
            Sb = h[t0:t1] @ W[v0:v1].T
            qb = np.exp(Sb / tau - lse[t0:t1, None])
            for t in range(t0, t1):
                for k in range(K):
                    if v0 <= idx[t, k] < v1:
                        qb[t - t0, idx[t, k] - v0] -= p[t, k]
            Gb = coef[t0:t1, None] * qb
            Gb[~m[t0:t1]] = 0.0
            dH[t0:t1] += Gb @ W[v0:v1]
            dW[v0:v1] += Gb.T @ h[t0:t1]
    out["dH"] = dH
    out["dW"] = dW
    return out


def kl_loops(h, W, teacher_idx, teacher_logit, mask=None, tau=1.0):
    """Scalar-loop evaluation with math.fsum, for tiny shapes only.  Written
    independently of the array versions above (no numpy arithmetic)."""
    h = [[float(x) for x in row] for row in np.asarray(h)]
    W = [[float(x) for x in row] for row in np.asarray(W)]
    idx = [[int(x) for x in row] for row in np.asarray(teacher_idx)]
    lg = [[float(x) for x in row] for row in np.asarray(teacher_logit)]
    T, H, V = len(h), len(h[0]) if h else 0, len(W)
    K = len(idx[0]) if idx else 0
    msk = [True] * T if mask is None else [int(x) != 0 for x in np.asarray(mask)]
    N = sum(1 for x in msk if x)
    tau = float(tau)
    S = [[math.fsum(h[t][i] * W[v][i] for i in range(H)) for v in range(V)] for t in range(T)]
    kl = []
    Q = []
    Pd = []
    for t in range(T):
        z = [s / tau for s in S[t]]
        zmax = max(z)
        lse = zmax + math.log(math.fsum(math.exp(x - zmax) for x in z))
        q = [math.exp(x - lse) for x in z]
        u = [x / tau for x in lg[t]]
        umax = max(u)
        zz = math.fsum(math.exp(x - umax) for x in u)
        p = [math.exp(x - umax) / zz for x in u]
        P = [0.0] * V
        for k in range(K):
            P[idx[t][k]] += p[k]
        terms = [P[v] * (math.log(P[v]) - (z[v] - lse)) for v in range(V) if P[v] > 0]
        kl.append(math.fsum(terms))
        Q.append(q)
        Pd.append(P)
    row_loss = [kl[t] if msk[t] else 0.0 for t in range(T)]
    loss = math.fsum(row_loss) / N if N > 0 else 0.0
    G = [[((Q[t][v] - Pd[t][v]) / (N * tau)) if (msk[t] and N > 0) else 0.0
          for v in range(V)] for t in range(T)]
    dH = [[math.fsum(G[t][v] * W[v][i] for v in range(V)) for i in range(H)] for t in range(T)]
    dW = [[math.fsum(G[t][v] * h[t][i] for t in range(T)) for i in range(H)] for v in range(V)]
    return dict(loss=loss, row_loss=np.array(row_loss), kl=np.array(kl),
                dH=np.array(dH).reshape(T, H), dW=np.array(dW).reshape(V, H), N=N)


def kl_logits(Z, teacher_idx, teacher_logit, mask=None, tau=1.0, grads=True):
    """Forward-chunked KL on already materialised student logits Z[T,V] (page
    "Making Knowledge Distillation Cheap Enough to Run at Scale", "Two systems
    changes", second variant: the teacher stays sparse, the student's logits
    exist in full).  Same loss as kl_dense with S replaced by Z; the gradient
    is with respect to the logits: dZ[t,v] = mask_t/(N tau) (q[t,v] - P[t,v]).

    Returns loss, row_loss, kl, lse (natural log of sum exp(Z/tau)), N and,
    if grads, dZ [T,V] (float64)."""
    Z = _f64(Z)
    T, V = Z.shape
    m = _mask(mask, T)
    N = int(np.sum(m))
    logq, lse = student_log_softmax(Z, tau)
    p = teacher_distribution(teacher_logit, tau)
    P = teacher_on_vocab(teacher_idx, p, V)
    with np.errstate(divide="ignore", invalid="ignore"):
        plogp = np.where(P > 0, P * np.log(np.where(P > 0, P, 1.0)), 0.0)
    kl = np.sum(plogp, axis=1) - np.sum(P * logq, axis=1)
    row_loss = np.where(m, kl, 0.0)
    loss = float(np.sum(row_loss) / N) if N > 0 else 0.0
    out = dict(loss=loss, row_loss=row_loss, kl=kl, lse=lse, N=N)
    if grads:
        coef = np.where(m, 1.0 / (N * float(tau)) if N > 0 else 0.0, 0.0)
        dZ = coef[:, None] * (np.exp(logq) - P)
        dZ[~m] = 0.0
        out["dZ"] = dZ
    return out


def topk_rows(X, K):
    """The teacher cache's content (page "Making Knowledge Distillation Cheap
    Enough to Run at Scale", "Two systems changes": the K most likely tokens
    per position are cached): for every row of X[T,V], the ids of its K
    largest values in descending order of value, equal values by ascending
    id, and those values.  Returns (idx int64 [T,K], values float64 [T,K])."""
    X = np.asarray(X)
    T, V = X.shape
    K = int(K)
    ids = np.arange(V)
    idx = np.empty((T, K), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((ids, -X[t].astype(np.float64)))
        idx[t] = order[:K]
    vals = np.take_along_axis(X.astype(np.float64), idx, axis=1)
    return idx, vals
