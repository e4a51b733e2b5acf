"""TEST INFRASTRUCTURE ONLY: brute-force enumeration of every TDT alignment.

Independent of the dynamic-programming oracle in ``tdt_oracle.c``: no alpha, no beta,
no recursion over lattice nodes.  Every move sequence from (0, 0) to the terminal is
listed explicitly, its log-probability is the sum of its move log-weights, and

    log P = log sum over alignments of exp(log-probability).

Move rules (the reading of the kernel description on the page "tdt-loss: add TDT loss
kernel", comment "What's in it", that the oracle also takes): from node (t, u)
  * a blank with duration d > 0 goes to (t + d, u) if t + d < T, and ends the
    alignment if u = U and t + d = T;
  * a label y_{u+1} with any duration d (0 allowed) goes to (t + d, u + 1) if
    u < U and t + d < T.
Each emission weighs log_softmax(h(t,u))[token] - sigma + log_softmax(g(t,u))[i].

Used only on tiny lattices (the number of alignments grows exponentially).
"""
from __future__ import annotations

import math

import numpy as np
import torch


def enumerate_alignments(T: int, U: int, durations) -> list:
    """All alignments as lists of moves (t, u, kind, i); kind 0 = blank, 1 = label."""
    durations = list(durations)
    out = []
    if T <= 0:
        return out
    stack = [(0, 0, ())]
    while stack:
        t, u, moves = stack.pop()
        for i, d in enumerate(durations):
            if d > 0:
                if t + d < T:
                    stack.append((t + d, u, moves + ((t, u, 0, i),)))
                elif t + d == T and u == U:
                    out.append(list(moves + ((t, u, 0, i),)))
            if u < U and t + d < T:
                stack.append((t + d, u + 1, moves + ((t, u, 1, i),)))
    return out


def _log_softmax_rows(x: np.ndarray) -> np.ndarray:
    m = x.max(axis=-1, keepdims=True)
    s = np.log(np.exp(x - m).sum(axis=-1, keepdims=True))
    return x - m - s


def utterance(h: np.ndarray, g: np.ndarray, labels, durations, blank: int, sigma: float = 0.0) -> dict:
    """Loss and per-node posteriors of one utterance by explicit enumeration.

    h: [T, U+1, V] float64 token logits, g: [T, U+1, D] float64 duration logits.
    Returns loss (= -log P), count of alignments, occupancy O(n) = probability that an
    alignment leaves n, expected blank / label departures c_blank(n), c_label(n), and
    c_dur(n, i), plus the gradient of the loss assembled from those posteriors.
    """
    T, U1, V = h.shape
    U = U1 - 1
    D = g.shape[2]
    lt = _log_softmax_rows(h.astype(np.float64))
    ld = _log_softmax_rows(g.astype(np.float64))
    paths = enumerate_alignments(T, U, durations)
    lw = np.empty(len(paths))
    for j, path in enumerate(paths):
        s = 0.0
        for (t, u, kind, i) in path:
            tok = blank if kind == 0 else labels[u]
            s += lt[t, u, tok] - sigma + ld[t, u, i]
        lw[j] = s
    res = {"count": len(paths)}
    if not paths:
        res["loss"] = math.inf
        return res
    m = lw.max()
    w = np.exp(lw - m)
    Z = w.sum()
    res["loss"] = -(m + math.log(Z))
    post = w / Z
    occ = np.zeros((T, U1))
    cb = np.zeros((T, U1))
    cl = np.zeros((T, U1))
    cd = np.zeros((T, U1, D))
    for j, path in enumerate(paths):
        for (t, u, kind, i) in path:
            occ[t, u] += post[j]
            if kind == 0:
                cb[t, u] += post[j]
            else:
                cl[t, u] += post[j]
            cd[t, u, i] += post[j]
    res.update(occ=occ, cblank=cb, clabel=cl, cdur=cd)
    gh = occ[:, :, None] * np.exp(lt)
    for t in range(T):
        for u in range(U1):
            gh[t, u, blank] -= cb[t, u]
            if u < U:
                gh[t, u, labels[u]] -= cl[t, u]
    gg = occ[:, :, None] * np.exp(ld) - cd
    res.update(grad_tok=gh, grad_dur=gg)
    return res


def autograd_utterance(h: np.ndarray, g: np.ndarray, labels, durations, blank: int, sigma: float = 0.0):
    """-log P and its gradient by torch float64 autograd over the explicit alignment list.

    Differentiates log-sum-exp over alignments of the summed torch.log_softmax entries, so
    it checks the oracle's gradient formula as well as its recursions.
    """
    T, U1, V = h.shape
    U = U1 - 1
    ht = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    gt = torch.tensor(g, dtype=torch.float64, requires_grad=True)
    lt = torch.log_softmax(ht, dim=-1)
    ld = torch.log_softmax(gt, dim=-1)
    paths = enumerate_alignments(T, U, durations)
    if not paths:
        return math.inf, np.zeros_like(h), np.zeros_like(g)
    L = max(len(p) for p in paths)
    P = len(paths)
    tt = np.zeros((P, L), dtype=np.int64)
    uu = np.zeros((P, L), dtype=np.int64)
    kk = np.zeros((P, L), dtype=np.int64)
    ii = np.zeros((P, L), dtype=np.int64)
    mask = np.zeros((P, L))
    for j, path in enumerate(paths):
        for s, (t, u, kind, i) in enumerate(path):
            tt[j, s], uu[j, s], ii[j, s] = t, u, i
            kk[j, s] = blank if kind == 0 else labels[u]
            mask[j, s] = 1.0
    tt, uu, kk, ii = (torch.from_numpy(a) for a in (tt, uu, kk, ii))
    mk = torch.from_numpy(mask)
    per_move = (lt[tt, uu, kk] - sigma + ld[tt, uu, ii]) * mk
    loss = -torch.logsumexp(per_move.sum(dim=1), dim=0)
    loss.backward()
    return float(loss), ht.grad.numpy().copy(), gt.grad.numpy().copy()
