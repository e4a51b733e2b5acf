"""Pin the oracle's gradient by central finite differences in float64.

The loss is evaluated on float64 logits (the oracle widens fp32/fp16/bf16 exactly, and
accepts float64 for this purpose), perturbed one entry at a time.  Entries are drawn from
the blank column, the label column, other token columns, the duration columns and the
padded region (whose derivative must be exactly 0).
"""
import numpy as np
import pytest
import torch

import oracle
from tdt_inputs import make_case


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_finite_differences(reduction):
    c = make_case(2, [10, 7], [4, 3], 11, [0, 1, 2, 3], "f64", sigma=0.05, seed=31, reduction=reduction,
                  Tmax=11, U1max=6)
    r = oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank, c.sigma,
                   reduction)
    rng = np.random.default_rng(0)
    eps = 1e-5
    picks = []
    for _ in range(24):
        b = int(rng.integers(0, 2))
        T, U = int(c.logit_lengths[b]), int(c.label_lengths[b])
        t, u = int(rng.integers(0, T)), int(rng.integers(0, U + 1))
        kind = rng.integers(0, 4)
        if kind == 0:
            v = c.blank
        elif kind == 1 and u < U:
            v = int(c.labels[b, u])
        else:
            v = int(rng.integers(0, c.V))
        picks.append(("tok", b, t, u, v))
        picks.append(("dur", b, t, u, int(rng.integers(0, c.D))))
    picks += [("tok", 0, 10, 2, 3), ("tok", 1, 3, 5, 0), ("dur", 1, 8, 1, 2)]  # padded nodes
    for kind, b, t, u, v in picks:
        view = c.tok if kind == "tok" else c.dur
        old = float(view[b, t, u, v])
        vals = []
        for s in (+1, -1):
            view[b, t, u, v] = old + s * eps
            vals.append(oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank,
                                   c.sigma, reduction, grads=False)["loss"])
        view[b, t, u, v] = old
        fd = (vals[0] - vals[1]) / (2 * eps)
        an = r["grad_tok" if kind == "tok" else "grad_dur"][b, t, u, v]
        assert abs(fd - an) <= 2e-9, (kind, b, t, u, v, fd, an)
