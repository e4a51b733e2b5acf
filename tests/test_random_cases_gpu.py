"""Seeded random small cases, loss, every gradient element and the status words against the
float64 oracle.

The draws straddle the thresholds the library switches on:
- the vocabulary around the short-row limits of the row statistics (V / elements per
  16-byte chunk + 1 <= 256 chunks) and of the gradient pass (+ 8 <= 256), and long rows;
- the label count on both sides of 64 (one tile, linked tiles);
- duration sets up to 16 (the kernel bounds 4, 8 and 16), unsorted, with or without 0;
- every reduction, sigma, the blank anywhere in the vocabulary (labels may equal it);
- ragged lengths (padding rows), and gradient buffers co-aligned with the logits (the
  short-row passes) or in separate contiguous buffers (the per-element path);
- and, separately, long label sequences (65 to 1500 labels: linked columns, bands).
"""
import random

import pytest
import torch

from parity_util import check_grads, check_loss, gpu_run, oracle_run
from tdt_inputs import make_case

pytestmark = pytest.mark.gpu

N_CASES = 64


def _draw(i):
    r = random.Random(9000 + i)
    dtype = r.choice(["f32", "f16", "bf16"])
    epc = 4 if dtype == "f32" else 8  # elements per 16-byte chunk
    lim = 256 * epc
    kind = r.choice(["tiny", "short", "grad_edge", "stat_edge", "long"])
    if kind == "tiny":
        V = r.randint(3, 60)
    elif kind == "short":
        V = r.randint(200, 900)
    elif kind == "grad_edge":  # the gradient pass's short-row limit
        V = lim - 8 * epc + r.randint(-epc, epc)
    elif kind == "stat_edge":  # the row statistics' short-row limit
        V = lim - epc + r.randint(-epc, epc)
    else:
        V = r.randint(lim + 1, 5000)
    wide = V > 1000
    B = r.randint(1, 3 if wide else 5)
    T = [r.randint(1, 40) for _ in range(B)]
    Umax = r.choice([r.randint(0, 20)] if wide else [r.randint(0, 20), r.randint(40, 70), r.randint(100, 140)])
    U = [r.randint(0, Umax) for _ in range(B)]
    maxd = r.choice([2, 4, 6, 8, 12, 16])
    durs = r.sample(range(maxd + 1), r.randint(1, min(maxd + 1, 8)))
    if max(durs) == 0:
        durs.append(r.randint(1, maxd))
    r.shuffle(durs)
    blank = r.choice([V - 1, 0, r.randrange(V)])
    red = r.choice(["none", "sum", "mean", "mean_batch", "mean_volume"])
    sigma = r.choice([0.0, 0.05, 0.2])
    scale = r.choice([1.0, 2.0, 4.0])
    separate = r.random() < 0.25
    name = f"rand{i}_{dtype}_V{V}_U{Umax}_d{max(durs)}_{red}{'_sep' if separate else ''}"
    case = make_case(B, T, U, V, durs, dtype, scale=scale, sigma=sigma, reduction=red, seed=9000 + i,
                     blank=blank, name=name)
    return case, separate


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    case, separate = _draw(i)
    gcase = case.to("cuda")
    grads = None
    if separate:
        grads = (torch.full(gcase.tok.shape, float("nan"), dtype=gcase.joint.dtype, device="cuda"),
                 torch.full(gcase.dur.shape, float("nan"), dtype=gcase.joint.dtype, device="cuda"))
    loss, gt, gd, st = gpu_run(gcase, grads=grads)
    orc = oracle_run(case)
    check_loss(loss, orc, case.reduction, case.joint.dtype)
    check_grads(gt, gd, orc, case.joint.dtype)
    assert st.cpu().tolist() == orc["status"].tolist()


N_LONG = 16


def _draw_long(i):
    """Long label sequences (65 to 1500 labels over few frames, duration 0 always allowed so
    that more labels than frames align): linked columns (durations up to 8), bands (16)."""
    r = random.Random(7000 + i)
    dtype = r.choice(["f32", "bf16"])
    V = r.randint(5, 40)
    B = r.randint(1, 4)
    T = [r.randint(4, 60) for _ in range(B)]
    Umax = r.choice([r.randint(257, 600), r.randint(900, 1500)])
    U = [r.randint(Umax // 2, Umax) for _ in range(B)]
    maxd = r.choice([2, 4, 8, 16])
    durs = [0] + r.sample(range(1, maxd + 1), r.randint(1, min(maxd, 6)))
    r.shuffle(durs)
    red = r.choice(["none", "sum", "mean", "mean_batch", "mean_volume"])
    name = f"long{i}_{dtype}_U{Umax}_d{max(durs)}_{red}"
    return make_case(B, T, U, V, durs, dtype, scale=r.choice([1.0, 2.0]), sigma=r.choice([0.0, 0.05]),
                     reduction=red, seed=7000 + i, name=name)


@pytest.mark.parametrize("i", range(N_LONG))
def test_random_long_labels(i):
    case = _draw_long(i)
    loss, gt, gd, st = gpu_run(case.to("cuda"))
    orc = oracle_run(case)
    check_loss(loss, orc, case.reduction, case.joint.dtype)
    check_grads(gt, gd, orc, case.joint.dtype)
    assert st.cpu().tolist() == orc["status"].tolist()
