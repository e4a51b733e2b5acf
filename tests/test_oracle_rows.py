"""Pin the oracle's row outputs to its full gradient.

The full gradient of ``oracle.run`` is pinned by brute-force enumeration, autograd and
finite differences (test_oracle_bruteforce.py, test_oracle_fd.py).  The GPU parity test of
the long-label workload reads the oracle's gradient one range of rows at a time instead
(its full float64 gradient would take about 25 GB), through the ``rows=`` list of
``oracle.run`` and through ``oracle.Session``.  Both must reproduce the full gradient's
rows bit for bit: the node index decode (b, t, u from the padded index), the choice of
utterance, the zero rows of padded nodes, of utterances with a data error and of
utterances without alignment.
"""
import numpy as np
import pytest
import torch

import oracle
from tdt_inputs import make_case


def _case():
    # ragged and padded (Tmax 23, U1max 9), three extra columns after the duration
    # logits, a negative sigma; utterance 2 has no alignment (durations {2, 3, 4} cannot
    # fill T = 1) and utterance 4 a label outside the vocabulary
    c = make_case(5, [20, 23, 1, 9, 15], [6, 8, 0, 3, 2], 19, [0, 2, 3, 4], "bf16", seed=90, sigma=-0.03,
                  reduction="mean", Tmax=23, U1max=9, extra_cols=3)
    c.labels[4, 1] = 19
    return c


def _full(c):
    return oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank, c.sigma,
                      c.reduction)


def test_full_reference_has_the_expected_structure():
    c = _case()
    r = _full(c)
    assert list(r["status"]) == [0, 0, oracle.ST_INFEASIBLE, 0, oracle.ST_BAD_LABEL]
    g = r["grad_tok"]
    for b in range(c.B):
        T, U = int(c.logit_lengths[b]), int(c.label_lengths[b])
        live = r["status"][b] == 0
        assert bool(np.abs(g[b, :T, :U + 1]).max() > 0) == live
        assert not g[b, T:].any() and not g[b, :, U + 1:].any()


def test_selected_rows_equal_full_gradient_rows_bitwise():
    c = _case()
    r = _full(c)
    B, Tm, U1 = c.tok.shape[:3]
    rng = np.random.default_rng(3)
    rows = list(rng.integers(0, B * Tm * U1, 300))
    # every utterance's corners, padded nodes past T and past U, the first and last index
    for b in range(B):
        for t in (0, 1, Tm - 1):
            for u in (0, 1, U1 - 1):
                rows.append((b * Tm + t) * U1 + u)
    rows += [0, B * Tm * U1 - 1]
    rows = np.array(rows, dtype=np.int64)  # unsorted, with repeats
    rs = oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank, c.sigma,
                    c.reduction, grads=False, rows=rows)
    full_t = r["grad_tok"].reshape(-1, c.V)
    full_d = r["grad_dur"].reshape(-1, c.D)
    np.testing.assert_array_equal(rs["rows_tok"], full_t[rows])
    np.testing.assert_array_equal(rs["rows_dur"], full_d[rows])
    np.testing.assert_array_equal(rs["loss"], r["loss"])  # NaN: utterance 4 has a data error
    np.testing.assert_array_equal(rs["status"], r["status"])
    # rows of padded nodes are exactly zero
    b, rem = rows // (Tm * U1), rows % (Tm * U1)
    t, u = rem // U1, rem % U1
    pad = (t >= c.logit_lengths.numpy()[b]) | (u > c.label_lengths.numpy()[b])
    assert pad.sum() > 20
    assert not rs["rows_tok"][pad].any() and not rs["rows_dur"][pad].any()


@pytest.mark.parametrize("chunk", [1, 37, 1000])
def test_session_rows_equal_full_gradient_bitwise(chunk):
    c = _case()
    r = _full(c)
    with oracle.Session(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank, c.sigma,
                        c.reduction) as s:
        np.testing.assert_array_equal(s.loss, r["loss"])
        np.testing.assert_array_equal(s.loss_utt, r["loss_utt"])
        np.testing.assert_array_equal(s.status, r["status"])
        full_t = r["grad_tok"].reshape(-1, c.V)
        full_d = r["grad_dur"].reshape(-1, c.D)
        for first in range(0, s.nodes, chunk):
            n = min(chunk, s.nodes - first)
            gt, gd = s.rows(first, n)
            np.testing.assert_array_equal(gt, full_t[first:first + n])
            np.testing.assert_array_equal(gd, full_d[first:first + n])
        with pytest.raises(IndexError):
            s.rows(s.nodes - 1, 2)


def test_session_on_strided_fp32_views():
    c = make_case(3, [30, 17, 24], [10, 4, 12], 41, [0, 1, 2, 3, 4], "f32", seed=91, sigma=0.05,
                  reduction="mean_volume", extra_cols=2)
    r = _full(c)
    assert not c.tok.is_contiguous()
    with oracle.Session(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank, c.sigma,
                        c.reduction) as s:
        gt, gd = s.rows(0, s.nodes)
    np.testing.assert_array_equal(gt, r["grad_tok"].reshape(-1, c.V))
    np.testing.assert_array_equal(gd, r["grad_dur"].reshape(-1, c.D))
