"""Pin the oracle to brute-force enumeration of every alignment on tiny lattices.

The enumerator (oracle/bruteforce.py) lists every move sequence explicitly and never
recurses over lattice nodes; its gradient comes either from posterior counts over the
listed alignments or from torch float64 autograd of log-sum-exp over them.  A dropped
transition, a wrong duration rule, a wrong label index or a wrong gradient term in the
oracle changes at least one of these numbers.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import bruteforce, closed_form
from tdt_inputs import config_case, make_case

# (name, B, T, U, V, durations, dtype, sigma, extra padding (dT, dU), blank)
CASES = [
    ("d0to4_bf16_sigma", 2, [6, 5], [2, 2], 5, [0, 1, 2, 3, 4], "bf16", 0.05, (2, 1), None),
    ("d12_f16_negsigma", 1, [7], [3], 4, [1, 2], "f16", -0.1, (1, 1), None),
    ("d023_f32", 2, [5, 6], [4, 1], 6, [0, 2, 3], "f32", 0.3, (0, 0), None),
    ("no_labels", 1, [6], [0], 3, [0, 1, 2, 3], "f32", 0.05, (1, 2), None),
    ("more_labels_than_frames", 1, [4], [5], 7, [0, 1], "f32", 0.0, (1, 0), None),
    ("unsorted_durations", 1, [6], [2], 5, [3, 0, 1], "f64", 0.02, (0, 1), None),
    ("single_duration_1", 1, [6], [2], 5, [1], "f32", 0.1, (1, 1), None),
    ("blank_not_last", 1, [5], [2], 6, [0, 1, 2], "f32", 0.0, (0, 0), 2),
]


def _run_case(name, B, T, U, V, durs, dt, sigma, pad, blank, seed=7):
    Tmax = max(T) + pad[0]
    U1 = max(U) + 1 + pad[1]
    c = make_case(B, T, U, V, durs, dt, sigma=sigma, reduction="none", seed=seed, Tmax=Tmax, U1max=U1,
                  blank=blank, label_high=V)
    return c


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_oracle_matches_enumeration(case):
    c = _run_case(*case)
    r = oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank, c.sigma,
                   "none", nodes=True)
    for b in range(c.B):
        T, U = int(c.logit_lengths[b]), int(c.label_lengths[b])
        h = c.tok[b, :T, :U + 1].double().numpy()
        g = c.dur[b, :T, :U + 1].double().numpy()
        lab = c.labels[b, :U].tolist()
        bf = bruteforce.utterance(h, g, lab, c.durations, c.blank, c.sigma)
        assert bf["count"] == closed_form.count_alignments(T, U, c.durations)
        assert bf["count"] > 0
        assert r["status"][b] == 0
        assert r["loss_utt"][b] == pytest.approx(bf["loss"], rel=1e-12)
        for key in ("occ", "cblank", "clabel"):
            np.testing.assert_allclose(r[key][b, :T, :U + 1], bf[key], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["cdur"][b, :T, :U + 1], bf["cdur"], rtol=0, atol=1e-12)
        loss_ad, gh, gg = bruteforce.autograd_utterance(h, g, lab, c.durations, c.blank, c.sigma)
        assert loss_ad == pytest.approx(bf["loss"], rel=1e-12)
        np.testing.assert_allclose(r["grad_tok"][b, :T, :U + 1], gh, rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["grad_dur"][b, :T, :U + 1], gg, rtol=0, atol=1e-12)
        # every padded position of the gradient is exactly zero
        gt = r["grad_tok"][b].copy()
        gt[:T, :U + 1] = 0
        gd = r["grad_dur"][b].copy()
        gd[:T, :U + 1] = 0
        assert not gt.any() and not gd.any()


def test_tiny_config_second_utterance():
    """Workload 0 (B=2, T={12,9}, U={4,3}, V=17, fp32): the 9x4 utterance has 40,080
    alignments; enumerate them all and compare loss and gradient."""
    c = config_case(0)
    r = oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank, c.sigma,
                   c.reduction)
    b, T, U = 1, 9, 3
    h = c.tok[b, :T, :U + 1].double().numpy()
    g = c.dur[b, :T, :U + 1].double().numpy()
    lab = c.labels[b, :U].tolist()
    loss, gh, gg = bruteforce.autograd_utterance(h, g, lab, c.durations, c.blank, c.sigma)
    assert r["loss_utt"][b] == pytest.approx(loss, rel=1e-12)
    np.testing.assert_allclose(r["grad_tok"][b, :T, :U + 1], gh, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["grad_dur"][b, :T, :U + 1], gg, rtol=0, atol=1e-12)


def test_alignment_counts_of_tiny_config():
    """Counts of alignments for the two lattices of workload 0 (12x4 and 9x3 with
    durations 0..4), as computed independently: 2,552,850 and 40,080."""
    assert closed_form.count_alignments(12, 4, range(5)) == 2552850
    assert closed_form.count_alignments(9, 3, range(5)) == 40080
    assert len(bruteforce.enumerate_alignments(9, 3, range(5))) == 40080


@pytest.mark.parametrize("T,U,durs", [(1, 0, [0, 1]), (3, 2, [0, 1, 2]), (5, 1, [2, 3]), (6, 3, [0, 1, 2, 3, 4]),
                                       (4, 6, [0, 1]), (7, 2, [1]), (8, 2, [0, 4])])
def test_enumeration_count_matches_combinatorics(T, U, durs):
    assert len(bruteforce.enumerate_alignments(T, U, durs)) == closed_form.count_alignments(T, U, durs)


def test_infeasible_utterance():
    """Durations {2} and an odd frame count admit no alignment: +inf loss, zero gradient."""
    c = make_case(1, [5], [1], 4, [2], "f32", seed=3, reduction="none")
    assert closed_form.count_alignments(5, 1, [2]) == 0
    r = oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank, 0.0, "none")
    assert math.isinf(r["loss_utt"][0]) and r["loss_utt"][0] > 0
    assert r["status"][0] == oracle.ST_INFEASIBLE
    assert not r["grad_tok"].any() and not r["grad_dur"].any()


def test_zero_frames():
    c = make_case(2, [0, 4], [0, 1], 5, [0, 1, 2], "f32", seed=4, reduction="none", Tmax=4, U1max=2)
    r = oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank, 0.0, "none")
    assert math.isinf(r["loss_utt"][0]) and r["status"][0] == oracle.ST_INFEASIBLE
    assert not r["grad_tok"][0].any()
    assert np.isfinite(r["loss_utt"][1]) and r["status"][1] == 0
