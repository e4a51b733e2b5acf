"""Pin the oracle to exact results that hold at any size.

* All-zero logits: every emission weighs -log V - log D - sigma and log P follows from
  exact alignment counts (oracle/closed_form.py), also at the full workload shapes.
* A single duration {1}: every alignment has exactly T emissions, so the loss moves by
  exactly sigma * T when sigma changes.
* A single duration {1} and no labels: one alignment of T blanks, whose loss is a sum
  of torch.log_softmax entries.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import closed_form
from tdt_inputs import make_case


def _zero_case(T, U, V, durs, sigma, dtype="f32"):
    c = make_case(1, [T], [U], V, durs, dtype, sigma=sigma, seed=11, reduction="none")
    c.joint.zero_()
    return c


@pytest.mark.parametrize("T,U,V,durs,sigma", [
    (12, 4, 17, [0, 1, 2, 3, 4], 0.0),
    (30, 10, 5, [0, 1, 2, 3, 4], 0.05),
    (40, 60, 9, [0, 1, 2], 0.0),
    (25, 3, 4, [2, 3, 5], -0.2),
    (200, 40, 8193, [0, 1, 2, 3, 4], 0.05),     # Parakeet-size lattice
    (1000, 1500, 5, list(range(9)), 0.05),       # long-label lattice (U > T)
])
def test_zero_logits_closed_form(T, U, V, durs, sigma):
    c = _zero_case(T, U, V, durs, sigma)
    r = oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank, sigma, "none",
                   grads=False)
    exact = closed_form.zero_logit_loss(T, U, V, durs, sigma)
    assert r["loss_utt"][0] == pytest.approx(exact, rel=2e-13)
    assert r["logp_alpha"][0] == pytest.approx(-exact, rel=2e-13)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_duration_sigma_shift(dtype):
    """Durations {1}: loss(sigma) = loss(0) + sigma * T for every utterance."""
    c = make_case(3, [10, 7, 12], [3, 0, 5], 9, [1], dtype, seed=5, reduction="none")
    r0 = oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, [1], c.blank, 0.0, "none")
    r1 = oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, [1], c.blank, 0.37, "none")
    T = c.logit_lengths.double().numpy()
    np.testing.assert_allclose(r1["loss_utt"] - r0["loss_utt"], 0.37 * T, rtol=1e-12)
    # the gradient does not depend on sigma in this case (every path has T emissions)
    np.testing.assert_allclose(r1["grad_tok"], r0["grad_tok"], atol=1e-13)


def test_single_duration_no_labels_is_sum_of_blank_log_softmax():
    T, V, sigma = 14, 11, 0.2
    c = make_case(1, [T], [0], V, [1], "f32", seed=9, sigma=sigma, reduction="none", U1max=1)
    r = oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, [1], c.blank, sigma, "none")
    lp = torch.log_softmax(c.tok[0, :T, 0].double(), dim=-1)[:, c.blank]
    expected = float(-(lp.sum()) + sigma * T)
    assert r["loss_utt"][0] == pytest.approx(expected, rel=1e-13)
    # its gradient: softmax - onehot(blank) on every frame
    sm = torch.softmax(c.tok[0, :T, 0].double(), dim=-1).numpy()
    sm[:, c.blank] -= 1.0
    np.testing.assert_allclose(r["grad_tok"][0, :T, 0], sm, atol=1e-13)
    np.testing.assert_allclose(r["grad_dur"][0, :T, 0], 0.0, atol=1e-13)
