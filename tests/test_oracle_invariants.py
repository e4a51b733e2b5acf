"""Pin the oracle with identities that any correct TDT loss satisfies.

* alpha/beta agreement: log P from the alpha terminal equals beta(0, 0);
* zero-sum rows: the token gradient and the duration gradient of every node sum to 0;
* posterior counts: every alignment emits exactly U labels, spends exactly T frames and
  its number of emissions is d loss / d sigma;
* layout: padding values are irrelevant, padded gradients are 0, a strided view gives
  the result of a contiguous copy, a batch gives the per-utterance results;
* reductions: the five reductions follow from the per-utterance losses and the
  gradients scale by the per-utterance weights;
* data errors: an out-of-range label or length gives NaN and a zero gradient for that
  utterance only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tdt_inputs import config_case, make_case


def _run(c, reduction=None, sigma=None, **kw):
    return oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank,
                      c.sigma if sigma is None else sigma, reduction or c.reduction, **kw)


CASES = {
    "tiny": lambda: config_case(0),
    "ragged": lambda: make_case(4, None, None, 33, [0, 1, 2, 3, 4], "f16", scale=1.5, seed=21, Tmax=40,
                                U1max=16, T_range=(10, 40), U_range=(2, 15), reduction="mean"),
    "long_label": lambda: make_case(1, [60], [90], 9, list(range(9)), "bf16", seed=22, sigma=0.05,
                                    reduction="sum"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_alpha_beta_agree(name):
    c = CASES[name]()
    r = _run(c)
    np.testing.assert_allclose(r["logp_alpha"], r["logp_beta"], rtol=1e-12)
    assert np.all(np.isfinite(r["logp_beta"]))


@pytest.mark.parametrize("name", list(CASES))
def test_zero_sum_rows_and_posterior_counts(name):
    c = CASES[name]()
    r = _run(c, reduction="none", nodes=True)
    np.testing.assert_allclose(r["grad_tok"].sum(-1), 0.0, atol=1e-12)
    np.testing.assert_allclose(r["grad_dur"].sum(-1), 0.0, atol=1e-12)
    d = np.asarray(c.durations, dtype=np.float64)
    for b in range(c.B):
        T, U = int(c.logit_lengths[b]), int(c.label_lengths[b])
        assert r["clabel"][b].sum() == pytest.approx(U, rel=1e-11, abs=1e-11)
        assert (r["cdur"][b] * d).sum() == pytest.approx(T, rel=1e-11)
        # occupancy of the start node is 1
        assert r["occ"][b, 0, 0] == pytest.approx(1.0, rel=1e-12)


def test_sigma_derivative_is_expected_emissions():
    c = CASES["ragged"]()
    eps = 1e-5
    rp = _run(c, reduction="none", sigma=0.05 + eps, grads=False)
    rm = _run(c, reduction="none", sigma=0.05 - eps, grads=False)
    r = _run(c, reduction="none", sigma=0.05, nodes=True, grads=False)
    fd = (rp["loss_utt"] - rm["loss_utt"]) / (2 * eps)
    emis = (r["cblank"] + r["clabel"]).sum(axis=(1, 2))
    np.testing.assert_allclose(fd, emis, rtol=1e-8)


def test_padding_is_ignored():
    c = CASES["ragged"]()
    r = _run(c)
    c2 = make_case(4, None, None, 33, [0, 1, 2, 3, 4], "f16", scale=1.5, seed=21, Tmax=40, U1max=16,
                   T_range=(10, 40), U_range=(2, 15), reduction="mean")
    noise = torch.randn(c2.joint.shape, generator=torch.Generator().manual_seed(5)).to(c2.joint.dtype)
    for b in range(c.B):
        T, U = int(c.logit_lengths[b]), int(c.label_lengths[b])
        mask = torch.ones(c2.joint.shape[1:3], dtype=torch.bool)
        mask[:T, :U + 1] = False
        c2.joint[b][mask] = noise[b][mask]
        c2.labels[b, U:] = 12345  # junk past U is never read
    r2 = _run(c2)
    assert r2["loss"] == r["loss"]
    np.testing.assert_array_equal(r2["grad_tok"], r["grad_tok"])
    for b in range(c.B):
        T, U = int(c.logit_lengths[b]), int(c.label_lengths[b])
        assert not r["grad_tok"][b, T:].any() and not r["grad_tok"][b, :, U + 1:].any()
        assert not r["grad_dur"][b, T:].any() and not r["grad_dur"][b, :, U + 1:].any()


def test_strided_view_equals_contiguous_and_batch_equals_single():
    c = CASES["ragged"]()
    r = _run(c, reduction="none")
    rc = oracle.run(c.tok.contiguous(), c.dur.contiguous(), c.labels, c.logit_lengths, c.label_lengths,
                    c.durations, c.blank, c.sigma, "none")
    np.testing.assert_array_equal(rc["loss_utt"], r["loss_utt"])
    np.testing.assert_array_equal(rc["grad_tok"], r["grad_tok"])
    for b in range(c.B):
        rb = oracle.run(c.tok[b:b + 1], c.dur[b:b + 1], c.labels[b:b + 1], c.logit_lengths[b:b + 1],
                        c.label_lengths[b:b + 1], c.durations, c.blank, c.sigma, "none")
        assert rb["loss_utt"][0] == r["loss_utt"][b]
        np.testing.assert_array_equal(rb["grad_tok"][0], r["grad_tok"][b])


def test_reductions_and_gradient_weights():
    c = CASES["ragged"]()
    rn = _run(c, reduction="none")
    L = rn["loss_utt"]
    U = c.label_lengths.double().numpy()
    B = c.B
    expect = {"sum": L.sum(), "mean_batch": L.sum() / B, "mean": (L / np.maximum(U, 1)).sum() / B,
              "mean_volume": L.sum() / max(U.sum(), 1)}
    w = {"sum": np.ones(B), "mean_batch": np.full(B, 1.0 / B), "mean": 1.0 / (B * np.maximum(U, 1)),
         "mean_volume": np.full(B, 1.0 / max(U.sum(), 1))}
    for red, val in expect.items():
        r = _run(c, reduction=red)
        assert r["loss"] == pytest.approx(val, rel=1e-13)
        np.testing.assert_allclose(r["weight"], w[red], rtol=1e-15)
        np.testing.assert_allclose(r["grad_tok"], rn["grad_tok"] * w[red][:, None, None, None], rtol=1e-14,
                                   atol=1e-300)


def test_data_errors_poison_only_their_utterance():
    c = CASES["ragged"]()
    base = _run(c, reduction="none")
    c.labels[1, 0] = 33  # == V: out of range
    c.logit_lengths[2] = 41  # > Tmax
    r = _run(c, reduction="none")
    assert r["status"][1] == oracle.ST_BAD_LABEL and math.isnan(r["loss_utt"][1])
    assert r["status"][2] == oracle.ST_BAD_LOGIT_LENGTH and math.isnan(r["loss_utt"][2])
    assert not r["grad_tok"][1].any() and not r["grad_tok"][2].any()
    for b in (0, 3):
        assert r["status"][b] == 0 and r["loss_utt"][b] == base["loss_utt"][b]
    assert math.isnan(_run(c, reduction="sum")["loss"])
