"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on identical
seeded inputs.  Tolerances: fp32 logits loss rel <= 1e-6 and gradient max-abs <= 1e-6;
fp16/bf16 logits loss rel <= 1e-3 and gradient max-abs <= 2e-3."""
import math

import numpy as np
import pytest
import torch

import tdt_transducer_loss_amd as tdt
from parity_util import TOL, check_grads, check_loss, gpu_run, oracle_run, say
from tdt_inputs import config_case, make_case

pytestmark = pytest.mark.gpu


def _full_parity(case, reduction=None):
    red = reduction or case.reduction
    loss, gt, gd, st = gpu_run(case, reduction=red)
    orc = oracle_run(case.to("cpu"), reduction=red)
    check_loss(loss, orc, red, case.joint.dtype)
    check_grads(gt, gd, orc, case.joint.dtype)
    np.testing.assert_array_equal(st.cpu().numpy(), orc["status"])
    return loss, gt, gd, orc


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_config_full_parity(cfg):
    """Workloads 0-3 at their full sizes; every loss and every gradient element."""
    case = config_case(cfg, device="cuda")
    _full_parity(case)


def test_long_label_config_full():
    """Workload 4 (B=2, T=1000, U=1500, V=1025, durations 0..8, bf16, sum): the loss, and
    every one of the 3,002,000 token and duration gradient rows against the oracle, read
    from an oracle session one range of rows at a time (the full float64 gradient would
    take about 25 GB of host memory)."""
    import oracle

    case = config_case(4, device="cuda")
    loss, gt, gd, st = gpu_run(case)
    cpu = case.to("cpu")
    _, tg = TOL[case.joint.dtype]
    V, D = case.V, case.D
    say("    oracle session (lattice and posteriors of both utterances)")
    with oracle.Session(cpu.tok, cpu.dur, cpu.labels, cpu.logit_lengths, cpu.label_lengths, cpu.durations,
                        cpu.blank, cpu.sigma, cpu.reduction) as s:
        check_loss(loss, {"loss": s.loss, "loss_utt": s.loss_utt}, case.reduction, case.joint.dtype)
        np.testing.assert_array_equal(st.cpu().numpy(), s.status)
        gt2 = gt.reshape(-1, V)
        gd2 = gd.reshape(-1, D)
        e1 = e2 = zs = 0.0
        chunk = 1 << 15
        for first in range(0, s.nodes, chunk):
            n = min(chunk, s.nodes - first)
            rt, rd = s.rows(first, n)
            g = gt2[first:first + n].cpu().double()
            e1 = max(e1, float((g - torch.from_numpy(rt)).abs().max()))
            e2 = max(e2, float((gd2[first:first + n].cpu().double() - torch.from_numpy(rd)).abs().max()))
            # zero-sum rows: the exact row sums to 0; each stored element is the
            # round-to-nearest-even bf16 value (8 significant bits: off by at most 2^-8 of
            # its magnitude) of a float32 result whose own relative error is below 2^-20,
            # so |sum_v g_v| <= (2^-8 + 2^-20) sum_v |g_v| (+ a subnormal allowance)
            excess = (g.sum(-1).abs() - (2.0 ** -8 + 2.0 ** -20) * g.abs().sum(-1) - 1e-30).max()
            zs = max(zs, float(excess))
            if first % (chunk * 16) == 0:
                say(f"    rows {first}..{first + n}: token {e1:.3e} duration {e2:.3e}")
    say(f"    full grad max-abs: token {e1:.3e}  duration {e2:.3e}  (tol {tg:g}); zero-sum excess {zs:.3e}")
    assert e1 <= tg and e2 <= tg
    assert zs <= 0.0


def _plain_sweep_underflow():
    # blank logits 200 above the rest: every move weight stays above 2^-300, so the plain
    # sweep runs (151 labels: three bands of 64-label tiles), but each label costs about
    # 2^-290, so the values along one anti-diagonal lie tens of thousands of binary orders
    # apart; the per-lane scales and the range check (a value leaving [2^-700, 2^700] sends
    # the tile to the extended-range sweep) must keep every node's value exact
    case = make_case(2, [40, 30], [150, 20], 5, [0, 1, 2], "f32", seed=57, reduction="none")
    case.joint[..., 4] += 200.0
    return case


def _all_negative(dtype):
    # every token logit below zero (shifted by -60; the loss is unchanged by the shift): the
    # bf16 row maximum of every segment comes from the order-preserving key pass
    case = make_case(2, [9, 7], [3, 4], 3000, [0, 1, 2, 4], dtype, seed=58, scale=2.0, reduction="none")
    case.joint[..., :3000] -= 60.0
    return case


def _masked(dtype):
    # logits masked with -1e10 (a common way to forbid a token or a duration): the blank
    # logit of some nodes, a duration logit of others, and both at a few; the move weights
    # there are exactly zero (log-weight far below the extended range) and the gradients
    # must stay finite and match the oracle, which works in the log domain
    case = make_case(2, [30, 22], [9, 6], 33, [0, 1, 2, 3, 4], dtype, seed=59, sigma=0.05, reduction="none")
    V = case.V
    g = torch.Generator().manual_seed(5)
    for b in range(case.B):
        T, U = int(case.logit_lengths[b]), int(case.label_lengths[b])
        for _ in range(12):
            t = int(torch.randint(1, T - 1, (1,), generator=g))
            u = int(torch.randint(0, U + 1, (1,), generator=g))
            what = int(torch.randint(0, 3, (1,), generator=g))
            if what in (0, 2):
                case.joint[b, t, u, case.blank] = -1e10
            if what in (1, 2):
                case.joint[b, t, u, V + int(torch.randint(0, case.D, (1,), generator=g))] = -1e10
    return case


EDGE = {
    "no_labels": lambda: make_case(3, [7, 5, 9], [0, 0, 0], 11, [0, 1, 2, 3, 4], "f32", seed=41, sigma=0.1,
                                   reduction="sum", U1max=2),
    "single_frame": lambda: make_case(2, [1, 2], [0, 1], 6, [0, 1, 2], "f32", seed=42, reduction="none"),
    "blank_first_label_is_blank": lambda: make_case(2, [9, 6], [4, 2], 13, [0, 1, 2, 3], "f32", seed=43,
                                                    reduction="none", blank=0, label_high=13),
    "durations_unsorted_no_zero": lambda: make_case(2, [11, 8], [3, 3], 9, [3, 1, 2], "bf16", seed=44,
                                                    reduction="mean", sigma=-0.2),
    "single_duration_1": lambda: make_case(2, [10, 7], [4, 6], 9, [1], "f16", seed=45, reduction="mean_batch"),
    "more_labels_than_frames": lambda: make_case(2, [6, 4], [12, 9], 17, [0, 1, 2], "f32", seed=46,
                                                 reduction="mean_volume"),
    "max_duration_16": lambda: make_case(2, [40, 33], [7, 5], 10, [0, 1, 5, 16, 9], "f32", seed=47,
                                         reduction="sum", sigma=0.05),
    "duration_8_long_labels": lambda: make_case(1, [30], [300], 21, list(range(9)), "bf16", seed=48,
                                              reduction="sum"),
    "long_labels_1100": lambda: make_case(1, [12], [1100], 7, [0, 1, 2], "f32", seed=49, reduction="sum"),
    "wide_vocab_multipass": lambda: make_case(1, [5], [2], 40000, [0, 1, 2, 3, 4], "bf16", seed=50,
                                              reduction="none"),
    "tiny_vocab": lambda: make_case(2, [8, 6], [3, 2], 2, [0, 1, 2], "f32", seed=51, reduction="none",
                                    label_high=1),
    # logits of standard deviation 12: move weights down to about e^-160, lattice values
    # spread over hundreds of binary orders within one anti-diagonal
    "large_logits_plain_range": lambda: make_case(2, [60, 45], [30, 20], 33, [0, 1, 2, 3, 4], "f32", seed=53,
                                                  scale=12.0, reduction="sum"),
    # standard deviation 400: weights far below 2^-300 (extended-range lattice path)
    "huge_logits_extended_range": lambda: make_case(2, [40, 31], [12, 9], 17, [0, 1, 2], "f32", seed=54,
                                                    scale=400.0, reduction="none"),
    # 300 labels with weights far below 2^-300: linked columns redone in extended range
    "huge_logits_long_labels": lambda: make_case(1, [24], [300], 9, [0, 1, 2], "f32", seed=55, scale=400.0,
                                               reduction="sum"),
    "plain_sweep_underflow_redo": _plain_sweep_underflow,
    "all_negative_logits_bf16": lambda: _all_negative("bf16"),
    "all_negative_logits_f16": lambda: _all_negative("f16"),
    "ragged_padded_f16": lambda: make_case(5, None, None, 129, [0, 1, 2, 3, 4], "f16", seed=52, Tmax=70, U1max=30,
                                           T_range=(1, 70), U_range=(0, 29), reduction="mean", extra_cols=3),
    "masked_minus_1e10_f32": lambda: _masked("f32"),
    "masked_minus_1e10_bf16": lambda: _masked("bf16"),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_case_parity(name):
    _full_parity(EDGE[name]().to("cuda"))


@pytest.mark.parametrize("reduction", ["none", "sum", "mean", "mean_batch", "mean_volume"])
def test_every_reduction(reduction):
    case = make_case(4, None, None, 65, [0, 1, 2, 3, 4], "f32", seed=60, Tmax=30, U1max=12, T_range=(5, 30),
                     U_range=(1, 11), sigma=0.05, device="cuda")
    _full_parity(case, reduction=reduction)


def test_infeasible_and_data_errors():
    case = make_case(5, [8, 5, 8, 8, 7], [2, 1, 3, 2, 2], 10, [2, 4], "f32", seed=61, reduction="none",
                     device="cuda", Tmax=10, U1max=5)
    # utt 1: durations {2,4} and T=5 (odd): no alignment; utt 2: a label out of range;
    # utt 3: logit length beyond T_max; utt 4: zero frames
    case.labels[2, 1] = 10
    case.logit_lengths[3] = 11
    case.logit_lengths[4] = 0
    loss, gt, gd, st = gpu_run(case)
    orc = oracle_run(case.to("cpu"))
    check_loss(loss, orc, "none", torch.float32)
    check_grads(gt, gd, orc, torch.float32)
    s = st.cpu().numpy()
    assert s[0] == 0 and s[1] == tdt.UTT_INFEASIBLE and s[2] == tdt.UTT_BAD_LABEL
    assert s[3] == tdt.UTT_BAD_LOGIT_LENGTH and s[4] == tdt.UTT_INFEASIBLE
    l = loss.cpu().numpy()
    assert math.isinf(l[1]) and math.isnan(l[2]) and math.isnan(l[3]) and math.isinf(l[4])
    for b in (1, 2, 3, 4):
        assert gt[b].abs().max().item() == 0 and gd[b].abs().max().item() == 0


@pytest.mark.parametrize("cfg", [0, 3])
def test_forward_only_matches(cfg):
    """The forward-only call (no gradient pointers) gives the loss of the fused call bit
    for bit, and the oracle's loss within the tolerance."""
    case = config_case(cfg, device="cuda")
    loss_f, g, gd, st = gpu_run(case, compute_grad=False)
    assert g is None and gd is None
    orc = oracle_run(case.to("cpu"), grads=False)
    check_loss(loss_f, orc, case.reduction, case.joint.dtype)
    np.testing.assert_array_equal(st.cpu().numpy(), orc["status"])
    loss_b, _, _, _ = gpu_run(case)
    assert torch.equal(loss_f, loss_b)


def test_separate_gradient_buffers_unaligned_path():
    """Gradients in separate contiguous buffers while the logits are slices of a joint
    tensor of odd width: logits and gradient rows are not co-aligned (per-element path)."""
    case = make_case(2, [9, 7], [3, 4], 37, [0, 1, 2, 3], "bf16", seed=62, reduction="mean", extra_cols=1,
                     device="cuda")
    g = torch.full(case.tok.shape, float("nan"), dtype=case.joint.dtype, device="cuda")
    gd = torch.full(case.dur.shape, float("nan"), dtype=case.joint.dtype, device="cuda")
    loss, gt, gdd, _ = gpu_run(case, grads=(g, gd))
    orc = oracle_run(case.to("cpu"))
    check_loss(loss, orc, "mean", case.joint.dtype)
    check_grads(gt, gdd, orc, case.joint.dtype)


def test_padding_rows_written_by_gradient_pass():
    """Gradient views with the logits' strides (rows co-aligned, the short-row gradient
    pass) in two separate buffers, so not one joint tensor: the lattice launch zeroes no
    padding rows and the gradient pass writes them itself (frame pieces outside the
    utterances included).  Every element of both views is written (NaN canaries disappear)
    and the result is bitwise that of the joint-buffer run."""
    case = config_case(3, device="cuda")
    loss_j, g_j, gd_j, _ = gpu_run(case)
    snap = (loss_j.clone(), g_j.clone(), gd_j.clone())
    n = case.joint.numel()
    g = torch.full((n,), float("nan"), dtype=case.joint.dtype, device="cuda").as_strided(
        case.tok.shape, case.tok.stride(), 0)
    gd = torch.full((n,), float("nan"), dtype=case.joint.dtype, device="cuda").as_strided(
        case.dur.shape, case.dur.stride(), 0)
    loss, gt, gdd, _ = gpu_run(case, grads=(g, gd))
    assert not torch.isnan(gt).any().item() and not torch.isnan(gdd).any().item()
    assert torch.equal(loss, snap[0]) and torch.equal(gt, snap[1]) and torch.equal(gdd, snap[2])


def test_padding_canary_and_determinism():
    """Every element of the gradient views is written (NaN canaries disappear) and two runs
    are bitwise identical."""
    case = config_case(3, device="cuda")
    g, gd = tdt.alloc_grads_like(case.tok, case.dur)
    g.fill_(float("nan"))
    gd.fill_(float("nan"))
    loss1, g1, gd1, _ = gpu_run(case, grads=(g, gd))
    assert not torch.isnan(g1).any().item() and not torch.isnan(gd1).any().item()
    snap = (loss1.clone(), g1.clone(), gd1.clone())
    loss2, g2, gd2, _ = gpu_run(case)
    assert torch.equal(snap[0], loss2) and torch.equal(snap[1], g2) and torch.equal(snap[2], gd2)


@pytest.mark.parametrize("n_events", [4, 7])
def test_timed_entry_point_matches_plain_bitwise(n_events):
    """The timed entry point (events between the kernels) produces the bits of the plain
    entry point."""
    from tdt_transducer_loss_amd import _native

    case = config_case(3, device="cuda")
    loss_a, ga, gda, _ = gpu_run(case)
    snap = (loss_a.clone(), ga.clone(), gda.clone())
    g, gd = tdt.alloc_grads_like(case.tok, case.dur)
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    B, Tm, U1, V = case.tok.shape
    ws_bytes = tdt.workspace_size(1, B, Tm, U1, V, case.durations)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_events)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    say(f"[gpu] ragged_f16 through the timed entry point, {n_events} events")
    rc = _native.fwd_bwd_raw(1, B, Tm, U1, V, case.tok.data_ptr(), list(case.tok.stride()[:3]),
                             case.dur.data_ptr(), list(case.dur.stride()[:3]), case.D, case.labels.data_ptr(),
                             case.labels.stride(0), case.logit_lengths.data_ptr(), case.label_lengths.data_ptr(),
                             case.durations, case.blank, case.sigma, tdt.REDUCTIONS[case.reduction],
                             loss.data_ptr(), g.data_ptr(), list(g.stride()[:3]), gd.data_ptr(),
                             list(gd.stride()[:3]), None, ws.data_ptr(), ws_bytes,
                             torch.cuda.current_stream().cuda_stream, events=[e.cuda_event for e in evs])
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(snap[0].reshape(1), loss) and torch.equal(snap[1], g) and torch.equal(snap[2], gd)
    order = [0, 2, 3, 1] if n_events == 4 else list(range(7))  # recording order on the stream
    times = [evs[a].elapsed_time(evs[b]) for a, b in zip(order, order[1:])]
    assert all(x >= 0.0 for x in times)
