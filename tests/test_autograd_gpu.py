"""GPU tests of the autograd layer (forward-only call, then ``tdt_loss_backward`` on the
kept workspace with the upstream gradient folded into the per-utterance weights) and of
in-place gradients (the gradient written over the logits).

With an upstream gradient of 1 the backward multiplies w_b by exactly 1.0 and runs the
kernels of the fused call on the same workspace state, so its gradients must equal the
fused call's bit for bit; other upstream gradients are checked against the float64
oracle, whose per-utterance gradients are scaled by the same factors."""
import numpy as np
import pytest
import torch

import tdt_transducer_loss_amd as tdt
from parity_util import TOL, check_grads, check_loss, gpu_run, max_abs_diff, oracle_run, say
from tdt_inputs import config_case, make_case

pytestmark = pytest.mark.gpu


def _ragged_extra_cols():
    return make_case(5, None, None, 129, [0, 1, 2, 3, 4], "f16", seed=70, Tmax=70, U1max=30, T_range=(1, 70),
                     U_range=(0, 29), reduction="mean", extra_cols=3, name="ragged_extra_cols")


CASES = {
    "tiny_f32": lambda: config_case(0),
    "parakeet_bf16": lambda: config_case(2),
    "ragged_f16": lambda: config_case(3),
    "ragged_extra_cols_f16": _ragged_extra_cols,
}


@pytest.mark.parametrize("name", list(CASES))
def test_autograd_unit_upstream_matches_fused_bitwise(name):
    case = CASES[name]().to("cuda")
    loss_f, g_f, gd_f, _ = gpu_run(case)
    snap = (loss_f.clone(), g_f.clone(), gd_f.clone())
    joint = case.joint.detach().clone().requires_grad_(True)
    V, D = case.V, case.D
    say(f"[gpu] autograd {name}: forward-only call, backward with upstream 1")
    loss = tdt.tdt_loss(joint[..., :V], joint[..., V:V + D], case.labels, case.logit_lengths, case.label_lengths,
                        case.durations, case.blank, case.sigma, case.reduction)
    if case.reduction == "none":
        loss.sum().backward()
    else:
        loss.backward()
    torch.cuda.synchronize()
    assert torch.equal(loss.detach().reshape(-1), snap[0].reshape(-1))
    assert torch.equal(joint.grad[..., :V], snap[1])
    assert torch.equal(joint.grad[..., V:V + D], snap[2])
    if joint.shape[-1] > V + D:  # columns past the duration logits get no gradient
        assert joint.grad[..., V + D:].abs().max().item() == 0


@pytest.mark.parametrize("reduction", ["none", "sum", "mean_volume"])
def test_autograd_upstream_scaling_against_oracle(reduction):
    """Upstream gradients other than 1: per utterance for 'none' (including a negative and
    a zero factor), a scalar otherwise."""
    case = make_case(4, None, None, 65, [0, 1, 2, 3, 4], "f32", seed=71, Tmax=30, U1max=12, T_range=(5, 30),
                     U_range=(1, 11), sigma=0.05).to("cuda")
    tok = case.tok.detach().clone().requires_grad_(True)
    dur = case.dur.detach().clone().requires_grad_(True)
    say(f"[gpu] autograd scaling, reduction {reduction}")
    loss = tdt.tdt_loss(tok, dur, case.labels, case.logit_lengths, case.label_lengths, case.durations, case.blank,
                        case.sigma, reduction)
    if reduction == "none":
        c = torch.tensor([0.5, -2.0, 0.0, 3.25], dtype=torch.float32, device="cuda")
        (loss * c).sum().backward()
        scale = c.double().cpu().numpy()
    else:
        loss.backward(torch.tensor(2.5, device="cuda"))
        scale = np.full(case.B, 2.5)
    torch.cuda.synchronize()
    orc = oracle_run(case.to("cpu"), reduction=reduction)
    check_loss(loss.detach(), orc, reduction, torch.float32)
    _, tg = TOL[torch.float32]
    shape = (-1, 1, 1, 1)
    e1 = max_abs_diff(tok.grad, orc["grad_tok"] * scale.reshape(shape))
    e2 = max_abs_diff(dur.grad, orc["grad_dur"] * scale.reshape(shape))
    say(f"    grad max-abs: token {e1:.3e} duration {e2:.3e}")
    assert e1 <= tg * np.abs(scale).max() and e2 <= tg * np.abs(scale).max()
    if reduction == "none":
        assert tok.grad[2].abs().max().item() == 0 and dur.grad[2].abs().max().item() == 0


def test_backward_entry_null_upstream_matches_fused_bitwise():
    """tdt_loss_backward with grad_loss = NULL (meaning 1), called through the C ABI."""
    from tdt_transducer_loss_amd import _native

    case = config_case(3, device="cuda")
    _, g_f, gd_f, _ = gpu_run(case)
    snap = (g_f.clone(), gd_f.clone())
    B, Tm, U1, V = case.tok.shape
    ws_bytes = tdt.workspace_size(1, B, Tm, U1, V, case.durations)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    say("[gpu] ragged_f16: forward-only call, then the backward entry point with NULL upstream")
    tdt.tdt_loss_fwd_bwd(case.tok, case.dur, case.labels, case.logit_lengths, case.label_lengths, case.durations,
                         case.blank, case.sigma, case.reduction, compute_grad=False, workspace=ws)
    g, gd = tdt.alloc_grads_like(case.tok, case.dur)
    rc = _native.backward_raw(1, B, Tm, U1, V, case.tok.data_ptr(), list(case.tok.stride()[:3]),
                              case.dur.data_ptr(), list(case.dur.stride()[:3]), case.D, case.labels.data_ptr(),
                              case.labels.stride(0), case.logit_lengths.data_ptr(), case.label_lengths.data_ptr(),
                              case.durations, case.blank, case.sigma, tdt.REDUCTIONS[case.reduction], None,
                              g.data_ptr(), list(g.stride()[:3]), gd.data_ptr(), list(gd.stride()[:3]),
                              ws.data_ptr(), ws_bytes, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(g, snap[0]) and torch.equal(gd, snap[1])


@pytest.mark.parametrize("name", list(CASES))
def test_inplace_gradient_matches_out_of_place_bitwise(name):
    """The gradient written over the logits equals the gradient written to a separate
    buffer; columns past the duration logits keep their values."""
    case = CASES[name]().to("cuda")
    loss_f, g_f, gd_f, _ = gpu_run(case)
    snap = (loss_f.clone(), g_f.clone(), gd_f.clone())
    joint = case.joint.clone()
    extra = joint[..., case.V + case.D:].clone()
    say(f"[gpu] in-place fused call {name}")
    loss, g, gd = tdt.tdt_loss_fwd_bwd(joint[..., :case.V], joint[..., case.V:case.V + case.D], case.labels,
                                       case.logit_lengths, case.label_lengths, case.durations, case.blank,
                                       case.sigma, case.reduction, inplace=True)
    torch.cuda.synchronize()
    assert g.data_ptr() == joint.data_ptr()
    assert torch.equal(loss, snap[0])
    assert torch.equal(joint[..., :case.V], snap[1]) and torch.equal(joint[..., case.V:case.V + case.D], snap[2])
    assert torch.equal(joint[..., case.V + case.D:], extra)


def test_autograd_inplace_gradient():
    """inplace_grad=True: the backward overwrites the logits with their gradient and hands
    those tensors to autograd; the values match the oracle."""
    case = config_case(0, device="cuda")
    tok = case.tok.detach().clone().requires_grad_(True)
    dur = case.dur.detach().clone().requires_grad_(True)
    say("[gpu] autograd with in-place gradients, tiny_f32")
    loss = tdt.tdt_loss(tok, dur, case.labels, case.logit_lengths, case.label_lengths, case.durations, case.blank,
                        case.sigma, "sum", inplace_grad=True)
    loss.backward()
    torch.cuda.synchronize()
    orc = oracle_run(case.to("cpu"), reduction="sum")
    check_loss(loss.detach(), orc, "sum", torch.float32)
    check_grads(tok.grad, dur.grad, orc, torch.float32)
    # the logits storage now holds the gradient
    assert torch.equal(tok.detach(), tok.grad) and torch.equal(dur.detach(), dur.grad)
