"""Helpers of the GPU parity tests: run the HIP path and the oracle on identical bits and
compare them element by element at the stated tolerances."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import tdt_transducer_loss_amd as tdt

# (loss relative error, gradient max-abs error) per logits dtype
TOL = {torch.float32: (1e-6, 1e-6), torch.float16: (1e-3, 2e-3), torch.bfloat16: (1e-3, 2e-3)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_run(case, compute_grad=True, grads=None, status=True, sigma=None, reduction=None):
    """Run the HIP path on a case that lives on the GPU."""
    st = torch.full((case.B,), -1, dtype=torch.int32, device=case.joint.device) if status else None
    g, gd = grads if grads is not None else (None, None)
    say(f"[gpu] {case.name} B={case.B} joint={tuple(case.joint.shape)} {case.joint.dtype} "
        f"red={reduction or case.reduction} grad={compute_grad}")
    loss, gt, gdd = tdt.tdt_loss_fwd_bwd(case.tok, case.dur, case.labels, case.logit_lengths, case.label_lengths,
                                         case.durations, case.blank, case.sigma if sigma is None else sigma,
                                         reduction or case.reduction, compute_grad=compute_grad,
                                         grad_logits=g, grad_dur_logits=gd, utt_status=st)
    torch.cuda.synchronize()
    return loss, gt, gdd, st


def oracle_run(case_cpu, **kw):
    return oracle.run(case_cpu.tok, case_cpu.dur, case_cpu.labels, case_cpu.logit_lengths,
                      case_cpu.label_lengths, case_cpu.durations, case_cpu.blank, kw.pop("sigma", case_cpu.sigma),
                      kw.pop("reduction", case_cpu.reduction), **kw)


def check_loss(gpu_loss: torch.Tensor, orc: dict, reduction: str, dtype):
    tl, _ = TOL[dtype]
    got = gpu_loss.detach().double().cpu().numpy().reshape(-1)
    exp = orc["loss_utt"] if reduction == "none" else np.array([orc["loss"]])
    assert got.shape == exp.shape
    for g, e in zip(got, exp):
        if math.isnan(e):
            assert math.isnan(g), (g, e)
        elif math.isinf(e):
            assert g == e, (g, e)
        else:
            assert abs(g - e) <= tl * abs(e) + 1e-30, (g, e, abs(g - e) / abs(e))


def max_abs_diff(gpu_grad: torch.Tensor, ref: np.ndarray, chunk_rows: int = 4096) -> float:
    """max |gpu - ref| over the whole tensor, in float64, streamed by rows."""
    g = gpu_grad.detach()
    B = g.shape[0]
    worst = 0.0
    gg = g.reshape(-1, g.shape[-1])
    rr = ref.reshape(-1, ref.shape[-1])
    for s in range(0, gg.shape[0], chunk_rows):
        a = gg[s:s + chunk_rows].double().cpu().numpy()
        d = np.abs(a - rr[s:s + chunk_rows])
        if np.isnan(d).any():
            return float("nan")
        worst = max(worst, float(d.max()))
    del B
    return worst


def check_grads(gt, gd, orc, dtype):
    _, tg = TOL[dtype]
    e1 = max_abs_diff(gt, orc["grad_tok"])
    e2 = max_abs_diff(gd, orc["grad_dur"])
    say(f"    grad max-abs: token {e1:.3e}  duration {e2:.3e}  (tol {tg:g})")
    assert e1 <= tg and e2 <= tg, (e1, e2)
    return e1, e2
