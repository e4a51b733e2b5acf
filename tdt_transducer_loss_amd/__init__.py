"""MI355X (gfx950) Token-and-Duration Transducer loss, forward and backward.

The computation runs in hand-written HIP kernels behind the C ABI of
``include/tdt_loss.h`` (``libtdt_loss.so``); this module only marshals PyTorch
tensors (device memory and the current stream) into that ABI.  There is no CPU or
PyTorch fallback: calling it without the built library or on a non-GPU tensor raises.
"""
from __future__ import annotations

import torch

from . import _native
from ._native import (TDT_OK, UTT_BAD_LABEL, UTT_BAD_LABEL_LENGTH, UTT_BAD_LOGIT_LENGTH, UTT_INFEASIBLE,
                      NativeLibraryMissing, status_string, workspace_size)

REDUCTIONS = {"none": 0, "sum": 1, "mean": 2, "mean_batch": 3, "mean_volume": 4}
_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

__all__ = ["tdt_loss", "TDTLoss", "tdt_loss_fwd_bwd", "workspace_size", "status_string", "REDUCTIONS",
           "NativeLibraryMissing", "TDTLossError", "UTT_BAD_LOGIT_LENGTH", "UTT_BAD_LABEL_LENGTH", "UTT_BAD_LABEL", "UTT_INFEASIBLE",
           "alloc_grads_like"]


class TDTLossError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"TDT loss call failed: {status_string(code)} ({code})")
        self.code = code


def _strides3(t: torch.Tensor):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a 4-D view [B, T, U+1, C] with a unit stride in the last dimension")
    return [t.stride(0), t.stride(1), t.stride(2)]


def alloc_grads_like(logits: torch.Tensor, dur_logits: torch.Tensor):
    """Gradient buffers with the exact memory layout of the logit views.

    When both views are slices of one joint tensor, the gradients are the same slices of
    one new joint buffer, so logits rows and gradient rows share their alignment."""
    if logits.untyped_storage().data_ptr() == dur_logits.untyped_storage().data_ptr():
        elt = logits.element_size()
        n = logits.untyped_storage().nbytes() // elt
        flat = torch.empty(n, dtype=logits.dtype, device=logits.device)
        g = flat.as_strided(logits.shape, logits.stride(), logits.storage_offset())
        gd = flat.as_strided(dur_logits.shape, dur_logits.stride(), dur_logits.storage_offset())
        return g, gd
    return torch.empty_like(logits), torch.empty_like(dur_logits)


def _marshal(logits, dur_logits, labels, logit_lengths, label_lengths, durations):
    """Checks the logits views and brings labels and lengths to contiguous int64 on the
    logits' device.  Returns (dtype code, B, T_max, U1_max, V, D, labels, tl, ul)."""
    if logits.device.type != "cuda":
        raise ValueError("the TDT loss runs on the GPU only")
    if logits.dtype not in _DTYPES or dur_logits.dtype != logits.dtype:
        raise ValueError(f"unsupported logits dtype {logits.dtype}")
    B, T_max, U1_max, V = logits.shape
    D = len(list(durations))
    if tuple(dur_logits.shape) != (B, T_max, U1_max, D):
        raise ValueError("dur_logits must be [B, T_max, U1_max, len(durations)]")
    dev = logits.device
    labels = labels.to(device=dev, dtype=torch.int64)
    if labels.dim() != 2 or labels.stride(1) != 1:
        labels = labels.reshape(B, -1).contiguous()
    if labels.shape[1] < U1_max - 1:
        raise ValueError("labels need at least U1_max - 1 columns")
    tl = logit_lengths.to(device=dev, dtype=torch.int64).contiguous()
    ul = label_lengths.to(device=dev, dtype=torch.int64).contiguous()
    return _DTYPES[logits.dtype], B, T_max, U1_max, V, D, labels, tl, ul


def tdt_loss_fwd_bwd(logits: torch.Tensor, dur_logits: torch.Tensor, labels: torch.Tensor,
                     logit_lengths: torch.Tensor, label_lengths: torch.Tensor, durations, blank: int,
                     sigma: float = 0.0, reduction: str = "mean_volume", compute_grad: bool = True,
                     grad_logits: torch.Tensor | None = None, grad_dur_logits: torch.Tensor | None = None,
                     utt_status: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     inplace: bool = False):
    """TDT loss and gradients on the current HIP stream.

    logits: token logits [B, T_max, U1_max, V] (e.g. ``joint[..., :V]``); dur_logits:
    duration logits [B, T_max, U1_max, D] (e.g. ``joint[..., V:]``); float32, float16 or
    bfloat16 GPU tensors read in place.  labels: int64 [B, >= U1_max-1], -100 padded.
    Returns ``(loss, grad_logits, grad_dur_logits)``; the gradients are None when
    ``compute_grad`` is False.  ``loss`` is float32 [B] for ``reduction='none'`` and a
    0-d tensor otherwise.  ``inplace=True`` writes the gradients over the logits (the
    returned gradients are then the ``logits`` and ``dur_logits`` tensors themselves).
    """
    dt, B, T_max, U1_max, V, D, labels, tl, ul = _marshal(logits, dur_logits, labels, logit_lengths,
                                                          label_lengths, durations)
    dev = logits.device
    red = REDUCTIONS[reduction]
    loss = torch.empty(B if red == 0 else 1, dtype=torch.float32, device=dev)
    if compute_grad and inplace:
        grad_logits, grad_dur_logits = logits, dur_logits
    if compute_grad and (grad_logits is None or grad_dur_logits is None):
        grad_logits, grad_dur_logits = alloc_grads_like(logits, dur_logits)
    if not compute_grad:
        grad_logits = grad_dur_logits = None
    nbytes = workspace_size(dt, B, T_max, U1_max, V, durations)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = _native.fwd_bwd_raw(
        dt, B, T_max, U1_max, V,
        logits.data_ptr(), _strides3(logits), dur_logits.data_ptr(), _strides3(dur_logits), D,
        labels.data_ptr(), labels.stride(0), tl.data_ptr(), ul.data_ptr(),
        list(durations), blank, sigma, red,
        loss.data_ptr(),
        grad_logits.data_ptr() if grad_logits is not None else None,
        _strides3(grad_logits) if grad_logits is not None else None,
        grad_dur_logits.data_ptr() if grad_dur_logits is not None else None,
        _strides3(grad_dur_logits) if grad_dur_logits is not None else None,
        utt_status.data_ptr() if utt_status is not None else None,
        workspace.data_ptr(), workspace.numel(), stream,
    )
    if rc != TDT_OK:
        raise TDTLossError(rc)
    if red != 0:
        loss = loss[0]
    return loss, grad_logits, grad_dur_logits


class _TDTLossFunction(torch.autograd.Function):
    """Forward: the forward-only launch sequence (loss written, workspace kept).
    Backward: ``tdt_loss_backward`` on that workspace with the upstream gradient folded
    into the per-utterance weights, so no extra pass scales the gradients."""

    @staticmethod
    def forward(ctx, logits, dur_logits, labels, logit_lengths, label_lengths, durations, blank, sigma, reduction,
                inplace):
        dt, B, T_max, U1_max, V, D, labels, tl, ul = _marshal(logits, dur_logits, labels, logit_lengths,
                                                              label_lengths, durations)
        durations = [int(d) for d in durations]
        ws = torch.empty(workspace_size(dt, B, T_max, U1_max, V, durations), dtype=torch.uint8,
                         device=logits.device)
        loss, _, _ = tdt_loss_fwd_bwd(logits, dur_logits, labels, tl, ul, durations, blank, sigma, reduction,
                                      compute_grad=False, workspace=ws)
        ctx.save_for_backward(logits, dur_logits)
        # labels and lengths are read again by the backward kernels: keep the marshalled copies
        ctx.state = (dt, B, T_max, U1_max, V, D, labels, tl, ul, durations, int(blank), float(sigma),
                     REDUCTIONS[reduction], ws, bool(inplace))
        return loss

    @staticmethod
    def backward(ctx, grad_loss):
        logits, dur_logits = ctx.saved_tensors
        dt, B, T_max, U1_max, V, D, labels, tl, ul, durations, blank, sigma, red, ws, inplace = ctx.state
        if inplace:
            g, gd = logits, dur_logits
        else:
            g, gd = alloc_grads_like(logits, dur_logits)
        gl = grad_loss.detach().to(device=logits.device, dtype=torch.float32).reshape(-1).contiguous()
        if gl.numel() != (B if red == 0 else 1):
            raise ValueError("unexpected shape of the upstream loss gradient")
        stream = torch.cuda.current_stream(logits.device).cuda_stream
        rc = _native.backward_raw(
            dt, B, T_max, U1_max, V,
            logits.data_ptr(), _strides3(logits), dur_logits.data_ptr(), _strides3(dur_logits), D,
            labels.data_ptr(), labels.stride(0), tl.data_ptr(), ul.data_ptr(),
            durations, blank, sigma, red, gl.data_ptr(),
            g.data_ptr(), _strides3(g), gd.data_ptr(), _strides3(gd),
            ws.data_ptr(), ws.numel(), stream,
        )
        if rc != TDT_OK:
            raise TDTLossError(rc)
        ctx.state = None  # the workspace holds one forward's state: one backward per forward
        return g, gd, None, None, None, None, None, None, None, None


def tdt_loss(logits: torch.Tensor, dur_logits: torch.Tensor, labels: torch.Tensor, logit_lengths: torch.Tensor,
             label_lengths: torch.Tensor, durations, blank: int, sigma: float = 0.0,
             reduction: str = "mean_volume", inplace_grad: bool = False) -> torch.Tensor:
    """Differentiable TDT loss (autograd).  Arguments as in :func:`tdt_loss_fwd_bwd`.

    ``inplace_grad=True`` makes the backward write the gradients over ``logits`` and
    ``dur_logits`` and hand those tensors to autograd as their gradients: it saves a
    logits-sized buffer, but the logits' values are gone after the backward, so nothing
    else may read them afterwards (autograd does not see this write)."""
    if reduction not in REDUCTIONS:
        raise ValueError(f"unknown reduction {reduction!r}")
    return _TDTLossFunction.apply(logits, dur_logits, labels, logit_lengths, label_lengths, list(durations), blank,
                                  sigma, reduction, inplace_grad)


class TDTLoss(torch.nn.Module):
    """Stateless layer around :func:`tdt_loss` (module form, for code that swaps layers)."""

    def forward(self, logits, dur_logits, labels, logit_lengths, label_lengths, durations, blank, sigma=0.0,
                reduction="mean_volume", inplace_grad=False):
        return tdt_loss(logits, dur_logits, labels, logit_lengths, label_lengths, durations, blank, sigma,
                        reduction, inplace_grad)
