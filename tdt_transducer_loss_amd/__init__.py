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

__all__ = ["tdt_loss_fwd_bwd", "workspace_size", "status_string", "REDUCTIONS", "NativeLibraryMissing",
           "TDTLossError", "UTT_BAD_LOGIT_LENGTH", "UTT_BAD_LABEL_LENGTH", "UTT_BAD_LABEL", "UTT_INFEASIBLE",
           "alloc_grads_like"]


class TDTLossError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"tdt_loss_fwd_bwd failed: {status_string(code)} ({code})")
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


def tdt_loss_fwd_bwd(logits: torch.Tensor, dur_logits: torch.Tensor, labels: torch.Tensor,
                     logit_lengths: torch.Tensor, label_lengths: torch.Tensor, durations, blank: int,
                     sigma: float = 0.0, reduction: str = "mean_volume", compute_grad: bool = True,
                     grad_logits: torch.Tensor | None = None, grad_dur_logits: torch.Tensor | None = None,
                     utt_status: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """TDT loss and gradients on the current HIP stream.

    logits: token logits [B, T_max, U1_max, V] (e.g. ``joint[..., :V]``); dur_logits:
    duration logits [B, T_max, U1_max, D] (e.g. ``joint[..., V:]``); float32, float16 or
    bfloat16 GPU tensors read in place.  labels: int64 [B, >= U1_max-1], -100 padded.
    Returns ``(loss, grad_logits, grad_dur_logits)``; the gradients are None when
    ``compute_grad`` is False.  ``loss`` is float32 [B] for ``reduction='none'`` and a
    0-d tensor otherwise.
    """
    if logits.device.type != "cuda":
        raise ValueError("tdt_loss_fwd_bwd runs on the GPU only")
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
    red = REDUCTIONS[reduction]
    loss = torch.empty(B if red == 0 else 1, dtype=torch.float32, device=dev)
    if compute_grad and (grad_logits is None or grad_dur_logits is None):
        grad_logits, grad_dur_logits = alloc_grads_like(logits, dur_logits)
    if not compute_grad:
        grad_logits = grad_dur_logits = None
    nbytes = workspace_size(_DTYPES[logits.dtype], B, T_max, U1_max, V, durations)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = _native.fwd_bwd_raw(
        _DTYPES[logits.dtype], B, T_max, U1_max, V,
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
