"""TEST INFRASTRUCTURE ONLY: the CPU float64 oracle of the TDT loss.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it, and the two
share no code: this package holds its own C source (``tdt_oracle.c``), a brute-force
path enumerator (``bruteforce.py``) and a closed form for all-zero logits
(``closed_form.py``).

The computation follows the kernel description on the page "tdt-loss: add TDT loss
kernel" (huggingface/kernels-community PR #882, comment "What's in it"): per-node
log-softmax over the vocabulary and over the durations, float64 alpha/beta over the
lattice, gradients for token and duration logits, and five reductions.

Pins (see tests/test_oracle_*.py): brute-force enumeration of every alignment on tiny
lattices, torch float64 autograd of that enumeration, a closed form for all-zero
logits, exact special cases (single duration 1, no labels), alpha/beta agreement,
zero-sum gradient rows, posterior count identities and central finite differences.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tdt_oracle.c")
LIB_PATH = os.path.join(_HERE, "libtdt_oracle.so")

REDUCTIONS = {"none": 0, "sum": 1, "mean": 2, "mean_batch": 3, "mean_volume": 4}
_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float64: 3}

ST_BAD_LOGIT_LENGTH = 1
ST_BAD_LABEL_LENGTH = 2
ST_BAD_LABEL = 4
ST_INFEASIBLE = 8

_lib = None


def build() -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, OpenMP)."""
    tmp = LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        i64, f64p, vp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.c_void_p
        lib.tdt_oracle_run.restype = ctypes.c_int
        lib.tdt_oracle_run.argtypes = (
            [ctypes.c_int] + [i64] * 5 + [vp, i64, i64, i64, vp, i64, i64, i64]
            + [vp, i64, vp, vp, vp, ctypes.c_int32, ctypes.c_double, ctypes.c_int]
            + [vp] * 6 + [vp] * 8 + [vp, vp] + [vp, i64, vp, vp, ctypes.c_int]
        )
        lib.tdt_oracle_max_threads.restype = ctypes.c_int
        lib.tdt_oracle_open.restype = ctypes.c_void_p
        lib.tdt_oracle_open.argtypes = (
            [ctypes.c_int] + [i64] * 5 + [vp, i64, i64, i64, vp, i64, i64, i64]
            + [vp, i64, vp, vp, vp, ctypes.c_int32, ctypes.c_double, ctypes.c_int]
            + [vp, vp, vp, ctypes.c_int]
        )
        lib.tdt_oracle_rows.restype = ctypes.c_int
        lib.tdt_oracle_rows.argtypes = [vp, i64, i64, vp, vp]
        lib.tdt_oracle_close.restype = None
        lib.tdt_oracle_close.argtypes = [vp]
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().tdt_oracle_max_threads())


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        return ctypes.c_void_p(a.data_ptr())
    return ctypes.c_void_p(a.ctypes.data)


def run(tok: torch.Tensor, dur: torch.Tensor, labels: torch.Tensor, logit_lengths: torch.Tensor,
        label_lengths: torch.Tensor, durations, blank: int, sigma: float = 0.0, reduction: str = "mean_volume",
        grads: bool = True, nodes: bool = False, rows=None, threads: int = 0) -> dict:
    """Evaluate loss, and optionally gradients / per-node posteriors, in float64.

    ``tok`` is the token-logit view [B, Tmax, U1max, V] and ``dur`` the duration-logit
    view [B, Tmax, U1max, D] (CPU tensors of dtype float32/float16/bfloat16, or float64
    for finite-difference checks; any strides
    with a unit last stride, e.g. two slices of one joint tensor).  ``labels`` is
    [B, >= U1max-1] int64 padded with -100.  ``rows`` is an optional list of padded node
    indices (b*Tmax + t)*U1max + u whose gradient rows are returned without building the
    full gradient.
    """
    lib = _load()
    assert tok.device.type == "cpu" and dur.device.type == "cpu"
    assert tok.dtype == dur.dtype and tok.dtype in _DTYPES
    assert tok.dim() == 4 and dur.dim() == 4 and tok.stride(3) == 1 and dur.stride(3) == 1
    B, Tmax, U1max, V = tok.shape
    D = dur.shape[3]
    assert tuple(dur.shape[:3]) == (B, Tmax, U1max)
    labels = labels.to(torch.int64).contiguous()
    if labels.dim() == 1:
        labels = labels.reshape(B, -1)
    Tl = logit_lengths.to(torch.int64).contiguous()
    Ul = label_lengths.to(torch.int64).contiguous()
    dd = np.ascontiguousarray(np.asarray(list(durations), dtype=np.int32))
    assert dd.shape[0] == D
    N = B * Tmax * U1max
    out = {
        "loss_utt": np.zeros(B), "loss": np.zeros(1), "logp_alpha": np.zeros(B), "logp_beta": np.zeros(B),
        "status": np.zeros(B, dtype=np.int32), "weight": np.zeros(B),
    }
    if nodes:
        for k in ("lse_h", "lse_g", "alpha", "beta", "occ", "cblank", "clabel"):
            out[k] = np.zeros(N)
        out["cdur"] = np.zeros(N * D)
    if grads:
        out["grad_tok"] = np.zeros(N * V)
        out["grad_dur"] = np.zeros(N * D)
    rows_arr = None
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out["rows_tok"] = np.zeros(rows_arr.shape[0] * V)
        out["rows_dur"] = np.zeros(rows_arr.shape[0] * D)
    g = out.get
    lib.tdt_oracle_run(
        _DTYPES[tok.dtype], B, Tmax, U1max, V, D,
        _ptr(tok), tok.stride(0), tok.stride(1), tok.stride(2),
        _ptr(dur), dur.stride(0), dur.stride(1), dur.stride(2),
        _ptr(labels), labels.stride(0), _ptr(Tl), _ptr(Ul), _ptr(dd), int(blank), float(sigma),
        REDUCTIONS[reduction],
        _ptr(out["loss_utt"]), _ptr(out["loss"]), _ptr(out["logp_alpha"]), _ptr(out["logp_beta"]),
        _ptr(out["status"]), _ptr(out["weight"]),
        _ptr(g("lse_h")), _ptr(g("lse_g")), _ptr(g("alpha")), _ptr(g("beta")), _ptr(g("occ")),
        _ptr(g("cblank")), _ptr(g("clabel")), _ptr(g("cdur")),
        _ptr(g("grad_tok")), _ptr(g("grad_dur")),
        _ptr(rows_arr), 0 if rows_arr is None else rows_arr.shape[0], _ptr(g("rows_tok")), _ptr(g("rows_dur")),
        int(threads),
    )
    if nodes:
        for k in ("lse_h", "lse_g", "alpha", "beta", "occ", "cblank", "clabel"):
            out[k] = out[k].reshape(B, Tmax, U1max)
        out["cdur"] = out["cdur"].reshape(B, Tmax, U1max, D)
    if grads:
        out["grad_tok"] = out["grad_tok"].reshape(B, Tmax, U1max, V)
        out["grad_dur"] = out["grad_dur"].reshape(B, Tmax, U1max, D)
    if rows_arr is not None:
        out["rows_tok"] = out["rows_tok"].reshape(-1, V)
        out["rows_dur"] = out["rows_dur"].reshape(-1, D)
    out["loss"] = float(out["loss"][0])
    return out


class Session:
    """The oracle's lattice, posteriors and losses of one batch, computed once; gradient
    rows are then produced a range of padded node indices at a time (for batches whose
    full float64 gradient would not fit in host memory).  Rows are bit-identical to the
    matching rows of :func:`run`'s ``grad_tok`` / ``grad_dur``.

    Arguments as in :func:`run`.  Use as a context manager; the input tensors are kept
    alive by the session."""

    def __init__(self, tok, dur, labels, logit_lengths, label_lengths, durations, blank, sigma=0.0,
                 reduction="mean_volume", threads: int = 0):
        lib = _load()
        assert tok.device.type == "cpu" and dur.device.type == "cpu"
        assert tok.dtype == dur.dtype and tok.dtype in _DTYPES
        assert tok.dim() == 4 and dur.dim() == 4 and tok.stride(3) == 1 and dur.stride(3) == 1
        B, Tmax, U1max, V = tok.shape
        D = dur.shape[3]
        labels = labels.to(torch.int64).contiguous()
        if labels.dim() == 1:
            labels = labels.reshape(B, -1)
        self._keep = (tok, dur, labels, logit_lengths.to(torch.int64).contiguous(),
                      label_lengths.to(torch.int64).contiguous(),
                      np.ascontiguousarray(np.asarray(list(durations), dtype=np.int32)))
        _, _, labels, Tl, Ul, dd = self._keep
        assert dd.shape[0] == D
        self.B, self.Tmax, self.U1max, self.V, self.D = B, Tmax, U1max, V, D
        self.loss_utt = np.zeros(B)
        loss = np.zeros(1)
        self.status = np.zeros(B, dtype=np.int32)
        self._h = lib.tdt_oracle_open(
            _DTYPES[tok.dtype], B, Tmax, U1max, V, D,
            _ptr(tok), tok.stride(0), tok.stride(1), tok.stride(2),
            _ptr(dur), dur.stride(0), dur.stride(1), dur.stride(2),
            _ptr(labels), labels.stride(0), _ptr(Tl), _ptr(Ul), _ptr(dd), int(blank), float(sigma),
            REDUCTIONS[reduction], _ptr(self.loss_utt), _ptr(loss), _ptr(self.status), int(threads))
        self.loss = float(loss[0])

    @property
    def nodes(self) -> int:
        return self.B * self.Tmax * self.U1max

    def rows(self, first: int, count: int, tok: bool = True, dur: bool = True):
        """Gradient rows of padded node indices [first, first + count): (tok [count, V],
        dur [count, D]) float64 arrays (None where not asked for)."""
        rt = np.zeros((count, self.V)) if tok else None
        rd = np.zeros((count, self.D)) if dur else None
        rc = _load().tdt_oracle_rows(self._h, int(first), int(count), _ptr(rt), _ptr(rd))
        if rc != 0:
            raise IndexError(f"rows [{first}, {first + count}) outside the batch")
        return rt, rd

    def close(self):
        if getattr(self, "_h", None):
            _load().tdt_oracle_close(self._h)
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        self.close()
