"""ctypes binding of libtdt_loss.so (include/tdt_loss.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtdt_loss.so")

TDT_OK = 0
TDT_ERR_INVALID_ARGUMENT = -1
TDT_ERR_UNSUPPORTED_DTYPE = -2
TDT_ERR_BAD_STRIDE = -3
TDT_ERR_WORKSPACE_TOO_SMALL = -4
TDT_ERR_UNSUPPORTED = -5
TDT_ERR_HIP = -6

UTT_BAD_LOGIT_LENGTH = 1
UTT_BAD_LABEL_LENGTH = 2
UTT_BAD_LABEL = 4
UTT_INFEASIBLE = 8

NOALLOC_SCRATCH_BYTES = 64 << 20  # TDT_NOALLOC_SCRATCH_BYTES of include/tdt_loss.h

# Every function the header declares, with its ctypes signature.
_i32, _i64, _vp, _f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
_i64p = ctypes.POINTER(ctypes.c_int64)
_i32p = ctypes.POINTER(ctypes.c_int32)
SIGNATURES = {
    "tdt_loss_workspace_size": (ctypes.c_int, [_i32, _i64, _i64, _i64, _i64, _i32p, _i32,
                                                ctypes.POINTER(ctypes.c_size_t)]),
    "tdt_loss_fwd_bwd": (ctypes.c_int, [
        _i32, _i64, _i64, _i64, _i64,       # dtype, B, T_max, U1_max, V
        _vp, _i64p, _vp, _i64p, _i32,       # logits, strides, dur_logits, strides, num_durations
        _vp, _i64, _vp, _vp,                # labels, labels_stride, logit_lengths, label_lengths
        _i32p, _i32, _f64, _i32,            # durations (host), blank, sigma, reduction
        _vp,                                # loss_out
        _vp, _i64p, _vp, _i64p,             # grad_logits, strides, grad_dur_logits, strides
        _vp, _vp, ctypes.c_size_t, _vp,     # utt_status, workspace, workspace_bytes, stream
    ]),
    "tdt_loss_fwd_bwd_timed": (ctypes.c_int, [
        _i32, _i64, _i64, _i64, _i64, _vp, _i64p, _vp, _i64p, _i32, _vp, _i64, _vp, _vp,
        _i32p, _i32, _f64, _i32, _vp, _vp, _i64p, _vp, _i64p, _vp, _vp, ctypes.c_size_t, _vp,
        ctypes.POINTER(ctypes.c_void_p), _i32,
    ]),
    "tdt_loss_backward": (ctypes.c_int, [
        _i32, _i64, _i64, _i64, _i64,       # dtype, B, T_max, U1_max, V
        _vp, _i64p, _vp, _i64p, _i32,       # logits, strides, dur_logits, strides, num_durations
        _vp, _i64, _vp, _vp,                # labels, labels_stride, logit_lengths, label_lengths
        _i32p, _i32, _f64, _i32,            # durations (host), blank, sigma, reduction
        _vp,                                # grad_loss
        _vp, _i64p, _vp, _i64p,             # grad_logits, strides, grad_dur_logits, strides
        _vp, ctypes.c_size_t, _vp,          # workspace, workspace_bytes, stream
    ]),
    "tdt_loss_fwd_bwd_noalloc": (ctypes.c_int, [
        _i32, _i64, _i64, _i64, _i64,       # dtype, B, T_max, U1_max, V
        _vp, _i64p, _vp, _i64p, _i32,       # logits, strides, dur_logits, strides, num_durations
        _vp, _i64, _vp, _vp,                # labels, labels_stride, logit_lengths, label_lengths
        _i32p, _i32, _f64, _i32,            # durations (host), blank, sigma, reduction
        _vp,                                # loss_out
        _vp, _i64p, _vp, _i64p,             # grad_logits, strides, grad_dur_logits, strides
        _vp, _vp,                           # utt_status, stream
    ]),
    "tdt_loss_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tdt_loss_abi_version": (ctypes.c_int, []),
}

_lib = None


class NativeLibraryMissing(RuntimeError):
    pass


def lib():
    """Load the HIP library (raises if it has not been built: there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NativeLibraryMissing(
                f"{LIB_PATH} is not built; run `python -m tdt_transducer_loss_amd.build` (hipcc, gfx950)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(code: int) -> str:
    return lib().tdt_loss_status_string(int(code)).decode()


def i64_array(vals):
    arr = (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])
    return arr


def i32_array(vals):
    return (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])


def workspace_size(dtype: int, B: int, T_max: int, U1_max: int, V: int, durations) -> int:
    d = i32_array(list(durations))
    out = ctypes.c_size_t(0)
    rc = lib().tdt_loss_workspace_size(int(dtype), int(B), int(T_max), int(U1_max), int(V), d, len(d),
                                       ctypes.byref(out))
    if rc != TDT_OK:
        raise ValueError(f"tdt_loss_workspace_size: {status_string(rc)} ({rc})")
    return int(out.value)


def fwd_bwd_raw(dtype, B, T_max, U1_max, V, logits, lstr, dur, dstr, D, labels, lab_stride, tlen, ulen,
                durations, blank, sigma, reduction, loss, glog, gstr, gdur, gdstr, status, ws, ws_bytes,
                stream, events=None) -> int:
    """Direct call with raw integers / pointers (device addresses as ints, None for NULL).
    With ``events`` (4 or 7 hipEvent_t handles as ints, see tdt_loss_fwd_bwd_timed) the
    timed entry point is used."""
    extra = ()
    fn = lib().tdt_loss_fwd_bwd
    if events is not None:
        fn = lib().tdt_loss_fwd_bwd_timed
        extra = ((ctypes.c_void_p * len(events))(*events), len(events))
    return fn(
        int(dtype), int(B), int(T_max), int(U1_max), int(V),
        logits, i64_array(lstr), dur, i64_array(dstr), int(D),
        labels, int(lab_stride), tlen, ulen,
        i32_array(durations), int(blank), float(sigma), int(reduction),
        loss,
        glog, i64_array(gstr) if gstr is not None else None, gdur, i64_array(gdstr) if gdstr is not None else None,
        status, ws, ctypes.c_size_t(int(ws_bytes)), stream, *extra,
    )


def backward_raw(dtype, B, T_max, U1_max, V, logits, lstr, dur, dstr, D, labels, lab_stride, tlen, ulen,
                 durations, blank, sigma, reduction, grad_loss, glog, gstr, gdur, gdstr, ws, ws_bytes, stream) -> int:
    """Direct call of tdt_loss_backward with raw integers / pointers (None for NULL)."""
    return lib().tdt_loss_backward(
        int(dtype), int(B), int(T_max), int(U1_max), int(V),
        logits, i64_array(lstr), dur, i64_array(dstr), int(D),
        labels, int(lab_stride), tlen, ulen,
        i32_array(durations), int(blank), float(sigma), int(reduction),
        grad_loss,
        glog, i64_array(gstr) if gstr is not None else None, gdur, i64_array(gdstr) if gdstr is not None else None,
        ws, ctypes.c_size_t(int(ws_bytes)), stream,
    )


def fwd_bwd_noalloc_raw(dtype, B, T_max, U1_max, V, logits, lstr, dur, dstr, D, labels, lab_stride, tlen, ulen,
                        durations, blank, sigma, reduction, loss, glog, gstr, gdur, gdstr, status, stream) -> int:
    """Direct call of tdt_loss_fwd_bwd_noalloc (no workspace arguments) with raw integers
    / pointers (None for NULL)."""
    return lib().tdt_loss_fwd_bwd_noalloc(
        int(dtype), int(B), int(T_max), int(U1_max), int(V),
        logits, i64_array(lstr), dur, i64_array(dstr), int(D),
        labels, int(lab_stride), tlen, ulen,
        i32_array(durations), int(blank), float(sigma), int(reduction),
        loss,
        glog, i64_array(gstr) if gstr is not None else None, gdur, i64_array(gdstr) if gdstr is not None else None,
        status, stream,
    )
