"""Host-side checks of the C ABI that need no GPU: the library loads, exports every
function include/tdt_loss.h declares, and rejects invalid arguments with the documented
codes before it launches anything (every call below is invalid on purpose, so nothing
reaches the device even on a GPU machine)."""
import ctypes
import os
import re

import pytest

from tdt_transducer_loss_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(tdt_\w+)\s*\(", src, flags=re.M))
    return names


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"tdt_loss_fwd_bwd", "tdt_loss_workspace_size", "tdt_loss_status_string",
            "tdt_loss_abi_version", "tdt_loss_fwd_bwd_timed", "tdt_loss_backward",
            "tdt_loss_fwd_bwd_noalloc"} <= names
    lib = _native.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(_native.SIGNATURES) == names


def test_status_strings():
    for code in range(0, -7, -1):
        assert _native.status_string(code) != "unknown status"
    assert _native.status_string(-99) == "unknown status"
    assert _native.lib().tdt_loss_abi_version() == 3


def test_workspace_size():
    small = _native.workspace_size(0, 1, 10, 5, 17, [0, 1, 2])
    big = _native.workspace_size(2, 4, 200, 41, 8193, [0, 1, 2, 3, 4])
    assert 0 < small < big
    assert big % 256 == 0
    for bad in ([], [0], [1, 1], [-1, 1], [0, 17]):
        with pytest.raises(ValueError):
            _native.workspace_size(0, 1, 10, 5, 17, bad)
    # no label-count limit: a long label sequence only needs its workspace
    assert _native.workspace_size(0, 1, 10, 20000, 17, [0, 1]) > 0
    with pytest.raises(ValueError):  # one utterance's box beyond 2^27 nodes
        _native.workspace_size(0, 1, 20000, 20000, 17, [0, 1])
    with pytest.raises(ValueError):
        _native.workspace_size(0, 0, 10, 5, 17, [0, 1])
    with pytest.raises(ValueError):
        _native.workspace_size(3, 1, 10, 5, 17, [0, 1])


FAKE = 1 << 20  # a 256-aligned non-null address that is never dereferenced


def _call(**over):
    args = dict(dtype=2, B=2, T_max=10, U1_max=5, V=9, logits=FAKE, lstr=[450, 45, 9], dur=FAKE + 4096,
                dstr=[450, 45, 9], D=3, labels=FAKE, lab_stride=4, tlen=FAKE, ulen=FAKE, durations=[0, 1, 2],
                blank=8, sigma=0.0, reduction=3, loss=FAKE, glog=None, gstr=None, gdur=None, gdstr=None,
                status=None, ws=FAKE, ws_bytes=0, stream=None)
    args.update(over)
    return _native.fwd_bwd_raw(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(dtype=3), _native.TDT_ERR_UNSUPPORTED_DTYPE),
    (dict(dtype=-1), _native.TDT_ERR_UNSUPPORTED_DTYPE),
    (dict(reduction=5), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(logits=None), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(loss=None), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(ws=None), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(blank=9), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(blank=-1), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(sigma=float("nan")), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(sigma=float("inf")), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(V=0), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(durations=[0, 0, 1]), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(durations=[0], D=1), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(durations=[0, 1, 99]), _native.TDT_ERR_UNSUPPORTED),
    (dict(T_max=20000, U1_max=9000, lab_stride=9000), _native.TDT_ERR_UNSUPPORTED),
    (dict(lab_stride=2), _native.TDT_ERR_BAD_STRIDE),
    (dict(glog=FAKE), _native.TDT_ERR_INVALID_ARGUMENT),  # one gradient pointer without the other
    (dict(), _native.TDT_ERR_WORKSPACE_TOO_SMALL),          # ws_bytes = 0
    (dict(ws_bytes=1 << 40, logits=FAKE + 1), _native.TDT_ERR_BAD_STRIDE),
    (dict(ws_bytes=1 << 40, ws=FAKE + 8), _native.TDT_ERR_BAD_STRIDE),
])
def test_invalid_arguments_are_rejected(over, code):
    assert _call(**over) == code


@pytest.mark.parametrize("n_events", [0, 1, 2, 3, 5, 6, 8, 11])
def test_timed_entry_rejects_bad_event_lists(n_events):
    lib = _native.lib()
    i64 = _native.i64_array
    evs = (ctypes.c_void_p * max(n_events, 1))()
    rc = lib.tdt_loss_fwd_bwd_timed(2, 2, 10, 5, 9, FAKE, i64([1, 1, 1]), FAKE, i64([1, 1, 1]), 3, FAKE, 4, FAKE,
                                    FAKE, _native.i32_array([0, 1, 2]), 8, 0.0, 3, FAKE, None, None, None, None,
                                    None, FAKE, ctypes.c_size_t(1 << 40), None, evs, n_events)
    assert rc == _native.TDT_ERR_INVALID_ARGUMENT


# Gradient views against the logits views of _call's shape (B 2, T 10, U1 5, V 9, D 3,
# rows of 450/45/9 elements; bf16): the token logits span FAKE .. FAKE + 900 B.
@pytest.mark.parametrize("over,code", [
    # in place (the same pointer and strides): accepted, then stopped by the empty workspace
    (dict(glog=FAKE, gstr=[450, 45, 9], gdur=FAKE + 4096, gdstr=[450, 45, 9]), _native.TDT_ERR_WORKSPACE_TOO_SMALL),
    # separate buffers: accepted likewise
    (dict(glog=FAKE + 8192, gstr=[450, 45, 9], gdur=FAKE + 12288, gdstr=[450, 45, 9]),
     _native.TDT_ERR_WORKSPACE_TOO_SMALL),
    # token gradient shifted by one element into the logits: rejected
    (dict(glog=FAKE + 2, gstr=[450, 45, 9], gdur=FAKE + 12288, gdstr=[450, 45, 9]),
     _native.TDT_ERR_INVALID_ARGUMENT),
    # same pointer, other strides: not in place, overlaps: rejected
    (dict(glog=FAKE, gstr=[900, 90, 18], gdur=FAKE + 12288, gdstr=[450, 45, 9]), _native.TDT_ERR_INVALID_ARGUMENT),
    # duration gradient over the token logits: rejected
    (dict(glog=FAKE + 8192, gstr=[450, 45, 9], gdur=FAKE + 100, gdstr=[450, 45, 9]),
     _native.TDT_ERR_INVALID_ARGUMENT),
    # duration gradient just past the end of the duration logits: accepted
    (dict(glog=FAKE + 8192, gstr=[450, 45, 9], gdur=FAKE + 4096 + 2 * (450 + 9 * 45 + 4 * 9 + 3),
          gdstr=[450, 45, 9]), _native.TDT_ERR_WORKSPACE_TOO_SMALL),
    # ... and one element earlier: rejected
    (dict(glog=FAKE + 8192, gstr=[450, 45, 9], gdur=FAKE + 4096 + 2 * (450 + 9 * 45 + 4 * 9 + 2),
          gdstr=[450, 45, 9]), _native.TDT_ERR_INVALID_ARGUMENT),
])
def test_gradient_overlap_rules(over, code):
    assert _call(**over) == code


def _bwd(**over):
    args = dict(dtype=2, B=2, T_max=10, U1_max=5, V=9, logits=FAKE, lstr=[450, 45, 9], dur=FAKE + 4096,
                dstr=[450, 45, 9], D=3, labels=FAKE, lab_stride=4, tlen=FAKE, ulen=FAKE, durations=[0, 1, 2],
                blank=8, sigma=0.0, reduction=3, grad_loss=None, glog=FAKE + 8192, gstr=[450, 45, 9],
                gdur=FAKE + 12288, gdstr=[450, 45, 9], ws=FAKE, ws_bytes=0, stream=None)
    args.update(over)
    return _native.backward_raw(*args.values())


@pytest.mark.parametrize("over,code", [
    (dict(), _native.TDT_ERR_WORKSPACE_TOO_SMALL),
    (dict(grad_loss=FAKE), _native.TDT_ERR_WORKSPACE_TOO_SMALL),
    (dict(glog=None, gstr=None, gdur=None, gdstr=None), _native.TDT_ERR_INVALID_ARGUMENT),  # gradients required
    (dict(gdur=None), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(dtype=5), _native.TDT_ERR_UNSUPPORTED_DTYPE),
    (dict(reduction=7), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(blank=9), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(durations=[1, 1, 2]), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(glog=FAKE + 2), _native.TDT_ERR_INVALID_ARGUMENT),  # overlaps the logits
    (dict(glog=FAKE, gdur=FAKE + 4096), _native.TDT_ERR_WORKSPACE_TOO_SMALL),  # in place
    (dict(ws_bytes=1 << 40, ws=FAKE + 8), _native.TDT_ERR_BAD_STRIDE),
])
def test_backward_rejects_invalid_arguments(over, code):
    assert _bwd(**over) == code


def _noalloc(**over):
    args = dict(dtype=2, B=2, T_max=10, U1_max=5, V=9, logits=FAKE, lstr=[450, 45, 9], dur=FAKE + 4096,
                dstr=[450, 45, 9], D=3, labels=FAKE, lab_stride=4, tlen=FAKE, ulen=FAKE, durations=[0, 1, 2],
                blank=8, sigma=0.0, reduction=3, loss=FAKE, glog=None, gstr=None, gdur=None, gdstr=None,
                status=None, stream=None)
    args.update(over)
    return _native.fwd_bwd_noalloc_raw(*args.values())


def test_noalloc_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "tdt_loss.h")).read()
    m = re.search(r"#define TDT_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == _native.NOALLOC_SCRATCH_BYTES


# Every call below fails a host check before the library looks up its device array, so
# nothing reaches the device (the pointers are fake).
@pytest.mark.parametrize("over,code", [
    (dict(dtype=3), _native.TDT_ERR_UNSUPPORTED_DTYPE),
    (dict(reduction=9), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(logits=None), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(blank=9), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(durations=[0, 0, 1]), _native.TDT_ERR_INVALID_ARGUMENT),
    (dict(lab_stride=2), _native.TDT_ERR_BAD_STRIDE),
    (dict(glog=FAKE + 2, gstr=[450, 45, 9], gdur=FAKE + 12288, gdstr=[450, 45, 9]), _native.TDT_ERR_INVALID_ARGUMENT),
    # a workspace beyond the library's array
    (dict(B=64, T_max=1000, U1_max=500, lstr=[500 * 1000 * 12, 500 * 12, 12], dstr=[500 * 1000 * 12, 500 * 12, 12],
          lab_stride=499), _native.TDT_ERR_WORKSPACE_TOO_SMALL),
])
def test_noalloc_host_checks(over, code):
    assert _noalloc(**over) == code


def test_workspace_is_small_next_to_the_logits():
    """The workspace holds per-node records of the padded box only (no per-diagonal
    bounding box, one plain weight record per node): at most 10% of the logits on the
    ragged fp16 batch and 20% on the long-label bf16 batch."""
    import sys
    sys.path.insert(0, ROOT)
    from tdt_inputs import CONFIGS

    for cid, limit in ((3, 0.10), (4, 0.20)):
        c = CONFIGS[cid]
        T = c.get("Tmax", max(c.get("T", [0])))
        U1 = c.get("U1max", max(c.get("U", [0])) + 1)
        dt = {"f32": 0, "f16": 1, "bf16": 2}[c["dtype"]]
        ws = _native.workspace_size(dt, c["B"], T, U1, c["V"], c["durations"])
        logits = c["B"] * T * U1 * (c["V"] + len(c["durations"])) * (4 if dt == 0 else 2)
        assert ws <= limit * logits, (c["name"], ws, logits)
