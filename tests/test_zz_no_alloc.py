"""GPU test of the allocation-free entry point tdt_loss_fwd_bwd_noalloc (workspace in a
library-owned device array instead of a caller buffer).  It runs the kernels of
tdt_loss_fwd_bwd, so its loss, gradients and status must equal that entry point's bit for
bit; two calls in a row, the second on a smaller input, check that the array's leftover
contents from the first call do not leak into the second."""
import pytest
import torch

import tdt_transducer_loss_amd as tdt
from parity_util import say
from tdt_inputs import config_case, make_case
from tdt_transducer_loss_amd import _native

pytestmark = pytest.mark.gpu


def _noalloc(case):
    B, Tm, U1, V = case.tok.shape
    dt = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[case.joint.dtype]
    red = tdt.REDUCTIONS[case.reduction]
    loss = torch.full((B if red == 0 else 1,), float("nan"), dtype=torch.float32, device="cuda")
    g, gd = tdt.alloc_grads_like(case.tok, case.dur)
    g.fill_(float("nan"))
    gd.fill_(float("nan"))
    st = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    labels = case.labels.contiguous()
    say(f"[gpu] no-alloc entry point: {case.name} joint={tuple(case.joint.shape)} {case.joint.dtype}")
    rc = _native.fwd_bwd_noalloc_raw(dt, B, Tm, U1, V, case.tok.data_ptr(), list(case.tok.stride()[:3]),
                                     case.dur.data_ptr(), list(case.dur.stride()[:3]), case.D, labels.data_ptr(),
                                     labels.stride(0), case.logit_lengths.data_ptr(), case.label_lengths.data_ptr(),
                                     case.durations, case.blank, case.sigma, red, loss.data_ptr(), g.data_ptr(),
                                     list(g.stride()[:3]), gd.data_ptr(), list(gd.stride()[:3]), st.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return rc, loss, g, gd, st


def _with_workspace(case):
    st = torch.full((case.B,), -1, dtype=torch.int32, device="cuda")
    loss, g, gd = tdt.tdt_loss_fwd_bwd(case.tok, case.dur, case.labels, case.logit_lengths, case.label_lengths,
                                       case.durations, case.blank, case.sigma, case.reduction, utt_status=st)
    torch.cuda.synchronize()
    return loss.reshape(-1), g, gd, st


def test_noalloc_matches_workspace_entry_point_twice():
    big = config_case(2, device="cuda")  # B4 T200 U40 V8193 bf16, a 22 MB workspace
    small = make_case(3, [17, 9, 12], [5, 2, 7], 33, [0, 1, 2, 3], "f32", seed=80, sigma=0.1, reduction="none",
                      device="cuda")
    for case in (big, small):
        ws = tdt.workspace_size({torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[case.joint.dtype],
                                *case.tok.shape, case.durations)
        assert ws <= _native.NOALLOC_SCRATCH_BYTES
        rc, loss, g, gd, st = _noalloc(case)
        assert rc == _native.TDT_OK, _native.status_string(rc)
        ref = _with_workspace(case)
        assert torch.equal(loss, ref[0]), (loss, ref[0])
        assert torch.equal(g, ref[1]) and torch.equal(gd, ref[2])
        assert torch.equal(st, ref[3])


def test_noalloc_rejects_sizes_beyond_its_array():
    case = config_case(3, device="cuda")  # ragged B16 batch: its workspace exceeds the array
    dt = 1
    assert tdt.workspace_size(dt, *case.tok.shape, case.durations) > _native.NOALLOC_SCRATCH_BYTES
    rc, loss, g, gd, st = _noalloc(case)
    assert rc == _native.TDT_ERR_WORKSPACE_TOO_SMALL
    assert torch.isnan(loss).all() and torch.isnan(g).all() and (st == -1).all()  # nothing was launched
