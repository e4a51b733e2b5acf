"""The fused call captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library launches kernels only (no memset, no allocation, no host synchronisation, no
host-side state that changes between calls), so a captured call replays as an eager call
on the same buffers.  Each replay follows eager work on the GPU (new logits, and for the
ragged batch new lengths, copied into the captured input buffers, then a device
synchronisation), and its loss and gradients must equal, bit for bit, those of an eager
call on the same inputs: the short-row path (the gradient pass computes the node
coefficients and the lattice launch zeroes the padding rows) on the ragged fp16 batch, and
the long-row path (a coefficient kernel) on a bf16 batch with an 8193-token vocabulary.
"""
import pytest
import torch

import tdt_transducer_loss_amd as tdt
from parity_util import say
from tdt_inputs import config_case, make_case

pytestmark = pytest.mark.gpu


def _call(case, ws):
    return tdt.tdt_loss_fwd_bwd(case.tok, case.dur, case.labels, case.logit_lengths, case.label_lengths,
                                case.durations, case.blank, case.sigma, case.reduction, workspace=ws)


def _cases():
    return {
        "ragged_f16": lambda: config_case(3, device="cuda"),
        "long_rows_bf16": lambda: make_case(3, [40, 31, 22], [9, 12, 5], 8193, [0, 1, 2, 3, 4], "bf16", scale=2.0,
                                            sigma=0.05, reduction="mean_batch", seed=71, device="cuda",
                                            name="long_rows_bf16"),
    }


@pytest.mark.parametrize("name", ["ragged_f16", "long_rows_bf16"])
def test_graph_replays_match_eager(name):
    case = _cases()[name]()
    B, Tm, U1, V = case.tok.shape
    dt = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[case.joint.dtype]
    nbytes = tdt.workspace_size(dt, B, Tm, U1, V, case.durations)
    ws_graph = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws_eager = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        _call(case, ws_graph)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say(f"[gpu] graph capture {name}")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loss_g, gt_g, gd_g = _call(case, ws_graph)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(5)
    for r in range(3):
        # eager work between the replays: new logits (and, for the ragged batch, lengths)
        # copied into the captured buffers
        fresh = (torch.randn(case.joint.shape, generator=gen) * 2.0).to(case.joint.dtype)
        case.joint.copy_(fresh.to("cuda"))
        if name == "ragged_f16" and r == 2:
            case.logit_lengths.copy_(torch.clamp(case.logit_lengths - 7, min=1))
            case.label_lengths.copy_(torch.clamp(case.label_lengths - 3, min=0))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (loss_g.clone(), gt_g.clone(), gd_g.clone())
        loss_e, gt_e, gd_e = _call(case, ws_eager)
        torch.cuda.synchronize()
        say(f"[gpu] replay {r}: loss {got[0].flatten()[:2].tolist()} eager {loss_e.flatten()[:2].tolist()}")
        assert torch.isfinite(got[0]).all().item()
        assert torch.equal(got[0], loss_e)
        assert torch.equal(got[1], gt_e)
        assert torch.equal(got[2], gd_e)
