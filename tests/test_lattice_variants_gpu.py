"""GPU parity of every lattice kernel variant against the float64 oracle.

The lattice launcher picks a kernel by the largest duration value (templates for
durations up to 4, 8 and 16; durations beyond 8 run the extended-range sweep only) and by
the padded label count U1_max = U + 1: one tile holding every frame with one label per
lane (U1_max <= 64), two to four such tiles swept at once by the waves of one work-group
and linked through LDS (U1_max <= 256), and beyond that columns of 64 labels over every
frame in work-groups of their own, linked through global memory (durations up to 8, when
all of them can be resident at once), else bands of 64-label x 48-frame tiles.  This matrix gives each (duration bound, label count) pair a small case whose
loss and every gradient element are compared with the oracle, plus a case per label count
whose logits (standard deviation 400) put the move weights far below 2^-300, which forces
the extended-range sweep.  Frames are few (24-40) so that the oracle and the GPU run in
well under a second per case; durations include 0 so that utterances with more labels
than frames have alignments.  A linked case with 600 frames runs the LDS rings (256
slots) through several turns.
"""
import pytest

from parity_util import check_grads, check_loss, gpu_run, oracle_run
from tdt_inputs import make_case

pytestmark = pytest.mark.gpu

# duration sets by their largest value (the kernel template bound)
DURATIONS = {4: [0, 1, 2, 3, 4], 8: [0, 1, 3, 8], 16: [0, 1, 2, 7, 16]}
# label counts: one tile (51), two and four linked tiles (101, 221), then 8 to 79 bands
# of tiles
LABELS = [50, 100, 220, 500, 1200, 2500, 5000]


def _case(dm, U, dtype, scale=1.0, seed=0):
    T = 24 + (U % 17)
    return make_case(1, [T], [U], 13, DURATIONS[dm], dtype, scale=scale, sigma=0.05, reduction="sum",
                     seed=seed, name=f"dm{dm}_U{U}_{dtype}_s{scale:g}")


def _parity(case):
    loss, gt, gd, st = gpu_run(case)
    orc = oracle_run(case.to("cpu"))
    check_loss(loss, orc, case.reduction, case.joint.dtype)
    check_grads(gt, gd, orc, case.joint.dtype)
    assert int(st.cpu()[0]) == int(orc["status"][0]) == 0


@pytest.mark.parametrize("U", LABELS)
@pytest.mark.parametrize("dm", sorted(DURATIONS))
def test_lattice_variant(dm, U):
    dtype = "f32" if (LABELS.index(U) + dm) % 2 == 0 else "bf16"
    _parity(_case(dm, U, dtype, seed=100 + U + dm).to("cuda"))


@pytest.mark.parametrize("U", LABELS)
def test_lattice_variant_extended_range(U):
    _parity(_case(4 if LABELS.index(U) % 2 == 0 else 8, U, "f32", scale=400.0, seed=200 + U).to("cuda"))


def test_more_than_8192_labels():
    """9000 labels in 12 frames (label moves of duration 0): 141 bands of 64-label tiles."""
    case = make_case(2, [12, 9], [9000, 8100], 9, [0, 1, 2], "f32", seed=300, sigma=0.02, reduction="mean")
    _parity(case.to("cuda"))


@pytest.mark.parametrize("dm", [4, 8])
def test_linked_tiles_long_frames(dm):
    """Three linked 64-label tiles over 600 frames: each link's ring turns over twice."""
    case = make_case(2, [600, 410], [180, 150], 11, DURATIONS[dm], "f32", seed=310 + dm, sigma=0.05,
                     reduction="mean")
    _parity(case.to("cuda"))


@pytest.mark.parametrize("dm", [4, 8])
@pytest.mark.parametrize("T,U", [(200, 300), (150, 400)])
def test_long_labels_many_frames(dm, T, U):
    """Linked columns over 150-200 frames (a float32 case, so that a lost move shows far
    above rounding)."""
    case = make_case(1, [T], [U], 9, list(range(dm + 1)), "f32", seed=7 + T + dm, sigma=0.05, reduction="sum",
                     name=f"bands_dm{dm}_T{T}_U{U}")
    _parity(case.to("cuda"))


def test_long_labels_many_frames_extended_range():
    """The same geometry with weights far below 2^-300 (the extended-range redo)."""
    case = make_case(1, [150], [300], 9, [0, 1, 2, 3, 4], "f32", seed=401, scale=400.0, sigma=0.05,
                     reduction="sum", name="bands_extended")
    _parity(case.to("cuda"))


# ragged batches over every lattice layout, with duration sets that have gaps, lack 0 or go
# beyond 8 (B, T per utterance, U per utterance, T_max, U1_max, durations); the seed
# follows the name
SHAPES = {
    "linked_gaps_ragged": (3, [255, 115, 211], [101, 57, 60], 255, 102, [0, 2, 5, 7]),
    "columns_no_zero_dm8": (3, [206, 163, 92], [396, 326, 32], 206, 397, [1, 3, 8]),
    "bands_dm16": (2, [246, 237], [298, 60], 246, 299, [0, 1, 9, 13]),
    "columns_short_frames": (3, [112, 91, 77], [323, 299, 232], 112, 324, [0, 1, 2, 3, 4]),
    "linked_ragged_dm8": (3, [224, 149, 104], [120, 42, 114], 224, 121, [0, 1, 2, 3, 4, 5, 6, 7, 8]),
    "linked_no_zero_dm16": (1, [253], [244], 253, 245, [1, 16]),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_lattice_shapes(name):
    B, Ts, Us, Tmax, U1max, durs = SHAPES[name]
    case = make_case(B, Ts, Us, 7, durs, "f32", seed=1000 + len(name), sigma=0.05, reduction="none", Tmax=Tmax,
                     U1max=U1max, name=name)
    loss, gt, gd, st = gpu_run(case.to("cuda"))
    orc = oracle_run(case.to("cpu"))
    check_loss(loss, orc, case.reduction, case.joint.dtype)
    check_grads(gt, gd, orc, case.joint.dtype)


def test_columns_data_errors():
    """Linked columns (301 padded labels) with an infeasible utterance, a label out of range,
    a logit length beyond T_max and zero frames: statuses, losses and zero gradients as the
    oracle has them (the first column finishes utterances with bad lengths)."""
    case = make_case(5, [20, 19, 20, 20, 20], [290, 200, 250, 120, 260], 9, [0, 2, 4], "f32", seed=71,
                     sigma=0.05, reduction="none", Tmax=20, U1max=301, name="columns_errors")
    case.labels[2, 100] = 9
    case.logit_lengths[3] = 21
    case.logit_lengths[4] = 0
    loss, gt, gd, st = gpu_run(case.to("cuda"))
    orc = oracle_run(case.to("cpu"))
    check_loss(loss, orc, "none", case.joint.dtype)
    check_grads(gt, gd, orc, case.joint.dtype)
    s = st.cpu().numpy()
    assert list(s) == list(orc["status"])
    assert s[0] == 0 and s[1] != 0 and s[2] != 0 and s[3] != 0 and s[4] != 0


@pytest.mark.parametrize("dm", [4, 8])
def test_bands_many_frame_tiles(dm):
    """80 utterances of 150-200 frames and 250-350 labels: more column work-groups than the
    linked-column path takes, so bands of 64-label x 48-frame tiles run, each utterance
    several frame tiles high; each tile's top-right node has a label move of the longest
    duration into the tile above and to the right."""
    import random

    rnd = random.Random(10 + dm)
    B = 80
    Ts = [rnd.randint(150, 200) for _ in range(B)]
    Us = [rnd.randint(250, 350) for _ in range(B)]
    case = make_case(B, Ts, Us, 5, list(range(dm + 1)), "f32", seed=80 + dm, sigma=0.05, reduction="sum",
                     Tmax=200, U1max=351, name=f"bands_frames_dm{dm}")
    loss, gt, gd, st = gpu_run(case.to("cuda"))
    orc = oracle_run(case.to("cpu"))
    check_loss(loss, orc, case.reduction, case.joint.dtype)
    check_grads(gt, gd, orc, case.joint.dtype)
    assert list(st.cpu().numpy()) == list(orc["status"])


def test_bands_extended_range():
    """Bands (80 utterances of 250-300 labels) with weights far below 2^-300: the
    extended-range sweep in every tile."""
    import random

    rnd = random.Random(3)
    B = 80
    Ts = [rnd.randint(3, 12) for _ in range(B)]
    Us = [rnd.randint(250, 300) for _ in range(B)]
    case = make_case(B, Ts, Us, 5, [0, 1, 2, 3, 4], "f32", seed=90, scale=400.0, sigma=0.05, reduction="mean",
                     Tmax=12, U1max=301, name="bands_extended")
    loss, gt, gd, st = gpu_run(case.to("cuda"))
    orc = oracle_run(case.to("cpu"))
    check_loss(loss, orc, case.reduction, case.joint.dtype)
    check_grads(gt, gd, orc, case.joint.dtype)
    assert list(st.cpu().numpy()) == list(orc["status"])


@pytest.mark.parametrize("dm,B", [(4, 80), (8, 60)])
def test_many_utterances_long_labels(dm, B):
    """Long label sequences in batches too large for every column work-group to be resident
    at once: 80 x 5 columns x 2 directions exceed the column limit (bands of tiles), and
    with durations up to 8 the 600 column work-groups are more than the GPU holds at the
    register count of that sweep (the occupancy check sends them to bands)."""
    import random

    rnd = random.Random(dm)
    Ts = [rnd.randint(3, 12) for _ in range(B)]
    Us = [rnd.randint(200, 300) for _ in range(B)]
    case = make_case(B, Ts, Us, 5, DURATIONS[dm], "f32", seed=72 + dm, sigma=0.05, reduction="mean", Tmax=12,
                     U1max=301, name=f"many_long_dm{dm}")
    loss, gt, gd, st = gpu_run(case.to("cuda"))
    orc = oracle_run(case.to("cpu"))
    check_loss(loss, orc, case.reduction, case.joint.dtype)
    check_grads(gt, gd, orc, case.joint.dtype)
    assert list(st.cpu().numpy()) == list(orc["status"])


@pytest.mark.parametrize("dm", [4, 8])
@pytest.mark.parametrize("U", [100, 220, 500, 1200])
def test_link_waits_give_up(dm, U, monkeypatch):
    """Every wait between linked waves or column work-groups bounded to one poll (set from
    the host through TDT_LINK_SPIN_LIMIT): links break, the plain sweeps' results are
    dropped, and the extended-range redo (wave 0 of the work-group, or the last column of
    the utterance to finish) must still give the oracle's loss and gradients."""
    monkeypatch.setenv("TDT_LINK_SPIN_LIMIT", "1")
    _parity(_case(dm, U, "f32", seed=500 + U + dm).to("cuda"))


@pytest.mark.parametrize("U", [30, 150])
def test_sixteen_durations(U):
    """The most durations a call takes (16, values up to 16): the short-row gradient pass
    gives each of its 16 lanes per node one duration's two moves, and the node weights
    write every slot pair of the duration bound 16; one tile and two linked tiles."""
    durations = list(range(15)) + [16]
    case = make_case(2, [40, 33], [U, U - 7], 13, durations, "bf16" if U > 100 else "f32", seed=400 + U,
                     sigma=0.05, reduction="mean", name=f"d16_U{U}")
    loss, gt, gd, st = gpu_run(case.to("cuda"))
    orc = oracle_run(case)
    check_loss(loss, orc, case.reduction, case.joint.dtype)
    check_grads(gt, gd, orc, case.joint.dtype)
    assert st.cpu().tolist() == orc["status"].tolist()
