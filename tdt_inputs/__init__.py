"""Seeded synthetic inputs for the TDT loss (shared by the GPU tests, the oracle tests
and the benchmark).

This module holds no part of the loss arithmetic: it only draws lengths, labels and
logits from a seeded torch generator and lays them out as a joint tensor
[B, Tmax, U1max, V + D] whose first V columns are token logits and whose last D
columns are duration logits (the layout of the joint output of a Parakeet-TDT model,
read in place as two slices, as the page "tdt-loss: add TDT loss kernel" describes
for ``logits[..., :V]``).

Draw order per case: lengths (ragged cases only) and labels from a seeded CPU generator
(so they, and the byte count of a ragged batch, are the same on every machine), then
logits from a generator on the target device seeded with seed + 1 (float32
``standard_normal * scale`` rounded to the storage dtype by torch's round-to-nearest-even
cast; padded nodes hold random values too).  The same tensor (copied to the host when
needed) feeds the GPU path and the oracle, so both sides see identical bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "f64": torch.float64}


@dataclass
class Case:
    name: str
    joint: torch.Tensor          # [B, Tmax, U1max, V + D (+ extra)]
    V: int
    D: int
    labels: torch.Tensor         # [B, U1max - 1] int64, -100 padded
    logit_lengths: torch.Tensor  # [B] int64
    label_lengths: torch.Tensor  # [B] int64
    durations: list
    blank: int
    sigma: float
    reduction: str
    meta: dict = field(default_factory=dict)

    @property
    def tok(self) -> torch.Tensor:
        return self.joint[..., : self.V]

    @property
    def dur(self) -> torch.Tensor:
        return self.joint[..., self.V: self.V + self.D]

    @property
    def B(self) -> int:
        return self.joint.shape[0]

    def to(self, device) -> "Case":
        return Case(self.name, self.joint.to(device), self.V, self.D, self.labels.to(device),
                    self.logit_lengths.to(device), self.label_lengths.to(device), list(self.durations),
                    self.blank, self.sigma, self.reduction, dict(self.meta))


# The five workloads.  Sizes, dtypes, distributions, sigma and reductions are those of
# the Parakeet-size benchmark on the pages (batch 4, 200 frames, 40 labels, vocab 8193)
# plus a tiny lattice, a ragged batch and a long-label stress case.
CONFIGS = {
    0: dict(name="tiny_f32", B=2, T=[12, 9], U=[4, 3], V=17, durations=[0, 1, 2, 3, 4], dtype="f32",
            scale=1.0, sigma=0.0, reduction="none"),
    1: dict(name="parakeet_f32", B=4, T=[200] * 4, U=[40] * 4, V=8193, durations=[0, 1, 2, 3, 4], dtype="f32",
            scale=2.0, sigma=0.0, reduction="mean_volume"),
    2: dict(name="parakeet_bf16", B=4, T=[200] * 4, U=[40] * 4, V=8193, durations=[0, 1, 2, 3, 4], dtype="bf16",
            scale=2.0, sigma=0.05, reduction="mean_batch"),
    3: dict(name="ragged_f16", B=16, Tmax=400, U1max=101, T_range=(100, 400), U_range=(10, 100), V=1025,
            durations=[0, 1, 2, 3, 4], dtype="f16", scale=1.5, sigma=0.0, reduction="mean"),
    4: dict(name="long_label_bf16", B=2, T=[1000] * 2, U=[1500] * 2, V=1025, durations=list(range(9)),
            dtype="bf16", scale=1.0, sigma=0.05, reduction="sum"),
}


def config_case(cfg: int, device="cpu", seed: int | None = None) -> Case:
    """Build workload ``cfg`` (0..4) on ``device`` from seed 1000 + cfg."""
    c = dict(CONFIGS[cfg])
    seed = 1000 + cfg if seed is None else seed
    if "T_range" in c:
        return make_case(c["B"], None, None, c["V"], c["durations"], c["dtype"], scale=c["scale"],
                         sigma=c["sigma"], reduction=c["reduction"], seed=seed, device=device,
                         Tmax=c["Tmax"], U1max=c["U1max"], T_range=c["T_range"], U_range=c["U_range"],
                         name=c["name"])
    return make_case(c["B"], c["T"], c["U"], c["V"], c["durations"], c["dtype"], scale=c["scale"],
                     sigma=c["sigma"], reduction=c["reduction"], seed=seed, device=device, name=c["name"])


def make_case(B, T, U, V, durations, dtype="f32", *, scale=1.0, sigma=0.0, reduction="none", seed=0,
              device="cpu", Tmax=None, U1max=None, T_range=None, U_range=None, blank=None, extra_cols=0,
              name="custom", label_high=None) -> Case:
    """Seeded case.  ``T``/``U`` are per-utterance lengths, or None with ``T_range``/``U_range``
    (inclusive integer-uniform draws, labels capped at 2 x frames).  ``blank`` defaults to
    V - 1; labels are uniform in [0, label_high) with label_high defaulting to the blank id
    when the blank is the last class.  ``extra_cols`` appends unused columns after the
    duration logits (a wider joint row)."""
    cgen = torch.Generator(device="cpu")
    cgen.manual_seed(int(seed))
    blank = V - 1 if blank is None else blank
    D = len(durations)
    if T is None:
        lo, hi = T_range
        T_t = torch.randint(lo, hi + 1, (B,), generator=cgen, dtype=torch.int64)
        ulo, uhi = U_range
        U_t = torch.randint(ulo, uhi + 1, (B,), generator=cgen, dtype=torch.int64)
        U_t = torch.minimum(U_t, 2 * T_t)
    else:
        T_t = torch.tensor(list(T), dtype=torch.int64)
        U_t = torch.tensor(list(U), dtype=torch.int64)
    Tmax = int(T_t.max().item()) if Tmax is None else Tmax
    U1max = int(U_t.max().item()) + 1 if U1max is None else U1max
    Lmax = max(U1max - 1, 1)
    high = (blank if blank == V - 1 else V) if label_high is None else label_high
    labels = torch.randint(0, high, (B, Lmax), generator=cgen, dtype=torch.int64)
    pos = torch.arange(Lmax)[None, :]
    labels = torch.where(pos < U_t[:, None], labels, torch.full_like(labels, -100))
    T_t, U_t, labels = T_t.to(device), U_t.to(device), labels.to(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 1)
    C = V + D + extra_cols
    joint = torch.empty((B, Tmax, U1max, C), dtype=_DT[dtype], device=device)
    for b in range(B):
        x = torch.randn((Tmax, U1max, C), generator=gen, device=device, dtype=torch.float32)
        if dtype == "f64":
            x = x.double()
        joint[b] = (x * scale).to(_DT[dtype])
        del x
    return Case(name, joint, V, D, labels, T_t, U_t, list(durations), blank, float(sigma), reduction,
                meta=dict(seed=int(seed), scale=scale, dtype=dtype))


def algorithmic_bytes(case: Case) -> int:
    """Bytes of the three streaming passes: two reads of every valid lattice row and one
    write of every row of the gradient, rows of V + D elements in the storage dtype."""
    elt = case.joint.element_size()
    row = (case.V + case.D) * elt
    Tl = case.logit_lengths.cpu()
    Ul = case.label_lengths.cpu()
    valid = int((Tl * (Ul + 1)).sum().item())
    B, Tmax, U1max = case.joint.shape[:3]
    return 2 * valid * row + B * Tmax * U1max * row
