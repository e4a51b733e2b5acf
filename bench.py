"""Benchmark of the TDT loss forward+backward on one MI355X.

One step = one call of the C ABI (row partials, node weights, lattice, coefficients,
gradient pass, loss reduction, in order on one stream) over one batch of the
Parakeet-size workload: B=4, T=200, U=40,
V=8193 (blank 8192), durations {0..4}, bf16 logits read in place as the slice
[..., :8193] of a [4, 200, 41, 8198] joint output, sigma 0.05, reduction mean_batch.
Inputs are seeded synthetic data resident in HBM; several input/gradient buffer sets are
rotated so that a step never finds the previous step's data in the 256 MB last-level
cache.

Prints one JSON line: value = algorithmic GB/s of the whole step (two reads of every
valid lattice row and one write of every gradient row, V + D elements each), the
roofline of the dominant kernel (the gradient pass, timed with HIP events the library
records on the stream right before and after its launch in every EVERY-th timed step:
an event between two kernels stalls the stream for a few microseconds, so the other
steps carry none), a per-kernel breakdown from a second loop with events between all
kernels, and the float64 CPU oracle timed on the host on the same workload.  A second
part times every workload of tdt_inputs.CONFIGS the same way (host clock over
back-to-back calls) and reports, per workload, ms per step, algorithmic GB/s, the
fraction of the 8 TB/s peak, a per-kernel breakdown and the oracle's host time
(``configs``; ``--headline-only`` skips it).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "TDT loss fwd+bwd ms and achieved HBM GB/s, B4 T200 U40 V8193 bf16"


class HipEvents:
    """Timing events of the HIP runtime torch has loaded, created with
    hipEventDisableSystemFence: recording them between kernels costs no cache write-back,
    so they time the kernels without slowing the step down."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        self.ct = ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.lib = ctypes.CDLL(path)
        self.lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.events = []

    def create(self) -> int:
        ev = self.ct.c_void_p()
        rc = self.lib.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.events.append(ev.value)
        return ev.value

    def record(self, ev: int, stream: int) -> None:
        rc = self.lib.hipEventRecord(self.ct.c_void_p(ev), self.ct.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed(self, a: int, b: int) -> float:
        ms = self.ct.c_float()
        rc = self.lib.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(a), self.ct.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        for ev in getattr(self, "events", []):
            self.lib.hipEventDestroy(self.ct.c_void_p(ev))


def measured_traffic(path: str):
    """HBM bytes per gradient-kernel launch from a committed counter summary, or None when
    the summary is missing or was taken on other kernel sources than the current ones."""
    import hashlib

    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if not line.startswith("#") and "=" in line:
                k, v = line.split("=", 1)
                fields[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for name in fields["hashed_files"].split():
            with open(os.path.join(ROOT, name), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != fields["kernel_source_sha256"]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_time(case, runs: int):
    """Wall time of the float64 oracle (loss and the whole gradient) on the host, in ms:
    the median of ``runs`` runs of oracle.run, or, when the full float64 gradient would
    not fit comfortably in host memory, one oracle session that computes every gradient
    row a range at a time (the same arithmetic, rows discarded after each range)."""
    import oracle

    c = case.to("cpu")
    B, Tm, U1, V = c.tok.shape
    full_bytes = B * Tm * U1 * (V + c.D) * 8
    times = []
    if full_bytes <= (8 << 30):
        for _ in range(runs):
            t = time.perf_counter()
            oracle.run(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank, c.sigma,
                       c.reduction)
            times.append(time.perf_counter() - t)
        how = f"median of {runs} runs of the full oracle (loss and gradient)"
    else:
        t = time.perf_counter()
        with oracle.Session(c.tok, c.dur, c.labels, c.logit_lengths, c.label_lengths, c.durations, c.blank,
                            c.sigma, c.reduction) as s:
            chunk = 1 << 16
            for first in range(0, s.nodes, chunk):
                s.rows(first, min(chunk, s.nodes - first))
        times.append(time.perf_counter() - t)
        how = "one oracle session: loss, lattice and every gradient row, computed a range of rows at a time"
    del c
    return sorted(times)[len(times) // 2] * 1e3, how, oracle.max_threads()


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--event-every", type=int, default=5,
                    help="record the gradient-kernel events in every N-th timed step")
    ap.add_argument("--config", type=int, default=2, help="workload id in tdt_inputs.CONFIGS")
    ap.add_argument("--rotate", type=int, default=3, help="input/gradient buffer sets cycled over the steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline workload (no per-workload table)")
    ap.add_argument("--traffic", type=str,
                    default=os.path.join(ROOT, "profiles", "k_grad_parakeet_bf16_hbm_bytes.txt"),
                    help="rocprofv3 counter summary holding the measured HBM bytes per gradient-kernel launch")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (calibrates the HBM byte "
                         "counters of rocprofv3 --pmc) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the loss shards by utterance with no exchange but a scalar all-reduce, which is not implemented.",
              file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)
        return 0

    import tdt_transducer_loss_amd as tdt
    from tdt_transducer_loss_amd import _native
    from tdt_inputs import CONFIGS, algorithmic_bytes, config_case

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hip = HipEvents()
    stream = torch.cuda.current_stream(dev)

    class Runner:
        """One workload resident in HBM: ``rotate`` input/gradient buffer sets (so that a
        step never finds the previous step's data in the 256 MB last-level cache), one
        workspace, and the raw C-ABI call of one step."""

        def __init__(self, cfg, rotate):
            self.case = case = config_case(cfg, device=dev)
            self.B, self.Tm, self.U1, _ = case.joint.shape
            self.V, self.D = case.V, case.D
            self.dtype_code = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}[case.joint.dtype]
            self.red = tdt.REDUCTIONS[case.reduction]
            self.sets = []
            for r in range(max(1, rotate)):
                joint = case.joint if r == 0 else case.joint.clone()
                tok, dur = joint[..., :self.V], joint[..., self.V:self.V + self.D]
                g, gd = tdt.alloc_grads_like(tok, dur)
                self.sets.append((joint, tok, dur, g, gd))
            self.loss = torch.empty(self.B if self.red == 0 else 1, dtype=torch.float32, device=dev)
            self.ws_bytes = tdt.workspace_size(self.dtype_code, self.B, self.Tm, self.U1, self.V, case.durations)
            self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev)
            self.labels = case.labels.contiguous()
            self.tl, self.ul = case.logit_lengths.contiguous(), case.label_lengths.contiguous()

        def step(self, i, events=None):
            _, tok, dur, g, gd = self.sets[i % len(self.sets)]
            c = self.case
            rc = _native.fwd_bwd_raw(
                self.dtype_code, self.B, self.Tm, self.U1, self.V, tok.data_ptr(), list(tok.stride()[:3]),
                dur.data_ptr(), list(dur.stride()[:3]), self.D, self.labels.data_ptr(), self.labels.stride(0),
                self.tl.data_ptr(), self.ul.data_ptr(), c.durations, c.blank, c.sigma, self.red,
                self.loss.data_ptr(), g.data_ptr(), list(g.stride()[:3]), gd.data_ptr(), list(gd.stride()[:3]),
                None, self.ws.data_ptr(), self.ws_bytes, stream.cuda_stream, events=events)
            if rc != 0:
                raise RuntimeError(f"tdt_loss_fwd_bwd: {_native.status_string(rc)}")

        def timed(self, steps, warmup):
            """Host-clock ms per step over ``steps`` back-to-back calls after ``warmup``."""
            for i in range(warmup):
                self.step(i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                self.step(i)
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e3 / steps

        def breakdown(self, steps):
            """Per-kernel ms from a loop with events between all kernels (diagnostic)."""
            names = ["row_partials", "node_weights", "lattice", "coef", "grad", "reduce"]
            evs = [[hip.create() for _ in range(7)] for _ in range(steps)]
            for i in range(steps):
                self.step(i, evs[i])
            torch.cuda.synchronize()
            out = {n: 0.0 for n in names}
            for row in evs:
                for j, n in enumerate(names):
                    out[n] += hip.elapsed(row[j], row[j + 1]) / steps
            return out

        def free(self):
            self.sets = self.case = self.ws = None
            torch.cuda.empty_cache()

    # ---- headline workload: the timed region with live gradient-kernel events ----
    run = Runner(args.config, args.rotate)
    case, cfg = run.case, CONFIGS[args.config]
    B, Tm, U1, V, D = run.B, run.Tm, run.U1, run.V, run.D
    elt = case.joint.element_size()
    for i in range(args.warmup):
        run.step(i)
    torch.cuda.synchronize()

    # Timed region: K steps.  In every EVERY-th step the library records events[2]/[3]
    # right around the gradient kernel (events[0]/[1] left out); two more events bracket
    # the whole region.  The step time is the host clock over the region.
    K = args.steps
    every = max(1, args.event_every)
    sampled = [i for i in range(K) if i % every == 0]
    gevs = {i: [None, None, hip.create(), hip.create()] for i in sampled}
    region = [hip.create(), hip.create()]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(region[0], stream.cuda_stream)
    for i in range(K):
        run.step(i, gevs.get(i))
    hip.record(region[1], stream.cuda_stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    grad_ms = sum(hip.elapsed(e[2], e[3]) for e in gevs.values()) / len(gevs)  # average gradient-kernel launch
    event_ms = hip.elapsed(region[0], region[1]) / K
    phase_ms = run.breakdown(K)
    serial_ms = sum(phase_ms.values())

    alg = algorithmic_bytes(case)
    value = alg / (ms_per_step * 1e-3) / 1e9
    # dominant kernel: the gradient pass reads every valid row once and writes every row
    # once, in one launch per step
    row_bytes = (V + D) * elt
    valid = int((case.logit_lengths.cpu() * (case.label_lengths.cpu() + 1)).sum())
    grad_bytes = valid * row_bytes + B * Tm * U1 * row_bytes
    achieved = grad_bytes / (grad_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.traffic) if cfg["name"] == "parakeet_bf16" else None
    run.free()

    # ---- every workload: ms per step, algorithmic GB/s, oracle time ----
    configs = {}
    cpu = None
    ids = [args.config] if args.headline_only else sorted(CONFIGS)
    for cid in ids:
        c = CONFIGS[cid]
        r = Runner(cid, args.rotate)
        long_run = r.B * r.Tm * r.U1 * (r.V + r.D) * r.case.joint.element_size() > (4 << 30)
        steps = max(2, min(K, 5)) if long_run else max(K, 20)
        ms = ms_per_step if cid == args.config else r.timed(steps, 2 if long_run else max(args.warmup, 3))
        a = algorithmic_bytes(r.case)
        entry = {"ms_per_step": round(ms, 4), "gbs": round(a / (ms * 1e-3) / 1e9, 1),
                 "frac_of_peak": round(a / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "algorithmic_bytes": a,
                 "steps": K if cid == args.config else steps,
                 "kernel_ms": {k: round(v, 4) for k, v in (phase_ms if cid == args.config
                                                              else r.breakdown(min(steps, 5))).items()},
                 "shape": f"B{r.B} Tmax{r.Tm} U1max{r.U1} V{r.V} D{r.D} {c['dtype']} sigma {c['sigma']} "
                          f"{c['reduction']}"}
        if not args.no_cpu_baseline:
            o_ms, how, threads = oracle_time(r.case, 1 if long_run else 3)
            entry["oracle_ms"] = round(o_ms, 1)
            entry["oracle_runs"] = how
            if cid == args.config:
                cpu = {"value": round(alg / (o_ms * 1e-3) / 1e9, 4), "unit": "GB/s", "ms": round(o_ms, 1),
                       "cores": threads, "cpu_model": cpu_model(), "kind": "oracle",
                       "sample": f"the full workload (B={B}), {how}, float64, OpenMP"}
        configs[c["name"]] = entry
        r.free()
        print(f"# {c['name']}: {entry['ms_per_step']} ms/step {entry['gbs']} GB/s "
              f"oracle {entry.get('oracle_ms')} ms", file=sys.stderr, flush=True)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "f32", 1: "f16", 2: "bf16"}[run.dtype_code],
        "data": "synthetic",
        "config": {"workload": f"{cfg['name']}: B{B} T{Tm} U{U1 - 1} V{V} D{D} {case.joint.dtype} joint "
                               f"[{B},{Tm},{U1},{case.joint.shape[3]}] read as slices, sigma {case.sigma}, "
                               f"{case.reduction}",
                   "global_batch": B, "seq_len": Tm, "labels": U1 - 1, "vocab": V,
                   "algorithmic_bytes": alg, "buffer_sets": args.rotate},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "k_grad (gradient pass)",
                     "kernel_ms": round(grad_ms, 4), "launches_per_step": 1, "bytes_per_launch": int(grad_bytes),
                     "timed_launches": len(gevs)},
        "event_ms_per_step": round(event_ms, 4),
        "kernel_ms": {k: round(v, 4) for k, v in phase_ms.items()},
        "kernel_sum_ms": round(serial_ms, 4),
        "frac_of_peak_whole_step": round(value / PEAK_HBM_GBS, 4),
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
