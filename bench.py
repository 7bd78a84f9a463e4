"""Benchmark of the replay decode path on one MI355X.

Headline: one decode step (``replay_step``) of a Mamba-2 layer whose float32
state is 4 MiB per sequence (128 heads, P = 64, N = 128, 8 B/C groups), batch
256, window L = 16, with its inputs already resident in HBM.  K steps are timed
(rounded up to whole windows of L steps, so folds are timed in proportion; the
count actually timed is reported as steps_timed).

Printed: one JSON line with the headline (microseconds per step), the roofline
of the step kernel (algorithmic bytes per launch over its measured average
launch time), the CPU oracle timed on a bounded sample, and an ``extra`` block
with the in-run baselines and the other layer measurements.

  python bench.py [--gpus 1] [--steps 256] [--warmup 32] [--no-extra] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
_CSRC = "hybrid_model_ssm_replay_amd/csrc/"
# Sources each kernel family is built from: a stored counter summary is used only
# while the hash of these files matches the one it records.
KERNEL_SOURCES = {"m2": [_CSRC + f for f in ("mamba2.hip", "state_io.h", "codecs.h", "common.h", "internal.h")],
                  "gdn": [_CSRC + f for f in ("gdn.hip", "state_io.h", "codecs.h", "common.h", "internal.h")]}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash(family: str) -> str:
    """Hash of a kernel family's sources with comments and blank space removed,
    so that a counter summary stays matched across comment-only edits."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        src = open(os.path.join(ROOT, f), encoding="utf-8").read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def stored_traffic(name: str, family: str):
    """Per-launch HBM bytes from a committed counter summary, if it matches the current kernel source."""
    path = os.path.join(PROFILE_DIR, name)
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m or not t or m.group(1) != kernel_source_hash(family):
        return None
    return float(t.group(1))


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, n):
        t = self.torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        t.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n  # microseconds per call


def dev_records(torch, ins, n, bf16=False, rec_fn=None):
    """n device records; with bf16 the vector fields are bfloat16 tensors; rec_fn
    (optional) edits each host record first."""
    from synth import VECTOR_FIELDS
    cast = (lambda k, t: t.to(torch.bfloat16) if bf16 and k in VECTOR_FIELDS else t)  # noqa: E731
    edit = rec_fn or (lambda r: r)  # noqa: E731
    return [{k: cast(k, torch.from_numpy(v).cuda()) for k, v in edit(ins.record()).items()} for _ in range(n)]


def _bf16(flags):
    from hybrid_model_ssm_replay_amd.binding import FLAG_BF16_RECORDS
    return bool(flags & FLAG_BF16_RECORDS)


def bench_replay(torch, shape, seed, steps, warmup, pool=32, flags=0, rec_fn=None):
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    from synth import InputStream
    ins = InputStream(shape, seed, bf16_vectors=_bf16(flags))
    recs = dev_records(torch, ins, pool, _bf16(flags), rec_fn)
    kw = dict(A=ins.params["A"], D=ins.params["D"]) if shape.kind == "mamba2" else {}
    lay = ReplayLayer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                      groups=shape.groups, flags=flags, **kw)
    y = torch.empty((shape.batch, shape.heads, shape.head_dim), device="cuda")
    tm = Timer(torch)
    tm.run(lambda i: lay.step(recs[i % pool], y), warmup)
    us = tm.run(lambda i: lay.step(recs[(warmup + i) % pool], y), steps)
    if lay.status != 0:
        raise RuntimeError(f"device status {lay.status:#x}")
    return us


def bench_replay_staggered(torch, shape, seed, steps, warmup, pool=32):
    """The replay step with the sequences' windows out of phase, as in serving:
    one verify of L - 1 drafts whose accepted counts are b mod L moves sequence b
    to window phase b mod L, so each step folds 1/L of the sequences instead of
    all of them every L-th step.  Same layer, same bytes per step on average."""
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    from synth import InputStream
    L = shape.window
    ins = InputStream(shape, seed)
    recs = dev_records(torch, ins, pool)
    kw = dict(A=ins.params["A"], D=ins.params["D"]) if shape.kind == "mamba2" else {}
    lay = ReplayLayer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, L,
                      groups=shape.groups, max_draft=L - 1, **kw)
    d = {k: torch.from_numpy(v).cuda() for k, v in ins.drafts(L - 1).items()}
    lay.verify(d)
    lay.commit(torch.arange(shape.batch, dtype=torch.int32, device="cuda") % L)
    y = torch.empty((shape.batch, shape.heads, shape.head_dim), device="cuda")
    tm = Timer(torch)
    tm.run(lambda i: lay.step(recs[i % pool], y), warmup)
    us = tm.run(lambda i: lay.step(recs[(warmup + i) % pool], y), steps)
    if lay.status != 0:
        raise RuntimeError(f"device status {lay.status:#x}")
    return us


def step_distribution(torch, shape, seed, windows=8, pool=32):
    """Per-step times of the replay step (an event pair around every step) over
    `windows` whole windows after one warm-up window: p50 and p99 over all
    steps, and the mean of the fold steps (window position 0) and of the others."""
    import statistics

    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    from synth import InputStream
    L = shape.window
    ins = InputStream(shape, seed)
    recs = dev_records(torch, ins, pool)
    kw = dict(A=ins.params["A"], D=ins.params["D"]) if shape.kind == "mamba2" else {}
    lay = ReplayLayer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, L,
                      groups=shape.groups, **kw)
    y = torch.empty((shape.batch, shape.heads, shape.head_dim), device="cuda")
    for i in range(L):
        lay.step(recs[i % pool], y)
    n = windows * L
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n):
        lay.step(recs[(L + i) % pool], y)
        ev[i + 1].record()
    torch.cuda.synchronize()
    d = [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n)]
    sorted_d = sorted(d)
    fold = [x for i, x in enumerate(d) if i % L == 0]   # the first step of each window folds the previous one
    rest = [x for i, x in enumerate(d) if i % L != 0]
    return {"p50_us": statistics.median(d), "p99_us": sorted_d[min(n - 1, int(0.99 * n))],
            "fold_step_mean_us": statistics.mean(fold), "non_fold_step_mean_us": statistics.mean(rest),
            "steps": n}


def bench_conv(torch, shape, seed, steps, warmup, pool=32, flags=0):
    from hybrid_model_ssm_replay_amd.layer import ConvLayer
    from synth import InputStream
    ins = InputStream(shape, seed, bf16_vectors=_bf16(flags))
    recs = dev_records(torch, ins, pool, _bf16(flags))
    kw = dict(A=ins.params["A"], D=ins.params["D"]) if shape.kind == "mamba2" else {}
    conv = ConvLayer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, groups=shape.groups,
                     flags=flags, **kw)
    y = torch.empty((shape.batch, shape.heads, shape.head_dim), device="cuda")
    tm = Timer(torch)
    tm.run(lambda i: conv.step(recs[i % pool], y), warmup)
    return tm.run(lambda i: conv.step(recs[(warmup + i) % pool], y), steps)


def bench_verify(torch, shape, T, seed, reps=16, snapshot=True):
    """Replay verify + commit vs snapshot verify + commit (None without `snapshot`),
    batch as in shape (accepted counts uniform in 0..T)."""
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer, SnapshotLayer
    from synth import InputStream
    ins = InputStream(shape, seed)
    drafts = [{k: torch.from_numpy(v).cuda() for k, v in ins.drafts(T).items()} for _ in range(4)]
    accs = [torch.from_numpy(ins.accepted(T)).cuda() for _ in range(4)]
    kw = dict(A=ins.params["A"], D=ins.params["D"]) if shape.kind == "mamba2" else {}
    lay = ReplayLayer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                      groups=shape.groups, max_draft=T, **kw)
    y = torch.empty((shape.batch, T, shape.heads, shape.head_dim), device="cuda")
    tm = Timer(torch)

    def rv(i):
        lay.verify(drafts[i % 4], y)
        lay.commit(accs[i % 4])

    tm.run(rv, 8)
    us_replay = tm.run(rv, reps)
    del lay
    if not snapshot:
        torch.cuda.empty_cache()
        return us_replay, None
    snap = SnapshotLayer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, T,
                         groups=shape.groups, **kw)

    def sv(i):
        snap.verify(drafts[i % 4], y)
        snap.commit(accs[i % 4])

    tm.run(sv, 4)
    us_snap = tm.run(sv, reps)
    del snap
    torch.cuda.empty_cache()
    return us_replay, us_snap


def bench_probe(torch, nbytes=2 << 30):
    from hybrid_model_ssm_replay_amd import binding as B
    src = torch.zeros(nbytes // 4, device="cuda")
    dst = torch.zeros(nbytes // 8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    tm = Timer(torch)
    tm.run(lambda i: B.replay_hbm_probe(src.data_ptr(), dst.data_ptr(), nbytes, 0, st), 3)
    us_read = tm.run(lambda i: B.replay_hbm_probe(src.data_ptr(), dst.data_ptr(), nbytes, 0, st), 10)
    half = nbytes // 2
    tm.run(lambda i: B.replay_hbm_probe(src.data_ptr(), dst.data_ptr(), half, 1, st), 3)
    us_copy = tm.run(lambda i: B.replay_hbm_probe(src.data_ptr(), dst.data_ptr(), half, 1, st), 10)
    del src, dst
    torch.cuda.empty_cache()
    return nbytes / us_read / 1e3, 2 * half / us_copy / 1e3


def bench_sweeps(torch, steps=64, warmup=16):
    """Mamba-2 replay step against the conventional step over the batch (L = 16)
    and over the window length L (batch 256), on the 128-head layer: the pages
    report no gain at batch 1, a gain that grows with the batch, and the lowest
    amortised cost at the full window.  steps and warmup are whole windows for
    every L swept."""
    import dataclasses

    from synth import WORKLOADS
    base = WORKLOADS["mamba2_b256_h128_p64_n128_g8_l16"]
    out = {"batch": [], "window": []}
    for B in (1, 4, 16, 64, 256):
        shp = dataclasses.replace(base, batch=B)
        r = bench_replay(torch, shp, 7, steps, warmup)
        c = bench_conv(torch, shp, 7, steps, warmup)
        out["batch"].append({"batch": B, "replay_us": r, "conventional_us": c, "speedup": c / r})
        torch.cuda.empty_cache()
    conv = out["batch"][-1]["conventional_us"]
    for L in (1, 2, 4, 8, 16):
        shp = dataclasses.replace(base, window=L)
        r = bench_replay(torch, shp, 7, steps, warmup)
        out["window"].append({"window": L, "replay_us": r, "speedup_vs_conventional": conv / r})
        torch.cuda.empty_cache()
    return out


SPLIT_PAIRS = ((0, 0), (0, 3), (1, 3), (2, 3), (3, 3), (0, 4), (1, 4))
M2_SPLIT_PAIRS = ((0, 0), (0, 3), (1, 3), (2, 3), (3, 3), (1, 1), (2, 2))
FMT_NAMES = {0: "f32", 1: "f16sr", 2: "e4m3", 3: "e2m1", 4: "e2m1cs"}


def bench_split(torch, seed=5, layers=8, steps=64, warmup=32, flags=0, pairs=None, name="gdn_b64_h32_d128_l16"):
    """Split-precision layer, by default Gated DeltaNet (32 heads, d = 128, L = 16,
    batch 64); also the Mamba-2 layer with the 4 MiB float32 state at batch 256.

    `layers` independent layer instances are stepped in rotation, so that the
    stored copies are not served from the 256 MB Infinity Cache; reported per
    format pair (checkpoint / read copy): microseconds per layer step (whole
    windows) and algorithmic GB/s from the format-aware byte model.  (The
    accuracy of the same pairs against the float64 oracle is a GPU test,
    tests/test_gpu_split.py.)
    """
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    from hybrid_model_ssm_replay_amd.traffic import Layer, split_window_mean
    from synth import WORKLOADS, InputStream
    shape = WORKLOADS[name]
    lm = Layer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.groups, shape.window,
               2 if _bf16(flags) else 4)
    ins = InputStream(shape, seed, bf16_vectors=_bf16(flags))
    recs = dev_records(torch, ins, 16, _bf16(flags))
    kw = dict(A=ins.params["A"], D=ins.params["D"]) if shape.kind == "mamba2" else {}
    y = torch.empty((shape.batch, shape.heads, shape.head_dim), device="cuda")
    out = {"workload": name, "layers_rotated": layers, "pairs": {}}
    tm = Timer(torch)
    for cf, rf in pairs or SPLIT_PAIRS:
        lays = [ReplayLayer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                            groups=shape.groups, ckpt_fmt=cf, read_fmt=rf, seed=seed, flags=flags, **kw)
                for _ in range(layers)]
        tm.run(lambda i: lays[i % layers].step(recs[(i // layers) % 16], y), warmup * layers)
        us = tm.run(lambda i: lays[i % layers].step(recs[(i // layers) % 16], y), steps * layers)
        rd, wr = split_window_mean(lm, cf, rf)
        out["pairs"][f"{FMT_NAMES[cf]}/{FMT_NAMES[rf]}"] = {"us_per_step": us, "model_bytes_per_step": rd + wr,
                                                          "gbs": (rd + wr) / us / 1e3,
                                                          "frac_of_peak": (rd + wr) / us / 1e3 / HBM_PEAK_GBS}
        del lays
        torch.cuda.empty_cache()
    return out


def bench_bf16_records(torch, steps, warmup):
    """bf16 records (REPLAY_FLAG_BF16_RECORDS) against float32 records, same run:
    the replay and conventional steps of the Mamba-2 and GDN batch-256 layers,
    and the split-precision GDN layer at batch 64."""
    from hybrid_model_ssm_replay_amd.binding import FLAG_BF16_RECORDS as F
    from hybrid_model_ssm_replay_amd.traffic import Layer, conventional_step_bytes, replay_window_mean
    from synth import WORKLOADS
    out = {}
    for name, seed in (("mamba2_b256_h128_p64_n128_g8_l16", 1), ("gdn_b256_h32_d128_l16", 2)):
        shape = WORKLOADS[name]
        r32 = bench_replay(torch, shape, seed, steps, warmup)
        r16 = bench_replay(torch, shape, seed, steps, warmup, flags=F)
        c16 = bench_conv(torch, shape, seed, steps, warmup, flags=F)
        lm = Layer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.groups, shape.window, 2)
        rb = sum(replay_window_mean(lm))
        out[name] = {"replay_f32_records_us": r32, "replay_bf16_records_us": r16, "speedup_vs_f32_records": r32 / r16,
                     "replay_bf16_model_bytes": rb, "replay_bf16_gbs": rb / r16 / 1e3,
                     "conventional_bf16_records_us": c16, "speedup_vs_conventional": c16 / r16,
                     "conventional_bf16_gbs": sum(conventional_step_bytes(lm)) / c16 / 1e3}
        torch.cuda.empty_cache()
    out["gdn_split_b64"] = bench_split(torch, flags=F, pairs=((0, 3), (2, 3), (3, 3)))["pairs"]
    return out


def bench_zero_copy(torch, steps, warmup, rounds=3):
    """Zero-copy append (REPLAY_FLAG_RECORDS_IN_RING) on the Mamba-2 and GDN
    batch-256 layers, float32 and bf16 records: every ring slot is filled with
    records before timing, and each timed step reads the record in its slot and
    takes only the other fields as arguments (Mamba-2 C; GDN q, v).  The
    producer's write of a record is its own output and is not in the timed
    step.  The copying step is the comparison; the three layers are timed in
    alternation, `rounds` times, and each reports its median."""
    import statistics

    from hybrid_model_ssm_replay_amd.binding import FLAG_BF16_RECORDS, FLAG_RECORDS_IN_RING
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    from hybrid_model_ssm_replay_amd.traffic import Layer, replay_window_mean
    from synth import WORKLOADS, InputStream
    out = {}
    for name, seed in (("mamba2_b256_h128_p64_n128_g8_l16", 1), ("gdn_b256_h32_d128_l16", 2)):
        shape = WORKLOADS[name]
        cases = {}
        for label, flags, bf16 in (("copying", 0, False), ("f32_records", FLAG_RECORDS_IN_RING, False),
                                   ("bf16_records", FLAG_RECORDS_IN_RING | FLAG_BF16_RECORDS, True)):
            ins = InputStream(shape, seed, bf16_vectors=bf16)
            recs = dev_records(torch, ins, 32, bf16)
            kw = dict(A=ins.params["A"], D=ins.params["D"]) if shape.kind == "mamba2" else {}
            lay = ReplayLayer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                              groups=shape.groups, flags=flags, **kw)
            if flags:
                f = lay.ring_fields()
                first = "x" if "x" in f else "k"
                for sl in range(f[first].shape[0]):  # every slot holds a record
                    r = recs[sl % 32]
                    f[first][sl] = r[first]
                    for n in (("B", "dt") if first == "x" else ("alpha", "beta")):
                        f[n][:, :, sl] = r[n]
            cases[label] = (lay, recs, bf16, [])
        y = torch.empty((shape.batch, shape.heads, shape.head_dim), device="cuda")
        tm = Timer(torch)
        for _ in range(rounds):
            for label, (lay, recs, _, times) in cases.items():
                tm.run(lambda i: lay.step(recs[i % 32], y), warmup)
                times.append(tm.run(lambda i: lay.step(recs[(warmup + i) % 32], y), steps))
        entry = {}
        for label, (lay, _, bf16, times) in cases.items():
            if lay.status != 0:
                raise RuntimeError(f"device status {lay.status:#x}")
            us = statistics.median(times)
            lm = Layer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.groups,
                       shape.window, 2 if bf16 else 4)
            mb = sum(replay_window_mean(lm, in_ring=label != "copying"))
            entry[label] = {"step_us": us, "model_bytes_per_step": mb, "gbs": mb / us / 1e3,
                            "frac_of_peak": mb / us / 1e3 / HBM_PEAK_GBS}
        for label in ("f32_records", "bf16_records"):
            entry[label]["speedup_vs_copying_step"] = entry["copying"]["step_us"] / entry[label]["step_us"]
        out[name] = entry
        del cases
        torch.cuda.empty_cache()
    return out


def bench_split_error_growth(torch, seed=7, steps=4096):
    """Output error of each split-precision pair against the float32 path of the
    same library (which matches the float64 oracle to float32 rounding) on the
    batch-64 GDN layer from a zero state, as the mean normwise error over step
    ranges: whether it grows with generation length.  (The 32768-step curves
    against the float64 oracle itself are a GPU test.)"""
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    from synth import WORKLOADS, DeviceInputStream
    shape = WORKLOADS["gdn_b64_h32_d128_l16"]
    pairs = ((0, 3), (1, 3), (2, 3), (3, 3), (1, 1), (2, 2), (0, 4))
    bins = ((16, 256), (256, 1024), (1024, steps))
    lays = {p: ReplayLayer("gdn", shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                           ckpt_fmt=p[0], read_fmt=p[1], seed=seed) for p in ((0, 0),) + pairs}
    ys = {p: torch.empty((shape.batch, shape.heads, shape.head_dim), device="cuda") for p in lays}
    err = {p: torch.zeros(steps, device="cuda", dtype=torch.float64) for p in pairs}
    ins = DeviceInputStream(shape, seed)
    for t in range(steps):
        r = ins.record()
        for p, lay in lays.items():
            lay.step(r, ys[p])
        nref = torch.linalg.vector_norm(ys[(0, 0)])
        for p in pairs:
            err[p][t] = (torch.linalg.vector_norm(ys[p] - ys[(0, 0)]) / nref).double()
    out = {"steps": steps, "bins": [list(b) for b in bins], "pairs": {}}
    for p in pairs:
        e = err[p].cpu()
        out["pairs"][f"{FMT_NAMES[p[0]]}/{FMT_NAMES[p[1]]}"] = [float(e[a:b].mean()) for a, b in bins]
    del lays
    torch.cuda.empty_cache()
    return out


def bench_read_copy_error(torch, seed=6, steps=512, skip=64):
    """Output error of the e2m1 read copies (block scales only, and two-axis)
    against the float32 path of the same library, on the split-precision layer
    (Gated DeltaNet, 32 heads, d = 128, L = 16, batch 64) with a float32
    checkpoint, for isotropic keys and for keys whose dimensions have log-normal
    magnitude weights (spread 1 and 2): mean over steps skip.. of
    ||y - y_f32|| / ||y_f32||, all heads and sequences."""
    from hybrid_model_ssm_replay_amd.layer import ReplayLayer
    from synth import WORKLOADS, DeviceInputStream
    shape = WORKLOADS["gdn_b64_h32_d128_l16"]
    out = {}
    for spread in (0.0, 1.0, 2.0):
        ins = DeviceInputStream(shape, seed, key_spread=spread)
        lays = {rf: ReplayLayer("gdn", shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.window,
                                read_fmt=rf, seed=seed) for rf in (0, 3, 4)}
        ys = {rf: torch.empty((shape.batch, shape.heads, shape.head_dim), device="cuda") for rf in lays}
        err = {3: torch.zeros((), device="cuda", dtype=torch.float64), 4: torch.zeros((), device="cuda", dtype=torch.float64)}
        for t in range(steps):
            r = ins.record()
            for rf, lay in lays.items():
                lay.step(r, ys[rf])
            if t >= skip:
                nref = torch.linalg.vector_norm(ys[0])
                for rf in (3, 4):
                    err[rf] += (torch.linalg.vector_norm(ys[rf] - ys[0]) / nref).double()
        e3, e4 = (float(err[rf]) / (steps - skip) for rf in (3, 4))
        out[f"key_spread_{spread:g}"] = {"e2m1": e3, "e2m1cs": e4, "e2m1_over_e2m1cs": e3 / e4}
        del lays
        torch.cuda.empty_cache()
    return out


def _oracle_worker(args):
    """One process of the CPU baseline: the float64 stepwise oracle on `nseq`
    sequences of the workload for about budget_s seconds, single-threaded."""
    kind, shape_fields, seed, first, nseq, budget_s = args
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle.session import StepwiseSession
    from synth import InputStream, LayerShape, take_batch
    shape = LayerShape(*shape_fields)
    ins = InputStream(shape, seed)
    idx = np.arange(first, first + nseq)
    recs = [take_batch(ins.record(), idx) for _ in range(8)]
    ref = StepwiseSession(kind, np.zeros((nseq, shape.heads, shape.head_dim, shape.state_dim)), ins.params)
    steps = 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            ref.step(recs[steps % len(recs)])
            steps += 1
        el = time.perf_counter() - t0
    return steps * nseq, el


def host_cores() -> int:
    """Cores this process may use: its CPU affinity, capped by OMP_NUM_THREADS when
    that is set (the share of the host a GPU job is given)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(cap))) if cap and cap.isdigit() else max(1, n)


def cpu_baseline(shape, seed, budget_s=12.0):
    """The float64 stepwise oracle on the host's cores: one single-threaded
    process per core, each stepping one sequence of the workload for about
    budget_s seconds; the summed sequence-steps per second give the time of a
    full-batch step.  Processes are spawned fresh (they never touch the GPU)."""
    import multiprocessing as mp
    from dataclasses import astuple
    cores = host_cores()
    nseq = 1
    jobs = [(shape.kind, astuple(shape), seed, (nseq * i) % shape.batch, nseq, budget_s) for i in range(cores)]
    with mp.get_context("spawn").Pool(cores) as pool:
        res = pool.map(_oracle_worker, jobs)
    rate = sum(n / el for n, el in res)                   # sequence-steps per second, all processes
    us_per_step_full = shape.batch / rate * 1e6
    nsteps = sum(n for n, _ in res)
    return {"value": us_per_step_full, "unit": "us/step", "cores": cores, "kind": "oracle",
            "sample": f"float64 stepwise oracle, {cores} processes (one per core, one thread each), {nseq} sequences "
                      f"each, {nsteps} sequence-steps in about {budget_s:.0f} s; the summed rate is scaled to "
                      f"{shape.batch} sequences per step"}


# Extras after the headline measurement, in run order.
SECTIONS = ("conv", "skip", "verify", "gdn", "gdn_verify", "split", "m2_split", "split_error", "read_error", "bf16",
            "zero_copy", "sweeps")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--no-extra", action="store_true", help="skip baselines and other layers")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--sections", default="all",
                    help="comma list of extras to run (default all): " + ",".join(SECTIONS))
    args = ap.parse_args(argv)
    wanted = set(SECTIONS) if args.sections == "all" else set(args.sections.split(","))
    if wanted - set(SECTIONS):
        print(f"unknown sections {sorted(wanted - set(SECTIONS))}", file=sys.stderr)
        return 2
    want = (lambda sec: not args.no_extra and sec in wanted)  # noqa: E731
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the replay decode path has no cross-GPU step "
              "(sequences and heads shard with no exchange); --gpus above 1 is not measured.", file=sys.stderr)
        return 2

    import torch

    from hybrid_model_ssm_replay_amd import load_library
    from hybrid_model_ssm_replay_amd.traffic import Layer, conventional_step_bytes, replay_window_mean
    from synth import WORKLOADS

    load_library()
    torch.cuda.set_device(0)
    name = "mamba2_b256_h128_p64_n128_g8_l16"
    shape = WORKLOADS[name]
    L = shape.window
    # Whole windows only: a window's fold is timed in proportion (one fold per L steps).
    steps_timed = -(-max(args.steps, 1) // L) * L
    warmup_timed = -(-args.warmup // L) * L
    if (steps_timed, warmup_timed) != (args.steps, args.warmup):
        log(f"timing {steps_timed} steps after {warmup_timed} warm-up steps (whole windows of L = {L})")
    log("replay step", name)
    us = bench_replay(torch, shape, 1, steps_timed, warmup_timed)
    lay = Layer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.groups, L)
    rd, wr = replay_window_mean(lay)
    gbs = (rd + wr) / us / 1e3
    extra = {"replay_step_us": us, "replay_model_bytes_per_step": rd + wr, "replay_gbs": gbs,
             "tokens_per_s": shape.batch / us * 1e6}
    log("per-step distribution", name)
    extra["replay_step_distribution"] = step_distribution(torch, shape, 1)
    log("replay step, windows out of phase", name)
    us_st = bench_replay_staggered(torch, shape, 1, steps_timed, warmup_timed)
    extra["replay_step_staggered"] = {"us": us_st, "gbs": (rd + wr) / us_st / 1e3,
                                      "frac_of_peak": (rd + wr) / us_st / 1e3 / HBM_PEAK_GBS,
                                      "note": "sequence b at window phase b mod L: each step folds 1/L of them"}
    log("hbm probe")
    rgbs, cgbs = bench_probe(torch)
    extra.update({"hbm_probe_read_gbs": rgbs, "hbm_probe_copy_gbs": cgbs})
    if want("conv"):
        log("conventional step", name)
        us_c = bench_conv(torch, shape, 1, steps_timed, warmup_timed)
        crd, cwr = conventional_step_bytes(lay)
        extra.update({"conventional_step_us": us_c, "conventional_gbs": (crd + cwr) / us_c / 1e3,
                      "speedup_vs_conventional": us_c / us})
    if want("skip"):
        from hybrid_model_ssm_replay_amd.binding import FLAG_DECAY_SKIP
        log("replay step with the decay skip", name)
        us_s = bench_replay(torch, shape, 1, steps_timed, warmup_timed, flags=FLAG_DECAY_SKIP)
        extra["decay_skip"] = {"replay_step_us": us_s, "speedup_vs_exact_replay": us / us_s,
                               "rule": "checkpoint term dropped where exp(A s) < 2^-24 (an approximation)"}
        if "conventional_step_us" in extra:
            extra["decay_skip"]["speedup_vs_conventional"] = extra["conventional_step_us"] / us_s
    if want("verify"):
        vshape = WORKLOADS["mamba2_b512_h128_p64_n128_g8_l16"]
        for T in (4, 8):
            log("verify T", T)
            us_rv, us_sv = bench_verify(torch, vshape, T, 3)
            extra[f"verify_b512_T{T}"] = {"replay_verify_commit_us": us_rv, "snapshot_verify_commit_us": us_sv}
        us_std = bench_conv(torch, vshape, 3, 32, 8)
        us_rep = bench_replay(torch, vshape, 3, 32, 16)
        extra["conventional_step_b512_us"] = us_std
        extra["replay_step_b512_us"] = us_rep
        for T in (4, 8):
            v = extra[f"verify_b512_T{T}"]
            v["replay_over_standard_step"] = v["replay_verify_commit_us"] / us_std
            v["snapshot_over_standard_step"] = v["snapshot_verify_commit_us"] / us_std
            v["replay_over_replay_step"] = v["replay_verify_commit_us"] / us_rep

    if want("gdn"):
        gname = "gdn_b256_h32_d128_l16"
        gshape = WORKLOADS[gname]
        log("gdn replay step", gname)
        us_g = bench_replay(torch, gshape, 2, steps_timed, warmup_timed)
        glay = Layer("gdn", gshape.batch, gshape.heads, gshape.head_dim, gshape.state_dim, gshape.groups,
                     gshape.window)
        grd, gwr = replay_window_mean(glay)
        log("gdn conventional step", gname)
        us_gc = bench_conv(torch, gshape, 2, steps_timed, warmup_timed)
        gcrd, gcwr = conventional_step_bytes(glay)
        extra["gdn_b256"] = {"replay_step_us": us_g, "replay_gbs": (grd + gwr) / us_g / 1e3,
                             "replay_frac_of_peak": (grd + gwr) / us_g / 1e3 / HBM_PEAK_GBS,
                             "replay_model_bytes_per_step": grd + gwr, "conventional_step_us": us_gc,
                             "conventional_gbs": (gcrd + gcwr) / us_gc / 1e3, "speedup_vs_conventional": us_gc / us_g,
                             "tokens_per_s": gshape.batch / us_g * 1e6,
                             "traffic_bytes_per_launch": stored_traffic("gdn_replay_step_b256_traffic.txt", "gdn")}
        extra["gdn_b256"]["replay_step_distribution"] = step_distribution(torch, gshape, 2)
        if want("skip"):
            import numpy as np

            from hybrid_model_ssm_replay_amd.binding import FLAG_DECAY_SKIP

            def fast_decay(r):  # every other head decays by e^-2.5 per token: below 2^-24 within 7 records
                r["alpha"][..., ::2] = np.float32(np.exp(-2.5))
                return r
            log("gdn replay step with the decay skip", gname)
            us_gs = bench_replay(torch, gshape, 2, steps_timed, warmup_timed, flags=FLAG_DECAY_SKIP)
            us_gf = bench_replay(torch, gshape, 2, steps_timed, warmup_timed, rec_fn=fast_decay)
            us_gfs = bench_replay(torch, gshape, 2, steps_timed, warmup_timed, flags=FLAG_DECAY_SKIP,
                                  rec_fn=fast_decay)
            extra["gdn_b256"]["decay_skip"] = {
                "synthetic_inputs": {"exact_us": us_g, "skip_us": us_gs, "speedup": us_g / us_gs},
                "half_heads_fast_decay": {"exact_us": us_gf, "skip_us": us_gfs, "speedup": us_gf / us_gfs},
                "rule": "checkpoint term dropped where exp(g) < 2^-24 (an approximation)"}

        for T in (4, 8, 16) if want("gdn_verify") else ():
            log("gdn verify T", T)
            us_rv, us_sv = bench_verify(torch, gshape, T, 2)
            extra["gdn_b256"][f"verify_T{T}"] = {"replay_verify_commit_us": us_rv, "snapshot_verify_commit_us": us_sv,
                                                 "replay_over_conventional_step": us_rv / us_gc,
                                                 "snapshot_over_conventional_step": us_sv / us_gc}

    if want("split"):
        log("split precision")
        extra["gdn_split_b64"] = bench_split(torch)
    if want("m2_split"):
        log("split precision, Mamba-2 batch 256")
        extra["mamba2_split_b256"] = bench_split(torch, seed=1, layers=4, steps=32, warmup=16,
                                                 pairs=M2_SPLIT_PAIRS, name="mamba2_b256_h128_p64_n128_g8_l16")
        base = extra.get("replay_step_us")
        for v in extra["mamba2_split_b256"]["pairs"].values():
            v["speedup_vs_f32_replay_step"] = base / v["us_per_step"]
    if want("split_error"):
        log("split-precision error growth")
        extra["split_error_growth_b64"] = bench_split_error_growth(torch)
    if want("read_error"):
        log("read copy error")
        extra["read_copy_error_b64"] = bench_read_copy_error(torch)
    if want("bf16"):
        log("bf16 records")
        extra["bf16_records"] = bench_bf16_records(torch, steps_timed, warmup_timed)
    if want("zero_copy"):
        log("zero-copy append")
        extra["zero_copy"] = bench_zero_copy(torch, steps_timed, warmup_timed)
    if want("sweeps"):
        log("batch and window sweeps")
        extra["mamba2_sweeps"] = bench_sweeps(torch)

    traffic = stored_traffic("m2_replay_step_b256_traffic.txt", "m2")
    roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": traffic, "kernel": "m2_replay_step<8, 2, false, float, false, 0, 0>",
            "bytes_per_launch": rd + wr}
    cpu = None if args.no_cpu else cpu_baseline(shape, 1)
    out = {
        "metric": "SSM decode us/step + achieved HBM GB/s, B=256 L=16 (Mamba-2 & GDN)",
        "value": us, "unit": "us/step", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "steps_timed": steps_timed, "warmup_timed": warmup_timed,
        "ms_per_step": us / 1e3, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": name, "layer": "Mamba-2", "batch": shape.batch, "heads": shape.heads,
                   "head_dim": shape.head_dim, "state_dim": shape.state_dim, "groups": shape.groups, "window": L,
                   "state_mib_per_seq": shape.heads * shape.head_dim * shape.state_dim * 4 / 2 ** 20},
        "roofline": roof,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
