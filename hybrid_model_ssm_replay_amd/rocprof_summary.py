"""Summaries of rocprofv3 output for the replay kernels.

    python -m hybrid_model_ssm_replay_amd.rocprof_summary trace <kernel_trace.csv>
    python -m hybrid_model_ssm_replay_amd.rocprof_summary verify <fetch_counter_collection.csv> \
        <write_counter_collection.csv> <kernel_trace.csv>
    python -m hybrid_model_ssm_replay_amd.rocprof_summary traffic <fetch_counter_collection.csv> \
        <write_counter_collection.csv> <kernel-substring> <probe-copy-bytes> [grid-size [first-n [skip-n]]]

``verify`` prints, for the verify measurements of bench.py (Mamba-2 at batch
512 and Gated DeltaNet at batch 256, T = 4 then T = 8, replay and snapshot
kernels), the calibrated traffic and mean duration per launch next to the byte
model, the replay model replaying the bench's seeded accepted counts.
``trace`` prints the mean, min and max duration per kernel and launch size
(grid size in work-items).  ``traffic`` prints FETCH_SIZE and WRITE_SIZE (KiB
per dispatch) of the named kernel (only its launches of the given grid size,
when one is given, and only the first n of those in dispatch order after
skipping the first skip-n, when n is given), calibrated
against the library's HBM probe copy kernel, whose bytes are known: it reads and
writes exactly the same number of bytes, so factor_read = WRITE_SIZE / FETCH_SIZE
of the probe and factor_write = 1 when the probe's WRITE_SIZE equals the bytes
it copies.  The calibrated traffic per launch is
FETCH_SIZE * 1024 * factor_read + WRITE_SIZE * 1024 * factor_write.
"""
from __future__ import annotations

import collections
import csv
import sys

PROBE_COPY = "probe_copy_k"


def _grid(r) -> int:
    if "Grid_Size" in r:
        return int(r["Grid_Size"])
    return int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y", 1) or 1) * int(r.get("Grid_Size_Z", 1) or 1)


def _order(r) -> int:
    for f in ("Dispatch_Id", "Correlation_Id"):
        if r.get(f):
            return int(r[f])
    return 0


def _by_kernel(path: str, value_field: str, grid: int | None = None, with_grid: bool = False,
               first: int | None = None, skip: int = 0):
    d = collections.defaultdict(list)
    seen = collections.Counter()
    for r in sorted(csv.DictReader(open(path)), key=_order):
        g = _grid(r)
        if grid is not None and g != grid and PROBE_COPY not in r["Kernel_Name"]:
            continue
        key = (r["Kernel_Name"], g) if with_grid else r["Kernel_Name"]
        if PROBE_COPY not in r["Kernel_Name"]:
            seen[key] += 1
            if seen[key] <= skip:
                continue
        if first is not None and PROBE_COPY not in r["Kernel_Name"] and len(d[key]) >= first:
            continue
        if value_field == "duration":
            d[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        else:
            d[key].append(float(r[value_field]))
    return d


def _find(d, sub):
    keys = [k for k in d if sub in k]
    if len(keys) != 1:
        raise KeyError(f"{sub!r} matches {len(keys)} kernels: {keys}")
    return keys[0]


def trace(path: str) -> str:
    d = _by_kernel(path, "duration", with_grid=True)
    lines = ["| kernel | grid (work-items) | dispatches | mean us | min us | max us |", "|---|---|---|---|---|---|"]
    for (k, g), v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k[:90]}` | {g} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} |")
    return "\n".join(lines)


def traffic(fetch_csv: str, write_csv: str, kernel: str, copy_bytes: int | None = None,
            grid: int | None = None, first: int | None = None, skip: int = 0) -> dict:
    fe = _by_kernel(fetch_csv, "Counter_Value", grid, first=first, skip=skip)
    wr = _by_kernel(write_csv, "Counter_Value", grid, first=first, skip=skip)
    pk_f, pk_w = _find(fe, PROBE_COPY), _find(wr, PROBE_COPY)
    probe_fetch = sum(fe[pk_f]) / len(fe[pk_f])
    probe_write = sum(wr[pk_w]) / len(wr[pk_w])
    f_w = 1.0 if copy_bytes is None else copy_bytes / (probe_write * 1024)
    f_r = probe_write * f_w / probe_fetch
    k_f, k_w = _find(fe, kernel), _find(wr, kernel)
    kf = sum(fe[k_f]) / len(fe[k_f])
    kw = sum(wr[k_w]) / len(wr[k_w])
    return {"kernel": k_f, "dispatches": len(fe[k_f]), "fetch_kib": kf, "write_kib": kw,
            "probe_fetch_kib": probe_fetch, "probe_write_kib": probe_write, "factor_read": f_r,
            "factor_write": f_w, "traffic_bytes_per_launch": kf * 1024 * f_r + kw * 1024 * f_w}


# The verify runs of bench.py: workload, seed, launch grid (work-items), the
# replay kernel for each T with the launches of that kernel to skip (the
# Gated DeltaNet verify is compiled per pass count, one kernel per T here), and
# the snapshot kernel.  Launches per T: 8 warm-up + 16 timed (replay), 4 + 16
# (snapshot).
VERIFY_RUNS = (("mamba2_b512_h128_p64_n128_g8_l16", 3, 8388608,
                {4: ("m2_replay_verify<8, 2, false, float, 0, 0>", 0),
                 8: ("m2_replay_verify<8, 2, false, float, 0, 0>", 1)},
                "m2_snapshot_verify<8, 2, float>"),
               ("gdn_b256_h32_d128_l16", 2, 2097152,
                {4: ("gdn_replay_verify<0, 0, 8, 2, float, false, 1>", 0),
                 8: ("gdn_replay_verify<0, 0, 8, 2, float, false, 2>", 0)},
                "gdn_snapshot_verify<8, 2, float>"))
VERIFY_TS, REPLAY_CALLS, SNAP_CALLS, DRAFT_SETS = (4, 8), 24, 20, 4


def verify(fetch_csv: str, write_csv: str, trace_csv: str, copy_bytes: int = 1 << 30) -> str:
    import os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from synth import WORKLOADS, InputStream
    from hybrid_model_ssm_replay_amd.traffic import Layer, snapshot_verify_bytes, verify_session_bytes
    lines = ["| workload | T | kernel | launches | mean us | traffic GB | model GB | traffic / model | GB/s (model) |",
             "|---|---|---|---|---|---|---|---|---|"]
    for name, seed, grid, rks, sk in VERIFY_RUNS:
        dur = _by_kernel(trace_csv, "duration", grid)
        shape = WORKLOADS[name]
        lay = Layer(shape.kind, shape.batch, shape.heads, shape.head_dim, shape.state_dim, shape.groups, shape.window)
        for ti, T in enumerate(VERIFY_TS):
            ins = InputStream(shape, seed)  # the bench's draws: draft sets first, then accepted counts
            for _ in range(DRAFT_SETS):
                ins.drafts(T)
            accs = [ins.accepted(T) for _ in range(DRAFT_SETS)]
            rd, wr = verify_session_bytes(lay, T, accs, REPLAY_CALLS)
            srd, swr = snapshot_verify_bytes(lay, T)
            rk, rskip = rks[T]
            for kern, calls, skip, model in ((rk, REPLAY_CALLS, rskip, rd + wr), (sk, SNAP_CALLS, ti, srd + swr)):
                r = traffic(fetch_csv, write_csv, kern, copy_bytes, grid, calls, skip * calls)
                ds = dur[_find(dur, kern)][skip * calls:(skip + 1) * calls]
                us = sum(ds) / len(ds)
                t = r["traffic_bytes_per_launch"]
                lines.append(f"| {name} | {T} | `{kern}` | {r['dispatches']} | {us:.1f} | {t / 1e9:.3f} | "
                             f"{model / 1e9:.3f} | {t / model:.3f} | {model / us / 1e3:.0f} |")
    return "\n".join(lines)


def main(argv):
    if argv[0] == "trace":
        print(trace(argv[1]))
    elif argv[0] == "verify":
        print(verify(argv[1], argv[2], argv[3]))
    elif argv[0] == "traffic":
        r = traffic(argv[1], argv[2], argv[3], int(argv[4]) if len(argv) > 4 else None,
                    int(argv[5]) if len(argv) > 5 else None, int(argv[6]) if len(argv) > 6 else None,
                    int(argv[7]) if len(argv) > 7 else 0)
        for k, v in r.items():
            print(f"{k}: {v}")
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
