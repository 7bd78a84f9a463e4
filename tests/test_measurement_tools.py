"""Host logic of the measurement tools (CPU): the algorithmic byte model behind
the bench's roofline, the verify-session model behind the verify traffic
summary, and the counter selection of the rocprofv3 summary tool.

The expected values are the model's terms written out by hand: bytes per
sequence of a state, a new record, a ring record and an output."""
import csv

import pytest

from hybrid_model_ssm_replay_amd import rocprof_summary as rs
from hybrid_model_ssm_replay_amd.traffic import (Layer, conventional_step_bytes, replay_window_mean,
                                                 verify_session_bytes)


def test_headline_window_mean_by_hand():
    # Mamba-2, 128 heads, P = 64, N = 128, 8 groups, L = 16, batch 256, float32 records.
    state = 128 * 64 * 128 * 4                     # 4 MiB checkpoint per sequence
    record_in = (128 * 64 + 2 * 8 * 128) * 4 + 128 * 4   # x, B, C, dt
    ring_rec = (128 * 64 + 8 * 128) * 4 + 128 * 4        # x, B, dt (C is not kept)
    y = 128 * 64 * 4
    # Per window: every step reads the checkpoint and its new record, step m reads
    # m - 1 older records (0 + 1 + ... + 15 = 120), the fold reads the 16 records
    # of the full window; every step appends a record and writes y, the fold
    # writes the checkpoint once.
    read = 16 * (state + record_in) + 120 * ring_rec + 16 * ring_rec
    write = 16 * (ring_rec + y) + state
    expected = (read + write) / 16 * 256
    rd, wr = replay_window_mean(Layer("mamba2", 256, 128, 64, 128, 8, 16))
    assert rd + wr == expected == 1250754560
    crd, cwr = conventional_step_bytes(Layer("mamba2", 256, 128, 64, 128, 8, 16))
    assert crd + cwr == (2 * state + record_in + y) * 256


def test_verify_session_by_hand():
    # Mamba-2, one head, P = N = 16, one group, L = 4, batch 2, T = 2; sequence 0
    # accepts both drafts every time, sequence 1 none.
    lay = Layer("mamba2", 2, 1, 16, 16, 1, 4)
    state, record_in, ring_rec, y = 16 * 16 * 4, (16 + 32) * 4 + 4, (16 + 16) * 4 + 4, 16 * 4
    T = 2
    draft_rw = 2 * T * record_in, 2 * T * (ring_rec + y)
    # counts before each call: (0, 0), (2, 0), (4, 0) -> sequence 0 folds first in call 3
    reads = [2 * state + draft_rw[0], 2 * state + 2 * ring_rec + draft_rw[0], 2 * state + 4 * ring_rec + draft_rw[0]]
    writes = [draft_rw[1], draft_rw[1], draft_rw[1] + state]
    rd, wr = verify_session_bytes(lay, T, [[2, 0]], 3)
    assert rd == pytest.approx(sum(reads) / 3) and wr == pytest.approx(sum(writes) / 3)


def _counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Value"])
        w.writeheader()
        for i, (name, grid, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Grid_Size": grid, "Counter_Value": v})


def test_traffic_selection_and_calibration(tmp_path):
    # The probe copies 1 MiB: FETCH_SIZE reads back half of it, WRITE_SIZE all of it.
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    kern = [("void k<1>(A)", 256, v) for v in (10, 20, 30, 40)] + [("void k<1>(A)", 512, 99)]
    _counters(fetch, [("probe_copy_k(x)", 1, 512)] + kern)
    _counters(write, [("probe_copy_k(x)", 1, 1024)] + [(n, g, v / 10) for n, g, v in kern])
    r = rs.traffic(str(fetch), str(write), "k<1>", 1 << 20, 256, 2, 1)  # launches 2 and 3 of grid 256
    assert r["dispatches"] == 2 and r["factor_read"] == 2.0 and r["factor_write"] == 1.0
    assert r["fetch_kib"] == 25.0 and r["write_kib"] == 2.5
    assert r["traffic_bytes_per_launch"] == 25.0 * 1024 * 2 + 2.5 * 1024
