"""Host-side checks of the benchmark's protocol (no GPU): the rotation over buffer sets
continues across warm-up and every timing, the set count covers the Infinity Cache four
times over, committed counter summaries are used only for the kernel sources they were
taken on, the flop count of cached replay, the CPU baseline's fields, and the refusal of
more than one GPU."""
import json
import math
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


class FakeGraph:
    """Stands in for a captured HIP graph: a replay records the sets its calls use."""

    def __init__(self, start, n, nsets, log):
        self.start, self.n, self.nsets, self.log = start, n, nsets, log

    def replay(self):
        self.log.extend((self.start + i) % self.nsets for i in range(self.n))


def graph_runner(sets, rot, per_replay, log):
    r = bench.Runner(lambda s: None, sets, rot, stream=None, eager=False, per_replay=per_replay)
    r._capture = lambda start, n: FakeGraph(start, n, len(sets), log)
    return r


@pytest.mark.parametrize("nsets,warmup,steps", [(7, 5, 20), (64, 5, 20), (64, 800, 8000), (3, 0, 1), (5, 4, 14)])
def test_rotation_continues_across_warmup_and_timings(nsets, warmup, steps):
    """Graph replays of the verify runner (its warm-up and five windows) and then of the
    step runner (W warm-up steps, then the K timed steps) use the sets in one unbroken
    rotation, as the bench drives them: every graph prepared first, then run."""
    sets = list(range(nsets))
    rot = bench.Rotation(nsets)
    per = bench.per_replay_of(nsets)
    assert per % nsets == 0
    log = []
    step = graph_runner(sets, rot, per, log)
    verify = graph_runner(sets, rot, per, log)
    n_vwarm = max(warmup, bench.SETTLE_LAUNCHES)
    n_ver = max(steps, bench.SETTLE_LAUNCHES)
    verify.prepare(n_vwarm)
    for k in range(5):
        verify.prepare(n_ver, ahead=n_vwarm + k * n_ver)
    off = n_vwarm + 5 * n_ver
    step.prepare(warmup, ahead=off)
    step.prepare(steps, ahead=off + warmup)
    captured = (len(verify.graphs), len(step.graphs))
    verify.run(n_vwarm)
    for _ in range(5):
        verify.run(n_ver)
    step.run(warmup)
    step.run(steps)
    assert (len(verify.graphs), len(step.graphs)) == captured  # nothing captured between phases
    total = n_vwarm + 5 * n_ver + warmup + steps
    assert log == [i % nsets for i in range(total)]
    # every launch uses a set the previous nsets - 1 launches did not touch
    for i in range(1, len(log)):
        window = log[max(0, i - nsets + 1):i]
        assert log[i] not in window


def test_settled_timing_runs_exactly_w_then_k(monkeypatch):
    """The single-kernel modes: untimed settling calls, then exactly W warm-up calls, then
    exactly K timed calls, in one rotation, all graphs captured before the first runs."""
    sets = list(range(5))
    log, timed = [], []
    r = graph_runner(sets, bench.Rotation(5), 5, log)
    monkeypatch.setattr(r, "warm", lambda n: r.run(n))

    def fake_timed(n):
        timed.append((len(log), n))
        r.run(n)
        return 1.0
    monkeypatch.setattr(r, "timed", fake_timed)
    n_settle = int(bench.SETTLE_SECONDS / 100e-6)
    bench.settled_timing(r, warmup=3, steps=7, est_us=100.0)
    assert timed == [(n_settle + 3, 7)]
    assert log == [i % 5 for i in range(n_settle + 3 + 7)]


def test_eager_rotation_matches_graph_rotation():
    sets = list(range(6))
    used = []
    rot = bench.Rotation(6)
    r = bench.Runner(lambda s: used.append(s), sets, rot, stream=None, eager=True, per_replay=6)
    r.run(4)
    r.run(9)
    assert used == [i % 6 for i in range(13)]
    assert rot.pos == 13


def test_rotating_sets_cover_the_cache_four_times():
    for read in (16 << 20, 29_360_128, 64 << 20, 536_870_912, 4 << 30):
        R = bench.rotating_sets(read, set_bytes=2 * read)
        assert R >= 2
        if 2 * read * math.ceil(4 * bench.INFINITY_CACHE_BYTES / read) <= 16e9:
            assert R * read >= 4 * bench.INFINITY_CACHE_BYTES
        assert R * 2 * read <= max(16e9, 2 * 2 * read)


def test_profile_record_requires_matching_kernel_sources(tmp_path, monkeypatch):
    h = bench.kernel_source_hash("recurrent")
    assert len(h) == 16 and h == bench.kernel_source_hash("recurrent")
    assert h != bench.kernel_source_hash("prefill")
    rec = {"kernel_source_sha256_16": h, "hbm_bytes_per_launch": 123.0}
    (tmp_path / "gdn_verify_wl_traffic.json").write_text(json.dumps(rec))
    (tmp_path / "gdn_verify_old_traffic.json").write_text(json.dumps(dict(rec, kernel_source_sha256_16="0" * 16)))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.traffic_from_profiles("gdn_verify", "wl", "recurrent") == 123.0
    assert bench.traffic_from_profiles("gdn_verify", "old", "recurrent") is None
    assert bench.traffic_from_profiles("gdn_verify", "missing", "recurrent") is None


def test_committed_traffic_summaries_are_consistent():
    """Every committed *_traffic.json: its bytes are the calibrated counter sums of its
    kernels, and its ratio is those bytes over the algorithmic bytes."""
    files = [f for f in os.listdir(bench.PROFILES) if f.endswith("_traffic.json")]
    assert files
    for f in files:
        rec = json.load(open(os.path.join(bench.PROFILES, f)))
        tot = sum(k["fetch_kib_per_dispatch"] * 1024 * rec["fetch_scale"] + k["write_kib_per_dispatch"] * 1024 * rec["write_scale"]
                  for k in rec["kernels"])
        assert tot == pytest.approx(rec["hbm_bytes_per_launch"], rel=1e-9), f
        assert rec["ratio"] == pytest.approx(rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"], rel=1e-9), f
        assert 1.9 < rec["fetch_scale"] < 2.1 and rec["write_scale"] == pytest.approx(1.0, abs=0.01), f


def test_replay_flops_closed_form():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    idx = np.array([0, 1, -1, 7] + [2] * (w.batch - 4), dtype=np.int32)
    rlen = np.array([4, 0, 3, 9] + [1] * (w.batch - 4), dtype=np.int32)  # 9 > T: replays nothing
    elems = w.Hv * w.dk * w.dv
    valid = w.batch - 1
    replayed = 4 + 0 + 0 + (w.batch - 4)  # the padding row's 3 and the out-of-range 9 do not count
    assert bench.replay_flops(w, idx, rlen) == valid * w.T * 7 * elems + replayed * 5 * elems


def test_cpu_baseline_reports_its_host():
    w = workloads.WORKLOADS[0]
    x = workloads.make_inputs(w, seed=0)
    cb = bench.cpu_baseline(w, x, budget_s=0.3)
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    assert len(cb["runs_tokens_per_s"]) == 3
    assert cb["value"] == sorted(cb["runs_tokens_per_s"])[1]
    assert cb["cores"] >= 1 and cb["nproc"] >= 1 and cb["hardware_concurrency"] >= cb["nproc"]
    assert isinstance(cb["cpu_model"], str) and cb["cpu_model"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
