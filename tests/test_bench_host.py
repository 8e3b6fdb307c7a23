"""bench.py's host logic, on the CPU: the timing stop rule (LR-AttnRes paper, App. I,
"Measurement protocol": windows of launches until two consecutive windows each have a
coefficient of variation of at most 1 % and medians within 0.5 %, at most 30 windows), the
byte, roofline and ceiling arithmetic, the stream fractions, the source digest (code only)
and the one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


class ReplayTimer:
    """Stands in for the HIP-event timer: each timed launch takes the next duration of seq."""
    seq = []

    def __init__(self, torch):
        self.buf = []

    def run(self, fn):
        fn()
        self.buf.append(ReplayTimer.seq.pop(0))

    def collect_ms(self):
        out, self.buf = self.buf, []
        return out


def stop_rule(monkeypatch, seq):
    ReplayTimer.seq = list(seq)
    monkeypatch.setattr(bench, "Timer", ReplayTimer)
    monkeypatch.setattr(bench, "FIXED_REPS", None)
    launches = []
    evictions = []
    t = bench.time_calls(None, lambda: evictions.append(1), lambda: launches.append(1), warm=0)
    return t, len(launches), len(evictions)


def window(*v):
    assert len(v) == bench.WINDOW
    return list(v)


def test_stop_rule_two_steady_windows(monkeypatch):
    t, launches, evictions = stop_rule(monkeypatch, [1.0] * (2 * bench.WINDOW))
    assert t.converged and t.windows == 2 and float(t) == 1.0
    assert launches == evictions == 2 * bench.WINDOW  # every launch follows an eviction


def test_stop_rule_waits_out_a_noisy_window(monkeypatch):
    noisy = window(1.0, 1.1, 0.9, 1.0, 1.05, 0.95)  # CV about 6 %
    steady = [1.0] * bench.WINDOW
    t, launches, _ = stop_rule(monkeypatch, noisy + steady + steady)
    assert t.converged and t.windows == 3 and launches == 3 * bench.WINDOW


def test_stop_rule_waits_out_a_drift(monkeypatch):
    a = [1.000] * bench.WINDOW
    b = [1.010] * bench.WINDOW  # 1 % above a: drift over 0.5 %
    c = [1.012] * bench.WINDOW  # 0.2 % above b
    t, _, _ = stop_rule(monkeypatch, a + b + c)
    assert t.converged and t.windows == 3
    assert float(t) == pytest.approx(1.011)  # median of the last two windows' launches
    assert t.mean == pytest.approx(1.011)


def test_stop_rule_gives_up_after_max_windows(monkeypatch):
    noisy = window(1.0, 1.2, 0.8, 1.0, 1.2, 0.8)
    t, launches, _ = stop_rule(monkeypatch, noisy * bench.MAX_WINDOWS)
    assert not t.converged and t.windows == bench.MAX_WINDOWS
    assert launches == bench.MAX_WINDOWS * bench.WINDOW
    assert t.cv > bench.CV_MAX


def test_fixed_reps(monkeypatch):
    ReplayTimer.seq = [3.0, 1.0, 2.0]
    monkeypatch.setattr(bench, "Timer", ReplayTimer)
    monkeypatch.setattr(bench, "FIXED_REPS", 3)
    t = bench.time_calls(None, lambda: None, lambda: None, warm=0)
    assert float(t) == 2.0 and t.windows == 0 and not t.converged


def test_bytes_and_row_entry():
    # a read of n sources moves n rows in and one row out per token
    assert bench.fwd_bytes(16384, 1024, 49, 2) == 2 * 50 * 1024 * 16384
    e = bench.row_entry(2.0, 16e9, tokens=1e6)
    assert e["GBps"] == 8000.0 and e["frac"] == 1.0 and e["tokens_per_s"] == 5e8


def test_mix_ceiling():
    ceil = {"read": {"GBps": 7000.0}, "write_GBps_derived": 5000.0}
    n = 9
    expect = 1.0 / ((n / (n + 1)) / 7000.0 + (1 / (n + 1)) / 5000.0)
    assert bench.mix_ceiling(ceil, n) == pytest.approx(expect)
    # between the write and the read rate, nearer the read rate as n grows
    assert 5000.0 < bench.mix_ceiling(ceil, 1) < bench.mix_ceiling(ceil, 49) < 7000.0
    assert bench.mix_ceiling(None, n) is None


def test_kernel_stream_fractions():
    name, (_, _, _, _, _, priced) = next(iter(bench.KERNEL_STREAMS.items()))
    group, key = priced[0]
    rows = {group: {key: {"GBps": 4000.0}}}
    bench.kernel_stream_fractions(rows, {"streams": {name: {"GBps": 5000.0}}})
    e = rows[group][key]
    assert e["stream"] == name and e["frac_of_stream_ceiling"] == 0.8
    # no stream measured: the row is left as it was
    rows2 = {group: {key: {"GBps": 4000.0}}}
    bench.kernel_stream_fractions(rows2, {})
    assert "frac_of_stream_ceiling" not in rows2[group][key]


def test_stream_shapes():
    assert bench.stream_slots(1024) == (2,)
    assert bench.stream_slots(2048) == (4,)
    assert bench.stream_slots(7168) == (4, 16)
    assert bench.stream_row_waves(2048) == (1,)
    assert bench.stream_row_waves(7168) == (1, 2, 4)


def test_code_text_and_digest(tmp_path, monkeypatch):
    src = 'int a = 1; // note\n/* block\n comment */\nconst char* s = "// kept";\n\n  int b;\n'
    assert bench.code_text(src) == 'int a = 1;\nconst char* s = "// kept";\nint b;'
    d = tmp_path / "csrc"
    d.mkdir()
    (d / "k.hip").write_text(src)
    monkeypatch.setattr(bench, "CSRC", str(d))
    before = bench.source_digest()
    (d / "k.hip").write_text("// a new comment\n" + src.replace("  int b;", "int b;   "))
    assert bench.source_digest() == before  # comments and layout do not count
    (d / "k.hip").write_text(src.replace("int b;", "int b = 2;"))
    assert bench.source_digest() != before  # code does


def test_traffic_entry_follows_the_digest(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"source_digest": "abc", "kernels": {"k": {"bytes_per_launch": 7}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_entry("abc", "k") == 7
    assert bench.traffic_entry("abd", "k") is None  # counters taken on other code
    assert bench.traffic_entry("abc", "other") is None


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
