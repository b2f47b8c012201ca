"""Host logic of bench.py (CPU only): the rocprofv3 trace summary and the
link between the committed counter summary and the kernel source."""
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _fake_trace(path, durations):
    """A database with the `kernels` view bench.summarize reads (name, start,
    duration), one row per dispatch."""
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, start integer, duration integer)")
    t = 0
    for name, ds in durations.items():
        for d in ds:
            con.execute("insert into kernels values (?, ?, ?)", (name, t, d))
            t += d + 10
    con.commit()
    con.close()


def test_summarize_leaves_out_the_warmup_dispatches(tmp_path, capsys):
    # a kernel whose first 3 dispatches are slow (the clock ramp), then steady
    _fake_trace(tmp_path / "x_results.db", {"fwd": [9000, 8000, 7000, 1000, 1000, 1200],
                                              "copy": [500, 500]})
    bench.summarize(str(tmp_path), skip=3)
    out = capsys.readouterr().out
    line = [ln for ln in out.splitlines() if "| fwd |" in ln][0]
    assert "calls=3" in line and "avg_us=1.07" in line and "max_us=1.20" in line
    # a kernel with no more dispatches than `skip` keeps them all
    line = [ln for ln in out.splitlines() if "| copy |" in ln][0]
    assert "calls=2" in line and "avg_us=0.50" in line
    bench.summarize(str(tmp_path), skip=0)
    out = capsys.readouterr().out
    line = [ln for ln in out.splitlines() if "| fwd |" in ln][0]
    assert "calls=6" in line and "max_us=9.00" in line


def test_kernel_hash_ignores_comments_and_whitespace_only():
    src = "// header\nint f(int a) {  /* note */ return a + 1; }\n"
    same = "/* other words */\nint f(int a)\n{\n    return a + 1;  // trailing\n}\n"
    changed = "int f(int a) { return a + 2; }\n"
    assert bench.kernel_sha(src) == bench.kernel_sha(same)
    assert bench.kernel_sha(src) != bench.kernel_sha(changed)
    # the committed forward kernel hashes to a 16-digit hex string
    h = bench.kernel_sha()
    assert len(h) == 16 and int(h, 16) >= 0


def test_traffic_is_null_unless_the_summary_matches_the_kernel(tmp_path, monkeypatch):
    summary = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(summary))
    assert bench.read_traffic() is None                      # no summary
    summary.write_text(f"- kernel_source_sha256_16: `{bench.kernel_sha()}`\n"
                       "- hbm_bytes_per_launch: 357821983\n")
    assert bench.read_traffic() == 357821983.0
    summary.write_text("- kernel_source_sha256_16: `0000000000000000`\n"
                       "- hbm_bytes_per_launch: 357821983\n")
    assert bench.read_traffic() is None                      # counters of another kernel

