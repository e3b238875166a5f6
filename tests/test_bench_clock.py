"""Host logic of bench.py (CPU only).  The clock sampler must average the
graphics clock of every XCD and the socket power over the readings stamped
inside the timed span, ignoring the memory, video and SoC clocks that the same
amd-smi listing holds, and readings stamped outside the span.  And bench.py
refuses to run on more than one GPU."""
import os
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _reading(stamp, gfx, power):
    lines = [f"T{stamp:.6f}", "GPU: 0", "    POWER:", f"        SOCKET_POWER: {power} W",
             "        THROTTLE_STATUS: N/A", "    CLOCK:"]
    for i, c in enumerate(gfx):
        lines += [f"        GFX_{i}:", f"            CLK: {c} MHz", "            MIN_CLK: 500 MHz",
                  "            MAX_CLK: 2400 MHz", "            DEEP_SLEEP: DISABLED"]
    lines += ["        MEM_0:", "            CLK: 2000 MHz", "        VCLK_0:", "            CLK: 59 MHz",
              "        DCLK_0:", "            CLK: 48 MHz", "        SOCCLK_0:", "            CLK: 47 MHz", ""]
    return "\n".join(lines)


def _summary(text, t0, t1):
    s = bench.ClockSampler.__new__(bench.ClockSampler)
    fd, s.path = tempfile.mkstemp()
    with os.fdopen(fd, "w") as fh:
        fh.write(text)
    return s.summary(t0, t1)


def test_graphics_clocks_and_power_inside_the_span():
    text = (_reading(100.0, [1000] * 8, 900) +            # before the span
            _reading(101.0, [1600, 1700] * 4, 1400) +
            _reading(102.0, [1500, 1700] * 4, 1398) +
            _reading(105.0, [2400] * 8, 500))              # after it
    got = _summary(text, 100.5, 103.0)
    assert got == {"sclk_mhz": 1625, "samples": 2, "socket_power_w": 1399}


def test_no_reading_in_the_span_gives_none():
    assert _summary(_reading(100.0, [1600] * 8, 1400), 200.0, 300.0) is None


def test_bench_refuses_more_than_one_gpu():
    """The path runs on one GPU: --gpus 2 exits with status 2 and says so,
    before touching a GPU."""
    import subprocess
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
