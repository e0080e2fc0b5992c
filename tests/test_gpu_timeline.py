"""The timeline build (libqam_timeline.so): one stamped decode step of a
two-layer Qwen3-0.6B-shaped decoder, run in a process of its own (the
timeline library replaces the product library there).  Every chosen product
must report its waves, a positive span, and its phases in order."""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "query_adaptive_mixed_amd", "libqam_timeline.so")

pytestmark = pytest.mark.gpu


def test_timeline_of_a_decode_step():
    if not os.path.exists(LIB):
        pytest.skip("the timeline library is not built")
    env = dict(os.environ, QAM_LIBRARY=LIB)
    r = subprocess.run([sys.executable, "-u", "-m", "query_adaptive_mixed_amd.timeline", "--n-layers", "2",
                        "--layers", "0", "--warmup", "1", "--rung", "4"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    lines = r.stdout.splitlines()
    heads = [l for l in lines if re.match(r"^(q\|k\|v|o|gate\|up|down|next q\|k\|v)\s+\d+ waves, span", l)]
    assert len(heads) == 5, r.stdout
    for h in heads:
        waves = int(re.search(r"(\d+) waves", h).group(1))
        span = float(re.search(r"span ([0-9.]+) us", h).group(1))
        assert waves > 0 and 0.0 < span < 1000.0, h
    # within each product, the median stamps follow the order of the phases
    order = ["work start", "x staged", "tiles done", "row sums", "wave exit"]
    block = []
    for l in lines + ["end"]:
        if l in heads or l == "end":
            if block:
                med = {m.group(1).strip(): float(m.group(2)) for m in
                       (re.match(r"^\s+(.+?)\s+n\s+\d+\s+min\s+[0-9.-]+\s+median\s+([0-9.-]+)", b) for b in block) if m}
                seq = [med[k] for k in order if k in med]
                assert len(seq) == len(order), block
                assert all(a <= b for a, b in zip(seq, seq[1:])), block
            block = []
        elif l.startswith("    "):
            block.append(l)
