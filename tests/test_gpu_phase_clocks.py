"""The phase-clock tool (``python -m linear_attention_prefill_amd.phase_clocks``)
on the instrumented library: every wave of workgroup 0 reports its items with
phases that add up to no more than the item."""
import os
import subprocess
import sys

import pytest
import torch

from kda_testlib import announce
from linear_attention_prefill_amd import kda as K

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rows(out, label):
    """(wave, items, item clocks, phase clocks) rows of one kernel's table."""
    lines = out.splitlines()
    i = lines.index(label + ":")
    rows = []
    for ln in lines[i + 2:]:
        f = ln.split()
        if not f or not f[0].isdigit():
            break
        rows.append((int(f[0]), int(f[1]), float(f[2]), [float(x) for x in f[3:]]))
    return rows


@pytest.mark.parametrize("workload,label", [("packed", "intra-chunk kernel"),
                                            ("short", "fused prefill")])
def test_phase_clock_tables(workload, label):
    if not os.path.exists(K.CLOCKS_LIB_PATH):
        pytest.skip("libkda_clocks.so is not built (build --phase-clocks)")
    announce("phase clocks --workload %s (child process)" % workload)
    r = subprocess.run([sys.executable, "-m", "linear_attention_prefill_amd.phase_clocks",
                        "--workload", workload], cwd=ROOT, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    rows = _rows(r.stdout, label)
    assert [w for w, *_ in rows] == list(range(8))
    for w, items, item, phases in rows:
        assert items >= 4
        assert all(p >= 0 for p in phases)
        assert 0 < sum(phases) <= item * 1.05, (w, item, phases)
    if workload == "packed":
        # the scan's workgroup 0 runs the longest sequence (37 chunks) of head 0
        rows = _rows(r.stdout, "state scan (steps of the longest chain)")
        assert [w for w, *_ in rows] == list(range(4))
        for w, items, step, phases in rows:
            assert items >= 30
            assert 0 < sum(phases) <= step * 1.05, (w, step, phases)
