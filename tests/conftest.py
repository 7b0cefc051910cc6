import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle runs of a minute or more")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Every parity gate's result, near ties included, also under ``pytest -q`` (which hides the
    tests' own output). The totals line comes last so that it survives in a tail of the log."""
    try:
        from parity_util import SUMMARIES
    except Exception:                                   # parity_util not importable: nothing ran
        return
    if not SUMMARIES:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity gates (GPU vs oracle)")
    for s in SUMMARIES:
        tie = f" near_tie_pos={s['near_tie_pos'][:8]}" if s["near_ties"] else ""
        tr.write_line(f"gate {s['name']}: positions={s['positions']} worst_nmse={s['worst_nmse']:.2e} "
                      f"(pos {s['worst_pos']}) mismatches={s['mismatches']} near_ties={s['near_ties']}{tie}")
    worst = max(SUMMARIES, key=lambda s: s["worst_nmse"])
    tr.write_line(f"gate totals: gates={len(SUMMARIES)} positions={sum(s['positions'] for s in SUMMARIES)} "
                  f"worst_nmse={worst['worst_nmse']:.2e} ({worst['name']}) "
                  f"mismatches={sum(s['mismatches'] for s in SUMMARIES)} "
                  f"near_ties={sum(s['near_ties'] for s in SUMMARIES)}")
    out = os.path.join(ROOT, "gpurun_out")
    try:
        os.makedirs(out, exist_ok=True)
        with open(os.path.join(out, "gate_summary.json"), "w") as f:
            json.dump(SUMMARIES, f, indent=1)
    except OSError:
        pass
