import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Per-case parity counts of the session: units whose selection equals the
    oracle's exactly, units that differ only between near-equal oracle scores
    (accepted), failures, units whose selection was replayed bit for bit on the
    GPU's own scores, and the largest relative score error seen."""
    try:
        from parity import TALLY
    except Exception:
        return
    if not TALLY:
        return
    import json
    w = terminalreporter
    w.write_sep("-", "parity counts (exact / near-tie accepted / failed; replayed bit-exact; max score rel err)")
    for case, t in sorted(TALLY.items()):
        w.write_line(f"{case}: exact {t['exact']}, near-tie {t['near_tie']}, failed {t['fail']}; "
                     f"replayed {t['replayed_bit_exact']}; max rel err {t['max_score_rel_err']:.3g}")
    path = os.environ.get("KARA_PARITY_REPORT")
    if path:
        with open(path, "w") as f:
            json.dump(TALLY, f, indent=1, sort_keys=True)
