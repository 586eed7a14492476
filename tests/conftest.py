import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes)")


def pytest_terminal_summary(terminalreporter):
    """Report the top-k selection near ties the GPU parity tests met."""
    mod = sys.modules.get("parity_util")
    if mod is None or not mod.TALLY["heads"]:
        return
    t = mod.TALLY
    terminalreporter.write_line(
        f"top-k selection near ties (within {mod.NEAR_TIE_REL:g} relative of the budget-th "
        f"key): {t['near_tie_pages']} pages on {t['heads_with_near_ties']} of {t['heads']} "
        f"checked heads; GPU and oracle selections differ on {t['differing_pages']} pages "
        f"({t['heads_differing']} heads)")
