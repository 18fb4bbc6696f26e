import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# test_oracle_mutants.py runs the oracle pins against altered copies of the
# oracle package placed in this directory
_ORACLE_UNDER_TEST = os.environ.get("LA_ORACLE_UNDER_TEST")
if _ORACLE_UNDER_TEST:
    sys.path.insert(0, _ORACLE_UNDER_TEST)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU check")


def pytest_terminal_summary(terminalreporter):
    helpers = sys.modules.get("gpu_helpers")
    if helpers is not None and helpers.WORST_ROW["where"]:
        w = helpers.WORST_ROW
        terminalreporter.write_line(f"worst per-row relative error in the GPU parity checks: {w['err']:.3e} "
                                    f"({w['where']})")
        terminalreporter.write_line("worst per-row relative error by check site:")
        for site, (err, detail) in sorted(helpers.WORST_BY_SITE.items(), key=lambda kv: -kv[1][0]):
            terminalreporter.write_line(f"  {err:.3e}  {site}  {detail}")
