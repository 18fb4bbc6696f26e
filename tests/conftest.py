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
