import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
# tests/test_oracle_mutations.py runs the oracle's pin tests against a mutated copy of the
# oracle package: that copy's parent directory then comes first on the import path
_MUTANT = os.environ.get("ORACLE_MUTANT_DIR")
if _MUTANT:
    sys.path.insert(0, _MUTANT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
