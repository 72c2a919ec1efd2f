import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # A mistake planted in the oracle (tests/oracle_mutations.py), for the
    # check that the pins catch it; never set in a normal run.
    name = os.environ.get("FP8PA_ORACLE_MUTATION")
    if name:
        from tests.oracle_mutations import apply

        apply(name)
