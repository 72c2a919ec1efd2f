"""Every plausible oracle mistake of tests/oracle_mutations.py fails a pin.

Each mistake is planted in a copy of the oracle inside a fresh pytest
process that runs the pin files of the part it touches; that run must
report failing tests.  A control run with the oracle as it is must pass.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from tests.oracle_mutations import MUTATIONS, ROOT


def _run_pins(mutation, files):
    env = dict(os.environ)
    env.pop("FP8PA_ORACLE_MUTATION", None)
    if mutation:
        env["FP8PA_ORACLE_MUTATION"] = mutation
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
           "-p", "no:randomly", *files]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:] + r.stderr[-2000:]


def test_every_planted_mistake_fails_a_pin():
    jobs = [(None, ("tests/test_oracle.py", "tests/test_writer_oracle.py", "tests/test_nvfp4_oracle.py",
                    "tests/test_mxfp8_oracle.py"))]
    jobs += [(name, m[3]) for name, m in MUTATIONS.items()]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        results = list(pool.map(lambda j: (j[0], *_run_pins(*j)), jobs))
    control = results[0]
    assert control[1] == 0, f"pins fail on the oracle as it is:\n{control[2]}"
    survived = []
    for name, rc, tail in results[1:]:
        # exit code 1: tests ran and some failed; anything else (2: an error
        # while collecting, e.g. a snippet that no longer matches) is a
        # broken harness, not a caught mistake
        if rc != 1 or "failed" not in tail:
            survived.append((name, rc, tail))
    assert not survived, "mistakes no pin catches (or harness errors):\n" + "\n\n".join(
        f"{n} (exit {rc}):\n{t}" for n, rc, t in survived)
