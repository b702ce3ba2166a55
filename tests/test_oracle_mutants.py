"""The oracle's pins bite: each planted mistake in the oracle
(``oracle_mutants.py``: off-by-ones, dropped terms, swapped constants, wrong
orders, strides and transposes in ``oracle.zero3``; wrong limits, marks,
distances and hashes in ``oracle.coordinator``; on the CPU only) must make
the oracle's own pin tests fail, and the unmodified oracle must pass them.

Every run is a separate pytest process over the oracle pin files with
``ZS3_ORACLE_MUTANT`` set; hypothesis runs derandomized and without
shrinking there, so a failure is found quickly and reproducibly.
"""

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle_mutants import COORD_MUTANTS, MUTANTS

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
COORD_PINS = [os.path.join(HERE, "test_oracle_coordinator.py")]
PIN_FILES = sorted(f for f in glob.glob(os.path.join(HERE, "test_oracle_*.py"))
                   if not f.endswith("test_oracle_mutants.py") and f not in COORD_PINS)


def _run(name):
    env = {k: v for k, v in os.environ.items() if k != "ZS3_ORACLE_MUTANT"}
    if name is not None:
        env["ZS3_ORACLE_MUTANT"] = name
    files = COORD_PINS if name in COORD_MUTANTS else PIN_FILES + (COORD_PINS if name is None else [])
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        *files], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return name, r.returncode, (r.stdout + r.stderr)[-1500:]


@pytest.mark.timeout(1800)
def test_every_planted_oracle_mistake_fails_a_pin():
    workers = max(1, min(4, (os.cpu_count() or 2) // 2))
    with ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(_run, [None] + sorted(MUTANTS)))
    name, rc, out = results[0]
    assert rc == 0, f"unmodified oracle fails its pins:\n{out}"
    survivors = [(n, rc, out) for n, rc, out in results[1:] if rc != 1]
    assert not survivors, "mutants not caught (pytest exit code 1 expected):\n" + "\n".join(
        f"--- {n}: exit {rc}\n{out}" for n, rc, out in survivors)
