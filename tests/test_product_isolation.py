"""The oracle is test infrastructure: the product path never imports it.

* nothing under ``zero_sharded_state_amd/`` or ``synth/`` imports ``oracle``;
* in ``bench.py`` only the CPU-baseline leg (``cpu_baseline``,
  ``cpu_baseline_coordinator``) does;
* the oracle imports nothing of the HIP path (``zero_sharded_state_amd``).
"""

import ast
import glob
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _imports(tree):
    """(module name, enclosing top-level function or None) of every import."""
    out = []
    for top in tree.body:
        fn = top.name if isinstance(top, (ast.FunctionDef, ast.AsyncFunctionDef)) else None
        for node in ast.walk(top):
            if isinstance(node, ast.Import):
                out += [(a.name, fn) for a in node.names]
            elif isinstance(node, ast.ImportFrom) and node.module:
                out.append((node.module, fn))
    return out


def _parse(path):
    with open(path, encoding="utf-8") as fh:
        return ast.parse(fh.read(), path)


def test_library_and_inputs_never_import_the_oracle():
    files = glob.glob(os.path.join(ROOT, "zero_sharded_state_amd", "**", "*.py"), recursive=True)
    files += glob.glob(os.path.join(ROOT, "synth", "**", "*.py"), recursive=True)
    assert files
    for f in files:
        bad = [m for m, _ in _imports(_parse(f)) if m == "oracle" or m.startswith("oracle.")]
        assert not bad, f"{f} imports {bad}"


def test_bench_uses_the_oracle_only_in_its_cpu_baseline_leg():
    uses = {fn for m, fn in _imports(_parse(os.path.join(ROOT, "bench.py")))
            if m == "oracle" or m.startswith("oracle.")}
    assert uses <= {"cpu_baseline", "cpu_baseline_coordinator"}, uses


def test_oracle_imports_nothing_of_the_hip_path():
    for f in glob.glob(os.path.join(ROOT, "oracle", "**", "*.py"), recursive=True):
        bad = [m for m, _ in _imports(_parse(f)) if m.startswith("zero_sharded_state_amd")]
        assert not bad, f"{f} imports {bad}"
