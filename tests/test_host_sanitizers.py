"""The host half of the library under AddressSanitizer (with leak checking)
and UndefinedBehaviorSanitizer, and under ThreadSanitizer, on the CPU: the
planner and C ABI (``api.cpp``) and the coordinator (``coord.cpp``) are
rebuilt with the sanitizers on the host side only (the gfx950 kernels are
linked unchanged and never launched), then host-only drivers run against
them: ``host_fuzz.cpp`` (seeded random layouts, plans, coordinator sequences
and argument errors, on one thread and then on four threads at once) and
``c_abi_host.c``.  Any sanitizer report fails."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "zero_sharded_state_amd", "csrc")
INC = os.path.join(ROOT, "include")
# each sanitizer flag applies to the host compilation only
COMMON = "-Xarch_host -fno-omit-frame-pointer -g".split()
SAN = {
    "asan+ubsan": "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
                  + "-Xarch_host -fno-sanitize-recover=all".split() + COMMON,
    "tsan": "-Xarch_host -fsanitize=thread".split() + COMMON,
}


def _hipcc():
    return os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    assert r.returncode == 0, " ".join(cmd) + "\n" + out


_objects = {}


def _sanitized_objects(tmp_path_factory, kind):
    if kind in _objects:
        return _objects[kind]
    if not os.path.exists(_hipcc()):
        pytest.skip("no hipcc")
    from zero_sharded_state_amd import build as B
    d = tmp_path_factory.mktemp(kind.replace("+", "_"))
    flags = [f for f in B.HIP_FLAGS if f not in ("-O3", "-fvisibility=hidden")] + ["-O1"]
    objs = []
    for src in ("api.cpp", "coord.cpp"):
        o = str(d / (src + ".o"))
        _run([_hipcc(), "-x", "hip", *flags, *SAN[kind], "-I", INC, "-I", CSRC, "-c", os.path.join(CSRC, src),
              "-o", o])
        objs.append(o)
    kobj = os.path.join(B.BUILD_DIR, "kernels.o")
    if not os.path.exists(kobj):
        kobj = str(d / "kernels.o")
        _run([_hipcc(), *B.HIP_FLAGS, "-I", INC, "-I", CSRC, "-c", os.path.join(CSRC, "kernels.hip"), "-o", kobj])
    objs.append(kobj)
    _objects[kind] = (d, objs)
    return _objects[kind]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("kind,driver", [("asan+ubsan", "host_fuzz.cpp"), ("asan+ubsan", "c_abi_host.c"),
                                         ("tsan", "host_fuzz.cpp")])
def test_host_code_is_clean_under_sanitizers(tmp_path_factory, kind, driver):
    d, objs = _sanitized_objects(tmp_path_factory, kind)
    drv = str(d / (driver + ".o"))
    _run([_hipcc(), "-x", "c++", "-std=c++17", *SAN[kind], "-I", INC, "-c", os.path.join(HERE, driver), "-o", drv])
    exe = str(d / (driver + ".exe"))
    _run([_hipcc(), "--offload-arch=gfx950", *SAN[kind], *objs, drv, "-pthread", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    report = r.stdout + r.stderr
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), report[-4000:]
    for marker in ("ERROR: AddressSanitizer", "runtime error", "WARNING: ThreadSanitizer"):
        assert marker not in report, report[-4000:]
