"""The C ABI from C: ``include/zs3.h`` compiles as C99 (and as C++17) with
warnings as errors, links against libzs3.so, and a plain C caller of the
host-only entry points (layout, bucket and sub-group planning, the
coordinator, error reporting) gets the toy model's values (no GPU needed).
On a GPU, a C caller with hipMalloc'd buffers and no Python in the process
runs partition, gather and reduce-scatter and checks them against their
definitions."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "zero_sharded_state_amd")
LIB = os.path.join(PKG, "libzs3.so")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
@pytest.mark.parametrize("lang", ["c99", "c++17"])
def test_c_caller_of_the_host_entry_points(tmp_path, lang):
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built")
    exe = str(tmp_path / "c_abi_host")
    if lang == "c99":
        cmd = ["gcc", "-std=c99", "-pedantic"]
    else:
        cmd = ["g++", "-std=c++17", "-x", "c++"]
    cmd += ["-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi_host.c")]
    cmd += ["-x", "none", "-L", PKG, "-lzs3", f"-Wl,-rpath,{PKG}", "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


@pytest.mark.gpu
@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_c_caller_of_the_device_entry_points(tmp_path):
    from gpu_util import note, require_gpu
    require_gpu()
    exe = str(tmp_path / "c_abi_device")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
           os.path.join(HERE, "c_abi_device.c"), "-L", PKG, "-lzs3", f"-Wl,-rpath,{PKG}",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-lm", "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr
    note("c_abi_device: partition, gathers, reduce-scatter, norm, master, Adam from C")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
