"""The C-ABI layer (santa_api.cpp) built for the host alone with the address
and undefined-behaviour sanitizers, its kernel launchers replaced by stubs
(tests/host_stubs.cpp): the plain C consumer (tests/c_consumer.c), every
entry point on valid arguments (tests/c_launch_paths.c), and the ABI tests
of tests/test_abi_host.py run against it. Any sanitizer report fails the
test. No GPU and no HIP runtime are involved."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
API = os.path.join(ROOT, "sampled_sparse_decode_amd", "csrc", "santa_api.cpp")
STUBS = os.path.join(ROOT, "tests", "host_stubs.cpp")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = {"ASAN_OPTIONS": "halt_on_error=1:detect_leaks=1:abort_on_error=0",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="gcc/g++ not available")


def _objects(tmp_path, pic=False):
    objs = []
    for src in (API, STUBS):
        obj = tmp_path / (os.path.basename(src) + ".o")
        subprocess.run(["g++", "-std=c++17", "-Wall", *SAN, *(["-fPIC"] if pic else []),
                        "-I", os.path.join(ROOT, "include"), "-c", src, "-o", str(obj)], check=True)
        objs.append(str(obj))
    return objs


def _run(cmd, env_extra=None):
    env = dict(os.environ)
    env.update(ENV)
    env.update(env_extra or {})
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600, env=env)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    return out


@pytest.mark.parametrize("driver", ["c_consumer.c", "c_launch_paths.c"])
def test_c_drivers_under_sanitizers(tmp_path, driver):
    objs = _objects(tmp_path)
    exe = tmp_path / driver.replace(".c", "")
    cobj = tmp_path / (driver + ".o")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", *SAN,
                    "-I", os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", driver),
                    "-o", str(cobj)], check=True)
    subprocess.run(["g++", *SAN, str(cobj), *objs, "-o", str(exe)], check=True)
    out = _run([str(exe)])
    assert " ok" in out


def test_abi_tests_under_sanitizers(tmp_path):
    """tests/test_abi_host.py against the sanitized host build, the
    sanitizer runtime preloaded into a child interpreter. Never displaces a
    preload the environment already has."""
    if os.environ.get("LD_PRELOAD") or os.path.exists("/etc/ld.so.preload"):
        pytest.skip("a preload is configured; the sanitizer runtime is not added to it")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan.so not found")
    objs = _objects(tmp_path, pic=True)
    so = tmp_path / "libsanta_host_sanitized.so"
    subprocess.run(["g++", "-shared", *SAN, *objs, "-o", str(so)], check=True)
    out = _run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"), "-q",
                "-p", "no:cacheprovider", "-k", "not c_consumer"],
               {"LD_PRELOAD": asan, "SANTA_TEST_LIB": str(so),
                "ASAN_OPTIONS": "halt_on_error=1:detect_leaks=0"})
    assert " passed" in out and " failed" not in out
