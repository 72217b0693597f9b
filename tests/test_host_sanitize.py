"""The C ABI's argument validation and workspace arithmetic under
AddressSanitizer and UndefinedBehaviorSanitizer (host code only: the sanitizer
flags go to the host pass of each hipcc line; the gfx950 device code is built
as usual).  The driver in host_sanitize/abi_validation.cpp calls every entry
point with invalid problems, parameters, pointers and workspaces; every call
must fail (or size its workspace) before any HIP call, so no GPU is needed."""
import concurrent.futures as cf
import os
import subprocess

import pytest

from exact_top_token_amd import build as hkbuild

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(hkbuild.ROOT, "_build", "sanitize")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, "\n".join(l for l in p.stdout.splitlines() if "packed-fp32" not in l)


@pytest.mark.timeout(600)
def test_abi_validation_under_host_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    cc = hkbuild.hipcc()
    jobs, objs = [], []
    for src in hkbuild.SOURCES:
        obj = os.path.join(OUT, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([cc, *hkbuild.FLAGS, *SAN, "-O1", "-g", "-c", os.path.join(hkbuild.CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(min(len(jobs), 8)) as ex:
        list(ex.map(_compile, jobs))
    drv = os.path.join(OUT, "abi_validation.o")
    _compile([cc, "-x", "c++", *SAN, "-g", "-I", hkbuild.INCLUDE, "-c",
              os.path.join(HERE, "host_sanitize", "abi_validation.cpp"), "-o", drv])
    exe = os.path.join(OUT, "abi_validation")
    _compile([cc, f"--offload-arch={hkbuild.ARCH}", *SAN, drv, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                       timeout=120)
    print(p.stdout[-4000:])
    assert p.returncode == 0, p.stdout[-4000:]
    assert "ok: 0 failure(s)" in p.stdout
