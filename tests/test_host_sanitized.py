"""Host code of the library under AddressSanitizer + UBSan, no GPU: plan.cpp and
capi.cpp are rebuilt with the sanitizers on the host side only (-Xarch_host before each
-fsanitize=), linked with the library's other objects and a C driver that creates host
plans at several sizes and widths, reads their tables and exercises the validation
paths of every entry point."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "negacyclic_ntt_amd", "csrc")


def test_host_paths_under_sanitizers(tmp_path):
    if shutil.which("hipcc") is None or shutil.which("g++") is None:
        pytest.skip("no hipcc / g++")
    from negacyclic_ntt_amd import build as nb
    objs = {s: os.path.join(nb.BUILD, os.path.splitext(s)[0] + ".o") for s in nb.SOURCES}
    if not all(os.path.exists(objs[s]) for s in ("ntt.hip", "elementwise.hip", "keyswitch.hip")):
        nb.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    host_objs = []
    for src in ("plan.cpp", "capi.cpp"):
        obj = str(tmp_path / (src + ".san.o"))
        cmd = ["hipcc", *nb.FLAGS, "-g", *san, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        host_objs.append(obj)
    drv = str(tmp_path / "drv.o")
    r = subprocess.run(["gcc", "-std=c11", "-g", "-fsanitize=address,undefined", "-c",
                        os.path.join(ROOT, "tests", "native", "host_sanitize.c"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "host_sanitize")
    link = ["g++", "-fsanitize=address,undefined", drv, *host_objs,
            objs["ntt.hip"], objs["elementwise.hip"], objs["keyswitch.hip"],
            "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0, run.stdout + run.stderr[-3000:]
    assert "host sanitized run ok" in run.stdout
