"""The C ABI's host-side argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).  Every library source is compiled
with both sanitizers on its host code only (device code is not instrumented),
and linked with
tests/sanitize/abi_check.cpp, which walks the rejection paths of every entry
point (and, with no device present, the device check).  A sanitizer report
fails the run.  Device code is not involved: GPU sanitizers are not used."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from dit_joint_self_amd import build as B  # noqa: E402

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _no_device():
    import torch
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="no hipcc")
def test_abi_checks_clean_under_host_sanitizers(tmp_path):
    cc = B.hipcc()
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Wno-unused-command-line-argument",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", B.INCLUDE, "-I", B.CSRC] + HOST_SAN
    objs, procs = [], []
    for src in B.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([cc, *flags, "-c", os.path.join(B.CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p, src in zip(procs, B.SOURCES):
        out = p.communicate()[0]
        assert p.returncode == 0, f"{src}: {out[-3000:]}"
    main_obj = str(tmp_path / "abi_check.o")
    r = subprocess.run([cc, *flags, "-c", os.path.join(ROOT, "tests", "sanitize", "abi_check.cpp"), "-o", main_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    # Host link with clang's sanitizer runtimes (device code is not instrumented).
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(cc)))
    clang = os.path.join(rocm, "lib", "llvm", "bin", "clang++")
    exe = str(tmp_path / "abi_check")
    r = subprocess.run([clang, "--hip-link", "-Xarch_host", "-fsanitize=address,undefined", main_obj, *objs,
                        "-L", os.path.join(rocm, "lib"),
                        "-Wl,-rpath," + os.path.join(rocm, "lib"), "-lamdhip64", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    args = [exe] + (["--no-device"] if _no_device() else [])
    r = subprocess.run(args, capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout[-4000:], r.stderr[-4000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0 and "0 failure(s)" in r.stdout, r.stdout[-4000:] + r.stderr[-4000:]
