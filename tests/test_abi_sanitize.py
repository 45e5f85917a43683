"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Every library source is compiled with its host code instrumented (the device code is
compiled as usual) and linked with tests/sanitize/abi_driver.cpp, which sweeps validation
failures and workspace-size queries over the shapes the library serves and over extreme
sizes.  A sanitizer report, an unexpected status or two size queries that disagree fail
the test.  Built objects are kept under the package's _build/sanitize and rebuilt when a
source is newer."""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_attention_25_amd")
CSRC = os.path.join(PKG, "csrc")
INC = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "_build", "sanitize")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")
ROCM = "/opt/rocm"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _newer(target, sources):
    return os.path.exists(target) and all(os.path.getmtime(target) >= os.path.getmtime(s) for s in sources)


def _build():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not found")
    os.makedirs(OUT, exist_ok=True)
    headers = glob.glob(os.path.join(CSRC, "*.hpp")) + glob.glob(os.path.join(INC, "*.h"))
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "abi.cpp")]
    objs, procs = [], []
    for s in srcs:
        o = os.path.join(OUT, os.path.basename(s) + ".o")
        objs.append(o)
        if _newer(o, [s] + headers):
            continue
        lang = ["-x", "hip"] if s.endswith(".cpp") else []
        cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-mcode-object-version=5",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
               *HOST_SAN, *lang, "-I", INC, "-c", s, "-o", o]
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    for s, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, f"{os.path.basename(s)}:\n{out.decode(errors='replace')[-4000:]}"
    exe = os.path.join(OUT, "abi_driver")
    if not _newer(exe, objs + [DRIVER] + headers):
        d_obj = os.path.join(OUT, "abi_driver.o")
        subprocess.run([clang, "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", INC, "-I",
                        os.path.join(ROCM, "include"), "-c", DRIVER, "-o", d_obj], check=True)
        subprocess.run([clang, *SAN, d_obj, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                        f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe], check=True)
    return exe


@pytest.mark.timeout(900)
def test_abi_host_code_is_clean_under_asan_and_ubsan():
    exe = _build()
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=600)
    text = r.stdout + r.stderr
    if r.returncode == 77:
        pytest.skip(r.stdout.strip())
    assert "ERROR: AddressSanitizer" not in text and "runtime error:" not in text, text[-6000:]
    assert r.returncode == 0 and "ok: 0 failures" in r.stdout, text[-6000:]
    answered = int(r.stdout.rsplit(";", 1)[1].split()[0])
    assert answered > 10000, r.stdout       # the sweep reached the plans, not only the argument checks
