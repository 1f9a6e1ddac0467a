"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle (oracle/q8ref.c) and the C ABI's host side (api.cpp: argument
checks, aliasing checks, dispatch; plan.cpp: work decomposition and workspace
layouts) are built with gcc / g++ -fsanitize=address,undefined (host code
only: no HIP compiler is involved, and the kernel launchers and the HIP
runtime's device queries are replaced by stand-ins that report no device, as
on a machine without a GPU).  The CPU test suite then runs against those
builds in a child process with the sanitizer runtime preloaded; any
sanitizer report fails it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_q8_amd", "csrc")


def _run(cmd, **kw):
    out = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert out.returncode == 0, " ".join(cmd) + "\n" + out.stdout[-4000:] + out.stderr[-4000:]
    return out


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    from decode_q8_amd import build
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
    oracle_so = str(tmp_path / "libq8ref_san.so")
    _run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", *san,
          os.path.join(ROOT, "oracle", "q8ref.c"), "-o", oracle_so, "-lm", "-lpthread"])
    rocm_inc = "/opt/rocm/include"
    objs = []
    for src in ("api.cpp", "plan.cpp", os.path.join(ROOT, "tests", "sanitize", "no_device.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(["g++", "-O1", "-std=c++17", "-fPIC", *san, "-D__HIP_PLATFORM_AMD__",
              f'-DQ8_BUILD_DIGEST="{build.source_digest()}"', "-I", rocm_inc, "-I", os.path.join(ROOT, "include"),
              "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    abi_so = str(tmp_path / "libq8_san.so")
    _run(["g++", "-shared", "-fPIC", *san, *objs, "-o", abi_so])

    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": f"{asan}:{ubsan}",
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1:exitcode=87",
        "Q8_LIB": abi_so, "Q8REF_LIB": oracle_so,
    })
    # the child maps the sanitized builds, not the regular ones
    probe = ("import oracle\nfrom decode_q8_amd import q8\noracle.lib(); q8.lib()\n"
             "maps = open('/proc/self/maps').read()\n"
             "print('san' if 'libq8_san.so' in maps and 'libq8ref_san.so' in maps and 'libq8.so' not in maps "
             "and 'libq8ref.so' not in maps else 'regular')\n")
    out = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True)
    assert out.stdout.strip().endswith("san"), out.stdout + out.stderr
    # and the runtime reports a real error (an out-of-bounds write in a
    # throwaway program, not in the oracle)
    bad = tmp_path / "oob.c"
    bad.write_text("#include <stdlib.h>\nint main(void){int *p = malloc(4 * sizeof(int)); p[4] = 1; "
                   "free(p); return 0;}\n")
    _run(["gcc", *san, str(bad), "-o", str(tmp_path / "oob")])
    out = subprocess.run([str(tmp_path / "oob")], capture_output=True, text=True, env=env)
    assert out.returncode != 0 and "heap-buffer-overflow" in out.stderr

    tests = sorted(os.path.join("tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                   if f.startswith(("test_oracle_", "test_abi")) and f.endswith(".py"))
    out = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                          *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    log = out.stdout[-6000:] + out.stderr[-6000:]
    assert "ERROR: AddressSanitizer" not in log and "runtime error:" not in log, log
    assert out.returncode == 0, log
    assert " passed" in out.stdout, log
