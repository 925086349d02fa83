"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle.c is rebuilt with both sanitizers (every report fatal) and the whole
pin suite runs against that build in a child process with the sanitizer
runtimes preloaded, so an out-of-bounds access, a signed overflow or a bad
shift anywhere the pins reach fails the test.  The GPU path is not involved.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


SAN_FLAGS = ["-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _env(asan, ubsan):
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{asan}:{ubsan}"
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=24"
    return env


def test_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    # the set-up reports a planted heap overflow (so a clean run means something)
    bad = tmp_path / "planted.c"
    bad.write_text("#include <stdlib.h>\nint planted(int i) { int* p = malloc(4 * sizeof(int));"
                   " int v = p[i]; free(p); return v; }\n")
    bad_so = tmp_path / "libplanted.so"
    subprocess.run(["gcc", *SAN_FLAGS, "-o", str(bad_so), str(bad)], check=True)
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({str(bad_so)!r}).planted(4)"],
                       env=_env(asan, ubsan), capture_output=True, text=True, timeout=120)
    caught = ((r.returncode == 23 and "heap-buffer-overflow" in r.stderr) or
              (r.returncode == 24 and "runtime error" in r.stderr))
    assert caught, (r.returncode, r.stderr[-2000:])

    so = tmp_path / "liboracle_san.so"
    src = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
    subprocess.run(["gcc", *SAN_FLAGS, "-o", str(so), src], check=True)
    script = (
        "import sys\n"
        f"sys.path.insert(0, {ROOT!r})\n"
        "import oracle\n"
        f"oracle._lib = oracle.load_library({str(so)!r})\n"
        "from tests import oracle_pins\n"
        "for pin in oracle_pins.ALL_PINS:\n"
        "    pin()\n"
        "    print('ok', pin.__name__, flush=True)\n")
    r = subprocess.run([sys.executable, "-c", script], env=_env(asan, ubsan), capture_output=True, text=True,
                       timeout=900, cwd=ROOT)
    done = r.stdout.count("\nok ") + r.stdout.startswith("ok ")
    assert r.returncode == 0, (f"exit {r.returncode} after {done} pins\n"
                               + r.stdout[-2000:] + r.stderr[-6000:])
    from tests import oracle_pins
    assert done == len(oracle_pins.ALL_PINS)
