"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc, CPU only) runs its
pins clean: every stored format through the decoders, the row products and the expert FFN, the
router (ties, k = E, k = 1), the permutation (including rejected indices), hash routing with
invalid ids, invalid entries and repeated experts, the MXFP8 and int8 quantisers on zero rows,
subnormals and saturating maxima, and whole layers. Any out-of-bounds access, use of freed
memory or undefined operation (an out-of-range float-to-int conversion, a signed overflow, a
shift past the width) aborts the run."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    return subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()


def test_oracle_pins_run_clean_under_asan_and_ubsan():
    env = dict(os.environ)
    env.update({
        "MOE_ORACLE_SANITIZE": "1",
        "LD_PRELOAD": _runtime("libasan.so") + ":" + _runtime("libubsan.so"),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "4",
    })
    build = subprocess.run([sys.executable, "-c", "from oracle import oracle as O; print(O.build())"],
                           cwd=ROOT, env={k: v for k, v in env.items() if k != "LD_PRELOAD"},
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    lib = build.stdout.strip()
    assert lib.endswith("libmoe_oracle_san.so")
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms  # the build is instrumented
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
