"""The CPU-side C and C++ code under AddressSanitizer and UBSan: the oracle,
the seeded input generator and the multi-threaded host-CPU pass are rebuilt
with -fsanitize=address,undefined (no recovery) and the oracle pins, the
oracle variant tests, the generator tests and the CPU-pass tests run against
those builds in a child process (the ASan runtime preloaded, as a library
loaded into Python needs).  Any sanitizer report fails the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all", "-fPIC", "-shared", "-Wall"]
TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_variants.py",
         "tests/test_oracle_codec_variants.py", "tests/test_oracle_matmul.py",
         "tests/test_synth.py", "tests/test_cpu_pass.py"]


def _asan_runtime() -> str:
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                       check=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    return p


def _env(d):
    env = dict(os.environ)
    env.update({
        "NF4_SANITIZED_DIR": str(d),
        "PYTHONPATH": os.pathsep.join([os.path.join(ROOT, "tests"), ROOT]),
        "LD_PRELOAD": _asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    return env


def _build(d):
    inc = ["-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROOT, "quantized_lora_fine_nf4_amd", "csrc")]
    cmds = [
        ["gcc", *SAN, "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-o",
         str(d / "liboracle_nf4.so"), os.path.join(ROOT, "oracle", "nf4_oracle.c"), "-lm"],
        ["gcc", *SAN, "-std=c11", "-fopenmp", "-o", str(d / "libsynth.so"),
         os.path.join(ROOT, "synth", "synth.c"), "-lm"],
        ["g++", *SAN, "-std=c++17", "-march=x86-64-v3", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", *inc, "-o", str(d / "libnf4cpu.so"),
         os.path.join(ROOT, "quantized_lora_fine_nf4_amd", "cpu", "nf4_cpu.cpp")],
    ]
    for c in cmds:
        r = subprocess.run(c, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_sanitizer_build_reports_a_planted_overflow(tmp_path):
    """The toolchain set-up itself: the same flags and runtime catch a heap
    overflow planted in a throwaway C file (not in any product code)."""
    src = tmp_path / "planted.c"
    src.write_text("#include <stdlib.h>\n"
                   "int planted(int i) { int* p = (int*)malloc(4 * sizeof(int));"
                   " p[0] = 1; int v = p[i]; free(p); return v; }\n")
    lib = tmp_path / "libplanted.so"
    r = subprocess.run(["gcc", *SAN, "-o", str(lib), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    code = (f"import ctypes; L = ctypes.CDLL({str(lib)!r}); L.planted.restype = ctypes.c_int; "
            "L.planted(0); print('in bounds ok', flush=True); L.planted(4)")
    r = subprocess.run([sys.executable, "-c", code], env=_env(tmp_path), capture_output=True,
                       text=True, timeout=120)
    assert "in bounds ok" in r.stdout
    # UBSan's object-size check or ASan's shadow memory, whichever reports first
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr or "runtime error" in r.stderr, r.stderr[-2000:]


def test_cpu_code_is_clean_under_asan_and_ubsan(tmp_path):
    _build(tmp_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-p", "sanitized_libs", "-q", "-x",
                        "-p", "no:cacheprovider", *TESTS],
                       cwd=ROOT, env=_env(tmp_path), capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    mapped = [l for l in r.stdout.splitlines() if l.startswith("[sanitized-libs-mapped]")]
    assert mapped, out[-2000:]
    for name in ("liboracle_nf4.so", "libsynth.so", "libnf4cpu.so"):
        assert os.path.join(str(tmp_path), name) in mapped[-1], mapped[-1]
