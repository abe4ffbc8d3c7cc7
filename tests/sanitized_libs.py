"""pytest plugin for the sanitizer run (loaded with `-p sanitized_libs` by
tests/test_sanitizers.py in a child process): points the oracle, the input
generator and the host-CPU pass at the AddressSanitizer + UBSan builds in
$NF4_SANITIZED_DIR before any test loads a library, and at the end prints
which shared objects of those three the process actually mapped."""
import os


def pytest_configure(config):
    d = os.environ["NF4_SANITIZED_DIR"]
    import oracle
    import synth
    from quantized_lora_fine_nf4_amd import cpu
    oracle.LIB_PATH = os.path.join(d, "liboracle_nf4.so")
    synth.LIB_PATH = os.path.join(d, "libsynth.so")
    cpu.LIB_PATH = os.path.join(d, "libnf4cpu.so")


def pytest_sessionfinish(session, exitstatus):
    names = ("liboracle_nf4.so", "libsynth.so", "libnf4cpu.so")
    mapped = set()
    with open("/proc/self/maps") as fh:
        for line in fh:
            path = line.split()[-1] if line.strip() else ""
            if os.path.basename(path) in names:
                mapped.add(path)
    print("\n[sanitized-libs-mapped]", " ".join(sorted(mapped)), flush=True)
