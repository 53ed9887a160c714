"""Host code under the address and undefined-behaviour sanitizers (CPU only):

* the library's packing loops (bit_linear_dynamic_amd/csrc/h3q_layout.hpp, the code h3q_pack_weight and
  h3q_register_adapter run on the host) in a host-only program that packs ragged plain and gate/up
  shapes and reads every element back through the layout (tests/host_layout_check.cpp);
* the fp64 oracle (oracle/oracle.cpp) built with the sanitizers and run through every pin.
Any out-of-bounds access, use after free or undefined behaviour aborts the run (no recovery)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _gxx_has_sanitizers(tmp_path) -> bool:
    src = tmp_path / "probe.cpp"
    src.write_text("int main() { return 0; }\n")
    r = subprocess.run(["g++", *SAN, str(src), "-o", str(tmp_path / "probe")], capture_output=True)
    return r.returncode == 0


def test_packing_loops_under_sanitizers(tmp_path):
    if not _gxx_has_sanitizers(tmp_path):
        pytest.skip("g++ has no sanitizer runtimes here")
    exe = tmp_path / "host_layout_check"
    subprocess.run(["g++", "-std=c++17", "-O1", *SAN, os.path.join(ROOT, "tests", "host_layout_check.cpp"),
                    "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.strip().endswith("ok")


def test_oracle_pins_under_sanitizers(tmp_path):
    if not _gxx_has_sanitizers(tmp_path):
        pytest.skip("g++ has no sanitizer runtimes here")
    import oracle
    lib = str(tmp_path / "liboracle_san.so")
    src = os.path.join(ROOT, "oracle", "oracle.cpp")
    subprocess.run(["g++", "-O1", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c++17",
                    *SAN, src, "-o", lib], check=True, capture_output=True)
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import oracle, pins\n"
            "lib = oracle.load(%r)\n"
            "for pin in pins.ALL_PINS:\n"
            "    pin(lib)\n"
            "print('pins', len(pins.ALL_PINS))\n") % (ROOT, os.path.join(ROOT, "tests"), lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-6000:]
    assert r.stdout.strip().startswith("pins")
    assert oracle  # the module loads its default library as usual outside this subprocess
