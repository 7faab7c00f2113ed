"""The CPU oracle and the host shard-layout planner under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/sanitize/sanitize_driver.cpp is built with
the two sources (gcc/g++, host code only, no GPU code) and run on a few
hundred random layouts; any memory error, undefined behaviour or failed check
ends it with a non-zero status.

Command (from the repository root; OUT is any scratch folder):
    gcc -std=c11 $FLAGS -c oracle/tide_oracle.c -o $OUT/oracle.o
    g++ -std=c++17 $FLAGS -I include -I param_collectives_amd/csrc -c param_collectives_amd/csrc/plan.cpp -o $OUT/plan.o
    g++ -std=c++17 $FLAGS -I include -I param_collectives_amd/csrc -c tests/sanitize/sanitize_driver.cpp -o $OUT/driver.o
    g++ $FLAGS $OUT/oracle.o $OUT/plan.o $OUT/driver.o -o $OUT/driver && $OUT/driver 300
with FLAGS = -O1 -g -fno-omit-frame-pointer -ffp-contract=off -pthread -fsanitize=address,undefined
-fno-sanitize-recover=all.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-pthread",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _build(out):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "param_collectives_amd", "csrc")]
    steps = [
        ["gcc", "-std=c11", *FLAGS, "-c", os.path.join(ROOT, "oracle", "tide_oracle.c"), "-o", f"{out}/oracle.o"],
        ["g++", "-std=c++17", *FLAGS, *inc, "-c", os.path.join(ROOT, "param_collectives_amd", "csrc", "plan.cpp"),
         "-o", f"{out}/plan.o"],
        ["g++", "-std=c++17", *FLAGS, *inc, "-c", os.path.join(ROOT, "tests", "sanitize", "sanitize_driver.cpp"),
         "-o", f"{out}/driver.o"],
        ["g++", *FLAGS, f"{out}/oracle.o", f"{out}/plan.o", f"{out}/driver.o", "-o", f"{out}/driver"],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, (" ".join(cmd), r.stderr[-3000:])
    return f"{out}/driver"


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="needs gcc and g++")
def test_oracle_and_planner_clean_under_sanitizers(tmp_path):
    driver = _build(str(tmp_path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver, "300"], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, r.stderr[-5000:]
    assert "300 cases clean" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
