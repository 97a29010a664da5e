"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The oracle is rebuilt with -fsanitize=address,undefined (no recovery), and
every pin of tests/pins.py runs against that build in a child interpreter
with the ASan runtime preloaded (the interpreter itself is not
instrumented).  An out-of-bounds access, a use of an uninitialised shift, a
signed overflow or any other undefined behaviour in the oracle aborts the
child, and the test fails with its report.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
import pins
orc = oracle.Oracle({lib!r})
for pin in pins.ALL_PINS:
    pin(orc)
    print("ok", pin.__name__, flush=True)
"""


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime is not installed")
def test_pins_under_sanitizers(tmp_path):
    lib = obuild.build(out=str(tmp_path / "liboracle_asan.so"),
                       extra=("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                              "-fno-omit-frame-pointer", "-g"))
    env = dict(os.environ)
    env["LD_PRELOAD"] = _runtime("libasan.so")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = CHILD.format(root=ROOT, tests=HERE, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=900)
    report = (r.stdout[-2000:] + "\n" + r.stderr[-6000:]).strip()
    assert r.returncode == 0, f"sanitized oracle run failed (rc {r.returncode}):\n{report}"
    assert r.stdout.count("ok ") == len(__import__("pins").ALL_PINS), report
