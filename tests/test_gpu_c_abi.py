"""libmbt called from plain C (tests/c_abi/abi_roundtrip.c): HIP-runtime
device buffers, no Python or PyTorch in the calling process, results checked
against the CPU oracle inside the program.  The program is built by
__graft_entry__.build() (and here if it is missing: one gcc line)."""
import importlib.util
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location("c_abi_build",
                                               os.path.join(HERE, "c_abi", "build.py"))
c_abi_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(c_abi_build)


def test_c_abi_program_builds(tmp_path):
    # the C caller compiles and links against the library and the oracle
    exe = c_abi_build.build(str(tmp_path / "abi_roundtrip"))
    assert os.path.exists(exe)


@pytest.mark.gpu
def test_c_abi_roundtrip():
    exe = c_abi_build.EXE
    if not os.path.exists(exe):
        c_abi_build.build()
    print("c abi round trip:", exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "every check passed" in r.stdout
