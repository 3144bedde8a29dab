"""The C ABI from plain C: tests/c/plan_from_c.c is compiled with gcc as
C99 against include/fsattn.h, linked to libfsattn.so and run (host entry
points only, no GPU); its plan must equal the binding's element for
element."""
import os
import shutil
import subprocess

import pytest

import frame_block_sparse_amd as fs
from frame_block_sparse_amd import fsattn as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def plan_exe(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    fs.lib()   # raises if the library is not built
    exe = str(tmp_path_factory.mktemp("c_abi") / "plan_from_c")
    libdir = os.path.dirname(F.LIB_PATH)
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "plan_from_c.c"), "-o", exe, "-L", libdir, "-lfsattn",
           f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


@pytest.mark.parametrize("mask", [(5, 48, 1, 1, 0, 16, 16), (21, 960, 1, 1, 0, 80, 80), (6, 96, 2, 0, -1, 32, 48)])
def test_plan_from_plain_c_matches_binding(plan_exe, mask):
    r = subprocess.run([plan_exe, *map(str, mask)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.splitlines()
    assert lines[0] == f"abi {F.ABI_VERSION}"
    nqb, nnz = map(int, lines[1].split())
    rp, ci = fs.plan(mask)
    assert (nqb, nnz) == (rp.numel() - 1, ci.numel())
    assert [int(x) for x in lines[2].split()] == rp.tolist()
    assert [int(x) for x in lines[3].split()] == ci.tolist()
    assert lines[4] == "bad 2"
