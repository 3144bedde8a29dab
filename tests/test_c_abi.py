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


def _build_path_exe(out_dir):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = os.path.join(out_dir, "path_from_c")
    libdir = os.path.dirname(F.LIB_PATH)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [gcc, "-std=c99", "-Wall", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-isystem", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "path_from_c.c"), "-o", exe,
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-L", libdir, "-lfsattn", "-lm",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_whole_path_driver_builds_from_plain_c(tmp_path):
    """The GPU driver below compiles and links as C99 (it is run by the GPU
    test)."""
    fs.lib()
    assert os.path.exists(_build_path_exe(str(tmp_path)))


@pytest.mark.gpu
def test_whole_path_from_plain_c(tmp_path):
    """tests/c/path_from_c.c runs the device plan, the head bounds and the
    forward through the C ABI with the HIP runtime's C API only, in a process
    of its own, on inputs from the shared generators written as bf16 bit
    patterns; its O and records are checked against the oracle."""
    import numpy as np
    import torch
    import oracle
    import workloads
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = _build_path_exe(str(tmp_path))
    w = workloads.make_workload("c_path", 2, 3, 4, 96, 128, "bf16", 1, 1, 0, 48, 32)
    q, k, v = workloads.make_inputs(w, seed=12)
    for name, x in (("q", q), ("k", k), ("v", v)):
        (np.ascontiguousarray(x).view(np.uint32) >> 16).astype(np.uint16).tofile(str(tmp_path / f"{name}.bin"))
    args = [w.batch, w.heads, w.num_frames, w.tokens_per_frame, w.head_dim, w.window_before, w.window_after,
            w.ref_frame, w.block_q, w.block_k]
    print(f"[c-path] {exe} {args}", flush=True)
    r = subprocess.run([exe, str(tmp_path), *map(str, args)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    o = (np.fromfile(str(tmp_path / "o.bin"), dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    o = o.reshape(q.shape)
    g = oracle.MaskGeometry(*w.mask_tuple())
    ref, _ = oracle.attention_ref(q, k, v, g)
    assert np.abs(o - ref).max() <= 2e-2
    rec = np.fromfile(str(tmp_path / "rec.bin"), dtype=np.float32).reshape(w.batch, w.heads, 8)
    rb = oracle.head_bounds_ref(q, k, g)
    np.testing.assert_allclose(rec[..., 0], rb["q_max"], rtol=1e-5)
    np.testing.assert_allclose(rec[..., 1], rb["k_max"], rtol=1e-5)
    np.testing.assert_allclose(rec[..., 4], rb["gap_est"], rtol=1e-5)
    assert np.array_equal(rec[..., 5].view(np.int32).astype(bool), rb["eligible"])
