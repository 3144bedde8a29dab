"""C-ABI tests that need no GPU: the library loads, exports every declared
symbol, plans bit-exactly like the oracle, and rejects bad arguments on the
host before any launch (no compute call is made here)."""
import ctypes
import subprocess

import numpy as np
import pytest

import frame_block_sparse_amd as fs
from frame_block_sparse_amd import fsattn as F
import oracle
import workloads


def test_library_loads_and_exports_every_declared_symbol():
    L = fs.lib()
    names = F.declared_functions()
    assert {"fsattn_plan", "fsattn_head_bounds", "fsattn_forward"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", F.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
    assert fs.abi_version() == F.ABI_VERSION == 3


def test_struct_layouts():
    assert ctypes.sizeof(F.Mask) == 36
    assert ctypes.sizeof(F.Shape) == 20
    assert ctypes.sizeof(F.Tensor) == 32
    assert ctypes.sizeof(F.HeadBound) == 32


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_plan_bit_exact_vs_oracle_on_workloads(i):
    w = workloads.workload(i)
    rp, ci = fs.plan(w)
    orp, oci = oracle.plan_bruteforce(oracle.MaskGeometry(*w.mask_tuple()))
    assert np.array_equal(rp.numpy(), orp)
    assert np.array_equal(ci.numpy(), oci)
    assert fs.plan_size(w) == (len(orp) - 1, len(oci))


def test_plan_bit_exact_vs_oracle_random_geometries():
    rng = np.random.default_rng(21)
    for _ in range(60):
        T = 16 * int(rng.integers(1, 9))
        divs = [b for b in range(16, T + 1, 16) if T % b == 0]
        Fn = int(rng.integers(1, 12))
        t = (Fn, T, int(rng.integers(0, 5)), int(rng.integers(0, 5)), int(rng.integers(-1, Fn)),
             int(rng.choice(divs)), int(rng.choice(divs)), int(rng.integers(0, 2)), int(rng.integers(0, 4)))
        if t[4] + max(1, t[8]) > Fn:
            t = t[:8] + (0,)
        rp, ci = fs.plan(t)
        orp, oci = oracle.plan_bruteforce(oracle.MaskGeometry(*t))
        assert np.array_equal(rp.numpy(), orp), t
        assert np.array_equal(ci.numpy(), oci), t


def test_plan_golden():
    import json, os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "plan_tiny.json")))["cases"]
    for c in cases:
        rp, ci = fs.plan(c["mask"])
        assert rp.tolist() == c["row_ptr"] and ci.tolist() == c["col_idx"], c["name"]


@pytest.mark.parametrize("mask,status", [
    ((3, 48, 1, 1, 0, 32, 16), 2), ((3, 48, 1, 1, 0, 24, 16), 2), ((3, 48, 1, 1, 0, 16, 0), 2),
    ((3, 48, -1, 1, 0, 16, 16), 2), ((3, 48, 1, 1, 3, 16, 16), 2), ((3, 48, 1, 1, -2, 16, 16), 2),
    ((0, 48, 1, 1, -1, 16, 16), 2), ((3, 40, 1, 1, 0, 16, 16), 2), ((3, 48, 1, 1, 0, 16, 16, 2), 2),
    ((3, 48, 1, 1, 0, 16, 16, -1), 2), ((3, 48, 1, 1, 2, 16, 16, 0, 2), 2), ((3, 48, 1, 1, 0, 16, 16, 0, -1), 2),
    ((3, 48, 1, 1, 0, 16, 16, 0, 4), 2)])
def test_plan_rejects_bad_geometry(mask, status):
    with pytest.raises(fs.FsattnError) as e:
        fs.plan_size(mask)
    assert e.value.status == status


def test_plan_buffer_too_small_leaves_output_untouched():
    m = F.to_mask((5, 48, 1, 1, 0, 16, 16))
    rp = (ctypes.c_int32 * 16)(*([-7] * 16))
    ci = (ctypes.c_int32 * 143)(*([-7] * 143))
    st = fs.lib().fsattn_plan(ctypes.byref(m), rp, 16, ci, 143)
    assert st == 4
    assert list(rp) == [-7] * 16 and list(ci) == [-7] * 143
    st = fs.lib().fsattn_plan(ctypes.byref(m), rp, 15, ci, 144 if False else 143)
    assert st == 4


def test_plan_device_validates_on_host():
    """fsattn_plan_device rejects what fsattn_plan rejects, before any
    launch (the device pointers here are never dereferenced)."""
    L = fs.lib()
    good = F.to_mask((5, 48, 1, 1, 0, 16, 16))        # 16 query blocks, 143 entries
    bad = F.to_mask((5, 48, 1, 1, 0, 24, 16))
    assert L.fsattn_plan_device(None, ctypes.byref(bad), FAKE, 16, FAKE, 143) == 2
    assert L.fsattn_plan_device(None, ctypes.byref(good), FAKE, 15, FAKE, 143) == 4
    assert L.fsattn_plan_device(None, ctypes.byref(good), FAKE, 16, FAKE, 142) == 4
    assert L.fsattn_plan_device(None, ctypes.byref(good), None, 16, FAKE, 143) == 1
    assert L.fsattn_plan_device(None, None, FAKE, 16, FAKE, 143) == 1


# ---- argument validation of the GPU entry points (host-side, nothing launched)

FAKE = 0x7f0000000000          # 16-byte aligned, never dereferenced: every call below fails validation


def _t(ptr=FAKE, n=240, d=64, h=2):
    return F.Tensor(ptr, h * n * d, n * d, d)


def _bounds_call(shape=None, mask=None, q=None, k=None, scale=0.125, thr=30.0, km=FAKE, rec=FAKE, ws=FAKE,
                 wsb=1 << 30):
    s = shape or F.Shape(1, 2, 240, 64, 0)
    m = mask or F.to_mask((5, 48, 1, 1, 0, 16, 16))
    return fs.lib().fsattn_head_bounds(None, ctypes.byref(s), ctypes.byref(m), q or _t(), k or _t(),
                                       scale, thr, km, rec, ws, wsb)


def _fwd_call(shape=None, mask=None, nnz=144, q=None, k=None, v=None, o=None, odt=0, km=FAKE, rec=FAKE,
              scale=0.125, flags=0, rp=FAKE, ci=FAKE):
    s = shape or F.Shape(1, 2, 240, 64, 0)
    m = mask or F.to_mask((5, 48, 1, 1, 0, 16, 16))
    return fs.lib().fsattn_forward(None, ctypes.byref(s), ctypes.byref(m), rp, ci, nnz, q or _t(), k or _t(),
                                   v or _t(), o or _t(), odt, km, rec, scale, flags, None)


def test_head_bounds_validation():
    assert _bounds_call(shape=F.Shape(1, 2, 241, 64, 0)) == 1                  # seq_len != F*T
    assert _bounds_call(shape=F.Shape(1, 2, 240, 96, 0)) == 3                  # head_dim
    assert _bounds_call(shape=F.Shape(1, 2, 240, 64, 7)) == 3                  # dtype
    assert _bounds_call(shape=F.Shape(0, 2, 240, 64, 0)) == 1
    assert _bounds_call(mask=F.to_mask((5, 48, 1, 1, 0, 32, 16))) == 2
    assert _bounds_call(q=_t(FAKE + 4)) == 1                                    # misaligned
    assert _bounds_call(k=F.Tensor(FAKE, 1, 1, 63)) == 1                       # rows overlap / stride
    assert _bounds_call(k=F.Tensor(0, 1, 1, 64)) == 1                          # null
    assert _bounds_call(scale=0.0) == 1
    assert _bounds_call(scale=float("nan")) == 1
    assert _bounds_call(thr=-1.0) == 1
    assert _bounds_call(km=None) == 1
    assert _bounds_call(rec=None) == 1
    assert _bounds_call(ws=None) == 1
    assert _bounds_call(wsb=16) == 4


def test_noalloc_bounds_validates_on_host():
    """The allocation-free bounds entry rejects bad arguments and shapes whose
    workspace exceeds its device-resident array before any HIP call."""
    L = fs.lib()
    assert L.fsattn_head_bounds_noalloc_max_workspace() == 4 << 20
    m = F.to_mask((16, 1024, 15, 15, 0, 64, 64))
    big = F.Shape(1, 64, 16 * 1024, 128, 1)
    assert L.fsattn_head_bounds_workspace_bytes(ctypes.byref(big), ctypes.byref(m)) > 4 << 20
    ok = F.Shape(1, 8, 16 * 1024, 128, 1)
    assert L.fsattn_head_bounds_workspace_bytes(ctypes.byref(ok), ctypes.byref(m)) <= 4 << 20

    def call(shape, km=FAKE, rec=FAKE, scale=0.125, mask=m):
        t = _t(n=16 * 1024, d=128, h=64)
        return L.fsattn_head_bounds_noalloc(None, ctypes.byref(shape), ctypes.byref(mask), t, t, scale, 30.0, km, rec)
    assert call(big) == 4                                   # beyond the array
    assert call(ok, km=None) == 1
    assert call(ok, rec=None) == 1
    assert call(ok, scale=-1.0) == 1
    assert call(F.Shape(1, 8, 16 * 1024, 96, 1)) == 3       # head_dim not built
    assert call(ok, mask=F.to_mask((16, 1024, 15, 15, 0, 48, 64))) == 2


def test_workspace_bytes():
    L = fs.lib()
    s = F.Shape(1, 4, 48960, 128, 1)
    m = F.to_mask(workloads.workload(5))
    assert L.fsattn_head_bounds_workspace_bytes(ctypes.byref(s), ctypes.byref(m)) > 4 * 128 * 6 * 4
    bad = F.Shape(1, 4, 48961, 128, 1)
    assert L.fsattn_head_bounds_workspace_bytes(ctypes.byref(bad), ctypes.byref(m)) == 0


def test_forward_validation():
    assert _fwd_call(nnz=143) == 1                                             # plan does not match mask
    assert _fwd_call(shape=F.Shape(1, 2, 240, 128, 3)) == 3
    assert _fwd_call(mask=F.to_mask((5, 48, 1, 1, 0, 48, 32))) == 2
    assert _fwd_call(flags=3) == 1                                             # both modes
    assert _fwd_call(flags=1 << 28) == 1                                       # unknown bit
    assert _fwd_call(flags=fs.make_flags(deal=3)) == 3                         # fp32 path has no dealing
    assert _fwd_call(km=None) == 1                                             # fixed path needs the record
    assert _fwd_call(rp=None) == 1
    assert _fwd_call(ci=None) == 1
    assert _fwd_call(o=_t(FAKE + 8)) == 1
    assert _fwd_call(odt=1) == 3                                               # fp32 input, bf16 output
    assert _fwd_call(scale=-1.0) == 1
    assert _fwd_call(flags=fs.make_flags(waves=4)) == 3                        # fp32 path has no overrides


def test_launch_info_choices():
    for i in (2, 3, 4, 5):
        w = workloads.workload(i)
        waves, rows, kstep, wgs, lds = fs.launch_info((w.batch, w.heads, w.seq_len, w.head_dim), fs.BF16, w)
        assert w.tokens_per_frame % rows == 0                  # a wave tile never straddles frames
        tiles = -(-w.tokens_per_frame // (waves * rows))       # the last tile of a frame may be ragged
        assert wgs == w.batch * w.heads * w.num_frames * tiles
        assert lds <= 160 * 1024
    w = workloads.workload(3)
    # an explicit rows-per-wave that does not divide the frame span (3600 = 56 * 64 + 16) is
    # accepted: a frame's last wave runs partly past the frame's end and stores only its live rows
    waves, rows, _, wgs, _ = fs.launch_info((1, 5, 32400, 128), fs.BF16, w, fs.make_flags(waves=4, rows_per_wave=64))
    assert (waves, rows) == (4, 64) and wgs == 5 * 9 * 15
    waves, rows, _, _, _ = fs.launch_info((1, 5, 32400, 128), fs.BF16, w, fs.make_flags(waves=2, rows_per_wave=48))
    assert (waves, rows) == (2, 48)
    with pytest.raises(fs.FsattnError):           # 5-wave workgroups are not built
        fs.launch_info((1, 5, 32400, 128), fs.BF16, w, fs.make_flags(waves=5, rows_per_wave=48))
    w2 = workloads.workload(2)
    shape2 = (w2.batch, w2.heads, w2.seq_len, w2.head_dim)
    for ring, kstep, lds_expect in ((2, 32, 2 * 2 * 32 * 256), (3, 32, 3 * 2 * 32 * 256),
                                    (4, 32, 4 * 2 * 32 * 256), (2, 64, 2 * 2 * 64 * 256)):
        _, _, ks, _, lds = fs.launch_info(shape2, fs.BF16, w2, fs.make_flags(key_step=kstep, ring=ring))
        assert ks == kstep and lds_expect <= lds < lds_expect + 1024
    with pytest.raises(fs.FsattnError):           # a 3-buffer ring of 64-key steps is not built
        fs.launch_info(shape2, fs.BF16, w2, fs.make_flags(key_step=64, ring=3))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(F, "_lib", None)
    monkeypatch.setattr(F, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        F.lib()


def test_mfma_probe_validates_on_host():
    L = fs.lib()
    flops = ctypes.c_int64()
    assert L.fsattn_mfma_probe(None, 0, 10, FAKE, ctypes.byref(flops)) == 1
    assert L.fsattn_mfma_probe(None, 1 << 21, 10, FAKE, ctypes.byref(flops)) == 1
    assert L.fsattn_mfma_probe(None, 4, 0, FAKE, ctypes.byref(flops)) == 1
    assert L.fsattn_mfma_probe(None, 4, 10, None, ctypes.byref(flops)) == 1


def test_prior_art_forward_validates_on_host():
    L = fs.lib()
    s = F.Shape(1, 2, 240, 64, 1)
    m = F.to_mask((5, 48, 1, 1, 0, 16, 16))
    need = L.fsattn_prior_art_workspace_bytes(ctypes.byref(s), ctypes.byref(m))
    assert need >= 2 * 2 * 240 * (64 + 1) * 4

    def call(shape=s, ws=FAKE, wsb=need, scale=0.125, odt=1):
        return L.fsattn_prior_art_forward(None, ctypes.byref(shape), ctypes.byref(m), _t(), _t(), _t(), _t(), odt,
                                          scale, ws, wsb)
    assert call(shape=F.Shape(1, 2, 240, 64, 0)) == 3      # fp32 inputs
    assert call(ws=None) == 1
    assert call(ws=FAKE + 8) == 1                          # misaligned workspace
    assert call(wsb=need - 1) == 4
    assert call(scale=0.0) == 1
    assert call(shape=F.Shape(1, 2, 241, 64, 1)) == 1      # seq_len != F*T
    assert L.fsattn_prior_art_workspace_bytes(ctypes.byref(F.Shape(1, 2, 240, 64, 0)), ctypes.byref(m)) == 0
    for t in ((5, 48, 1, 1, 0, 16, 16, 1), (5, 48, 1, 1, 0, 16, 16, 0, 2)):   # one keys-only reference frame
        mg = F.to_mask(t)
        assert L.fsattn_prior_art_forward(None, ctypes.byref(s), ctypes.byref(mg), _t(), _t(), _t(), _t(), 1,
                                          0.125, FAKE, need) == 3


def test_produce_validates_on_host():
    L = fs.lib()
    s = F.Shape(1, 2, 240, 64, 1)
    m = F.to_mask((5, 48, 1, 1, 0, 16, 16))
    need = L.fsattn_head_bounds_workspace_bytes(ctypes.byref(s), ctypes.byref(m))

    def call(shape=s, gq=FAKE, gk=FAKE, eps=1e-6, cs=FAKE, sn=FAKE, km=FAKE, ws=FAKE, wsb=need, qin=None,
             scale=0.125, mask=m):
        return L.fsattn_produce(None, ctypes.byref(shape), ctypes.byref(mask), qin or _t(), _t(), _t(), gq, gk, eps,
                                cs, sn, _t(), _t(), _t(), scale, 30.0, km, FAKE, ws, wsb)
    assert call(gq=FAKE + 4) == 1                  # misaligned gamma
    assert call(cs=None) == 1                      # one table without the other
    assert call(sn=None) == 1
    assert call(eps=-1.0) == 1
    assert call(eps=float("inf")) == 1
    assert call(km=None) == 1
    assert call(ws=None) == 1
    assert call(wsb=need - 1) == 4
    assert call(scale=0.0) == 1
    assert call(qin=F.Tensor(FAKE, 0, 0, 32)) == 1                     # stride_n < head_dim
    assert call(shape=F.Shape(1, 2, 240, 96, 1)) == 3                   # head_dim not built
    assert call(shape=F.Shape(1, 2, 241, 64, 1)) == 1                   # seq_len != F*T
    assert call(mask=F.to_mask((5, 48, 1, 1, 0, 32, 16))) == 2


def _cpu(shape=(1, 2, 240, 64), dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def test_binding_rejects_operands_that_do_not_match_before_any_call():
    """The binding checks what the C ABI cannot see: the operands' shapes,
    dtypes, buffer extents and devices. Each bad case raises status 1, with
    the message of its own check, before the library is asked to launch
    anything (the tensors are CPU tensors, which the last check rejects)."""
    import torch
    mask = (3, 80, 1, 1, 0, 16, 16)
    q = _cpu()
    plan = fs.device_plan(mask, "cpu")
    cases = [
        ("dtype", lambda: fs.head_bounds(q, _cpu(dtype=torch.float32), mask)),
        ("shape", lambda: fs.head_bounds(q, _cpu((1, 2, 160, 64)), mask)),
        ("dtype", lambda: fs.head_bounds_noalloc(q, _cpu(dtype=torch.float32), mask)),
        ("key_mean", lambda: fs.head_bounds(q, q, mask, out=fs.Bounds(torch.zeros(1, 2, 32), torch.zeros(1, 2, 8)))),
        ("rec", lambda: fs.head_bounds_noalloc(q, q, mask, out=fs.Bounds(torch.zeros(1, 2, 64), torch.zeros(1, 2, 4)))),
        ("shape", lambda: fs.forward(q, q, _cpu((1, 2, 240, 128)), plan, None)),
        ("dtype", lambda: fs.forward(q, _cpu(dtype=torch.float32), q, plan, None)),
        ("out must be", lambda: fs.forward(q, q, q, plan, None, out=_cpu((1, 2, 240, 32)))),
        ("out must be", lambda: fs.forward(q, q, q, plan, None, out=_cpu(dtype=torch.float16))),
        ("lse", lambda: fs.forward(q, q, q, plan, None, lse=torch.zeros(100, dtype=torch.float32))),
        ("row_ptr", lambda: fs.forward(q, q, q, fs.DevicePlan(fs.to_mask(mask), torch.zeros(3, dtype=torch.int32),
                                                              plan.col_idx), None)),
        ("dtype", lambda: fs.produce(q, q, q, mask, out=(q, q, _cpu(dtype=torch.float32)))),
        ("shape", lambda: fs.produce(q, _cpu((2, 2, 240, 64)), q, mask)),
        ("key_mean", lambda: fs.produce(q, q, q, mask, bounds=fs.Bounds(torch.zeros(5), torch.zeros(1, 2, 8)))),
        ("dtype", lambda: fs.prior_art_forward(q, _cpu(dtype=torch.float32), q, mask)),
        ("out must be", lambda: fs.prior_art_forward(q, q, q, mask, out=_cpu((1, 1, 240, 64)))),
        ("on a GPU", lambda: fs.head_bounds(q, q, mask)),
        ("on a GPU", lambda: fs.head_bounds_noalloc(q, q, mask)),
        ("on a GPU", lambda: fs.forward(q, q, q, plan, None)),
        ("on a GPU", lambda: fs.produce(q, q, q, mask)),
        ("on a GPU", lambda: fs.prior_art_forward(q, q, q, mask)),
    ]
    for what, call in cases:
        with pytest.raises(fs.FsattnError, match=what) as e:
            call()
        assert e.value.status == 1, what


def test_empty_inputs_are_rejected_by_every_entry_point():
    """Empty problems (no batch, no head, no frame, no token) are argument or
    geometry errors at every GPU entry point, before anything is launched;
    the workspace queries return 0 for them."""
    L = fs.lib()
    m = F.to_mask((5, 48, 1, 1, 0, 16, 16))
    t = _t()
    for s in (F.Shape(0, 2, 240, 64, 1), F.Shape(1, 0, 240, 64, 1), F.Shape(1, 2, 0, 64, 1)):
        assert L.fsattn_head_bounds_workspace_bytes(ctypes.byref(s), ctypes.byref(m)) == 0
        assert L.fsattn_prior_art_workspace_bytes(ctypes.byref(s), ctypes.byref(m)) == 0
        assert _bounds_call(shape=s) in (1, 2)
        assert L.fsattn_head_bounds_noalloc(None, ctypes.byref(s), ctypes.byref(m), t, t, 0.125, 30.0,
                                            FAKE, FAKE) in (1, 2)
        assert _fwd_call(shape=s) in (1, 2)
        assert L.fsattn_produce(None, ctypes.byref(s), ctypes.byref(m), t, t, t, None, None, 1e-6, None, None,
                                t, t, t, 0.125, 30.0, FAKE, FAKE, FAKE, 1 << 30) in (1, 2)
        assert L.fsattn_prior_art_forward(None, ctypes.byref(s), ctypes.byref(m), t, t, t, t, 1, 0.125,
                                          FAKE, 1 << 30) in (1, 2)
    for empty in ((0, 48, 1, 1, 0, 16, 16), (5, 0, 1, 1, 0, 16, 16)):
        me = F.to_mask(empty)
        nq, nz = ctypes.c_int64(), ctypes.c_int64()
        assert L.fsattn_plan_size(ctypes.byref(me), ctypes.byref(nq), ctypes.byref(nz)) == 2
        assert _bounds_call(mask=me) == 2
        assert _fwd_call(mask=me) == 2
