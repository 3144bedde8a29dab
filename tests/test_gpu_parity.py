"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances: max-abs <= 1e-5 for fp32 inputs and <= 2e-2 for bf16 inputs
(fp32 accumulation, P rounded to bf16 for PV, bf16 output). Bound records:
relative 1e-5 (fp32 reductions vs fp64), eligibility decisions equal.
"""
import dataclasses
import math
import sys
import time

import numpy as np
import pytest
import torch

import frame_block_sparse_amd as fs
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
# Log-sum-exp bound.  The bf16 kernel sums the probabilities after rounding them
# to bf16 (the same weights the PV product multiplies, so the output stays a
# convex combination of value rows).  bf16 keeps 8 significant bits, so rounding
# to nearest moves each weight by a relative error of at most 2^-8; the sum then
# carries at most that relative error too, and its log moves by at most
# -log(1 - 2^-8) = 3.914e-3.  The fp32 accumulation adds at most (number of
# sequential fp32 additions) x 2^-24 relative: <= 1.6e3 MFMA accumulations on
# the fixed path, <= 6.2e3 two-term dot steps plus 2 lane sums and the rescales
# on the online path for up to 49k keys, i.e. < 4e-4.  Hence 4.5e-3.
LSE_TOL = {"f32": 1e-5, "bf16": 4.5e-3}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fs.lib()
    return torch.device("cuda:0")


def _to_dev(x, dtype, dev):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(dtype).to(dev)


def _tdtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def _run(w, q, k, v, dev, flags=0, out_dtype=None, lse=False):
    td = _tdtype(w)
    qd, kd, vd = (_to_dev(x, td, dev) for x in (q, k, v))
    dp = fs.device_plan(w, dev)
    bnd = fs.head_bounds(qd, kd, w)
    lse_t = torch.empty((w.batch, w.heads, w.seq_len), dtype=torch.float32, device=dev) if lse else None
    out = fs.forward(qd, kd, vd, dp, bnd, flags=flags, out_dtype=out_dtype, lse=lse_t)
    torch.cuda.synchronize()
    return out, bnd, lse_t


def _geom(w):
    return oracle.MaskGeometry(*w.mask_tuple())


_ORACLE_CACHE = {}


def _oracle_full(w, q, k, v):
    """Every row of the workload from the fp64 oracle (each row's sums over
    its live keys), computed once per session per (workload, mask)."""
    key = (w.name,) + w.mask_tuple()
    if key not in _ORACLE_CACHE:
        t0 = time.perf_counter()
        _ORACLE_CACHE[key] = oracle.attention_live_ref(q, k, v, _geom(w))
        _say(f"    oracle (fp64, all {w.batch * w.heads * w.seq_len} rows) {time.perf_counter() - t0:.1f} s")
    return _ORACLE_CACHE[key]


def _max_abs_err(got, ref, chunk_rows=4096):
    """max |got - ref| over every element, with got a device tensor; compared
    in row chunks to bound host memory."""
    B, H, N, d = ref.shape
    err = 0.0
    for b in range(B):
        for h in range(H):
            for s0 in range(0, N, chunk_rows):
                g = got[b, h, s0:s0 + chunk_rows].float().cpu().numpy()
                err = max(err, float(np.abs(g - ref[b, h, s0:s0 + chunk_rows]).max()))
    return err


# ------------------------------------------------------------------ bounds

@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_plan_device_bit_exact_on_workloads(dev, i):
    """fsattn_plan_device writes the host plan's arrays element for element."""
    w = workloads.workload(i)
    _say(f"[plan-device] {w.name}")
    rp, ci = fs.plan(w)
    dp = fs.plan_on_device(w, dev)
    torch.cuda.synchronize()
    assert torch.equal(dp.row_ptr.cpu(), rp) and torch.equal(dp.col_idx.cpu(), ci)


def test_plan_device_bit_exact_on_random_geometries(dev):
    rng = np.random.default_rng(11)
    cases = [(3, 32, 10 ** 6, 10 ** 6, 1, 16, 32), (1, 16, 0, 0, -1, 16, 16), (7, 48, 0, 2, 6, 48, 16),
             (7, 48, 0, 2, 6, 48, 16, 1), (9, 32, 1, 1, 4, 16, 32, 1), (9, 32, 1, 1, 4, 16, 32, 0, 3),
             (9, 32, 0, 0, 0, 32, 16, 1, 2), (6, 16, 10 ** 6, 0, 3, 16, 16, 0, 3)]
    for _ in range(40):
        T = 16 * int(rng.integers(1, 7))
        divs = [b for b in range(16, T + 1, 16) if T % b == 0]
        F_ = int(rng.integers(1, 12))
        t = (F_, T, int(rng.integers(0, 4)), int(rng.integers(0, 4)), int(rng.integers(-1, F_)),
             int(rng.choice(divs)), int(rng.choice(divs)), int(rng.integers(0, 2)), int(rng.integers(0, 4)))
        cases.append(t if t[4] + max(1, t[8]) <= F_ else t[:8] + (0,))
    for g in cases:
        rp, ci = fs.plan(g)
        dp = fs.plan_on_device(g, dev)
        torch.cuda.synchronize()
        assert torch.equal(dp.row_ptr.cpu(), rp), g
        assert torch.equal(dp.col_idx.cpu(), ci), g
        if g[0] * g[1] <= 400:
            orp, oci = oracle.plan_bruteforce(oracle.MaskGeometry(*g))
            assert np.array_equal(rp.numpy(), orp) and np.array_equal(ci.numpy(), oci), g


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_head_bounds_parity(dev, config_inputs, i):
    w = workloads.workload(i)
    _say(f"[bounds] workload {i} {w.name}")
    q, k, v = config_inputs(i)
    td = _tdtype(w)
    b = fs.head_bounds(_to_dev(q, td, dev), _to_dev(k, td, dev), w)
    torch.cuda.synchronize()
    got = b.host()
    ref = oracle.head_bounds_ref(q, k, _geom(w))
    np.testing.assert_allclose(b.key_mean.cpu().numpy(), ref["mu"], rtol=1e-5,
                               atol=1e-6 * max(1.0, float(np.abs(ref["mu"]).max())))
    for name, rname in (("q_norm_max", "q_max"), ("k_norm_max", "k_max"), ("bound", "bound"),
                        ("gap_est", "gap_est")):
        np.testing.assert_allclose(got[name], ref[rname], rtol=1e-5, err_msg=name)
    np.testing.assert_allclose(got["c_max"], ref["c_max"], rtol=1e-4,
                               atol=1e-5 * float(ref["k_max"].max()))
    assert np.array_equal(got["eligible"].astype(bool), ref["eligible"])


def test_head_bounds_deterministic(dev, config_inputs):
    w = workloads.workload(2)
    q, k, _ = config_inputs(2)
    qd, kd = _to_dev(q, torch.bfloat16, dev), _to_dev(k, torch.bfloat16, dev)
    a = fs.head_bounds(qd, kd, w)
    b = fs.head_bounds(qd, kd, w)
    torch.cuda.synchronize()
    assert torch.equal(a.rec, b.rec) and torch.equal(a.key_mean, b.key_mean)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_head_bounds_threshold_inclusive(dev, dt):
    """One frame of 16 keys in d = 64: 8 x (5, 0, ...) and 8 x (-5, 0, ...)
    (key mean 0, K_max 5, C_max 0) and one query (6, 0, ...) (Q_max 6), so
    gap_est = scale * 30 (29.8828125, 30, 30.1171875 for scale 255/256, 1,
    257/256). The kernel's decision is gap_est <= threshold, inclusive: it
    holds at a threshold equal to the stored gap estimate and fails one fp32
    step below it; at the default 30 nats the three heads are eligible,
    eligible and not."""
    w = workloads.make_workload("thr", 1, 1, 1, 16, 64, dt, 0, 0, -1, 16, 16)
    k = np.zeros((1, 1, 16, 64), np.float32); k[0, 0, :8, 0] = 5.0; k[0, 0, 8:, 0] = -5.0
    q = np.zeros((1, 1, 16, 64), np.float32); q[0, 0, 0, 0] = 6.0
    td = _tdtype(w)
    qd, kd = _to_dev(q, td, dev), _to_dev(k, td, dev)
    for scale, gap, elig in ((255 / 256, 29.8828125, 1), (1.0, 30.0, 1), (257 / 256, 30.1171875, 0)):
        _say(f"[bounds-threshold] {dt} scale={scale}")
        r = fs.head_bounds(qd, kd, w, scale=scale).host()
        g = float(r["gap_est"][0, 0])
        assert g == pytest.approx(gap, rel=1e-6), (scale, g)
        assert int(r["eligible"][0, 0]) == elig, (scale, g)
        at = fs.head_bounds(qd, kd, w, scale=scale, threshold=g).host()
        below = fs.head_bounds(qd, kd, w, scale=scale, threshold=float(np.nextafter(np.float32(g), 0))).host()
        assert int(at["eligible"][0, 0]) == 1 and int(below["eligible"][0, 0]) == 0, (scale, g)


@pytest.mark.parametrize("mode", ["auto", "fixed", "fixed_per_row", "online"])
def test_forward_large_key_offset_along_queries(dev, mode):
    """Keys offset by 20 in every dimension and queries by 1: each row's raw
    logits sit 167-280 nats (scale * q_i . mu) above its centred ones, so a
    fixed shift without the scale * q_i . mu term would overflow fp32 exp
    (e^88.7), and one that dropped the scale would underflow every weight.
    The heads are eligible (the centred gap is small) and both shift variants
    must match the oracle."""
    w = workloads.make_workload("offset20", 1, 2, 4, 64, 128, "bf16", 1, 1, 0, 32, 32)
    rng = np.random.default_rng(21)
    shape = (1, 2, 256, 128)
    q = workloads.round_to_bf16(rng.standard_normal(shape, dtype=np.float32) + np.float32(1.0))
    k = workloads.round_to_bf16(rng.standard_normal(shape, dtype=np.float32) + np.float32(20.0))
    v = workloads.round_to_bf16(rng.standard_normal(shape, dtype=np.float32))
    _say(f"[fwd-offset] mode={mode}")
    flags = fs.make_flags("fixed" if mode == "fixed_per_row" else mode, per_row_shift=mode == "fixed_per_row")
    out, bnd, lse = _run(w, q, k, v, dev, flags=flags, lse=True)
    rec = bnd.host()
    assert rec["eligible"].all(), rec["gap_est"]
    g = _geom(w)
    ref, ref_lse = oracle.attention_ref(q, k, v, g)
    mu = k.astype(np.float64).mean(axis=2)
    qmu = np.einsum("bhnd,bhd->bhn", q.astype(np.float64), mu) / math.sqrt(128)
    # without the q . mu term a row's largest weight would be e^x with
    # x >= (scale q_i . mu - gap_est) - bound >= q_i . mu term - 2 gap_est
    assert qmu.min() - 2 * rec["gap_est"].max() > 89.0, (qmu.min(), rec["gap_est"])
    o = out.float().cpu().numpy()
    assert np.isfinite(o).all()
    assert np.abs(o - ref).max() <= TOL["bf16"], np.abs(o - ref).max()
    # LSE: the weights' rounding (LSE_TOL) plus the fp32 rounding of 128-term
    # logits of this size, d * 2^-24 * scale * |q| * |k|
    qn = np.linalg.norm(q.astype(np.float64), axis=-1).max()
    kn = np.linalg.norm(k.astype(np.float64), axis=-1).max()
    tol = LSE_TOL["bf16"] + 128 * 2.0 ** -24 * qn * kn / math.sqrt(128)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= tol


# ------------------------------------------------------------------ forward, small shapes

SMALL = [
    # (name, B, H, F, T, d, dtype, wb, wa, ref, bq, bk)
    ("odd16_tail", 2, 3, 5, 240, 128, "bf16", 1, 1, 0, 48, 80),
    ("ref_last", 1, 2, 4, 192, 128, "bf16", 1, 1, 3, 64, 32),
    ("causal_noref", 1, 2, 6, 160, 128, "bf16", 2, 0, -1, 32, 16),
    ("dense", 1, 2, 3, 256, 128, "bf16", 3, 3, 0, 64, 64),
    ("d64", 2, 2, 5, 96, 64, "bf16", 1, 1, 0, 48, 16),
    ("single_frame", 1, 1, 1, 64, 128, "bf16", 0, 0, -1, 16, 64),
    # 16-token frames: the reference frame is a 16-key run ending before
    # key 32, so its copy cannot start 32 rows before its end
    ("ref16_clamp", 1, 2, 6, 16, 128, "bf16", 1, 1, 0, 16, 16),
    ("ref16_clamp_d64", 2, 1, 3, 16, 64, "bf16", 1, 0, -1, 16, 16),
    # a sequence shorter than one 32-key step
    ("tiny16", 1, 1, 1, 16, 128, "bf16", 0, 0, -1, 16, 16),
    ("f32_d128", 1, 2, 4, 80, 128, "f32", 1, 1, 0, 16, 80),
    ("f32_d64", 2, 1, 6, 48, 64, "f32", 0, 2, 5, 48, 16),
]

# (waves, rows per wave) of every built launch shape, and the key steps
SHAPES = [(4, 32), (4, 48), (4, 16), (4, 64), (8, 32), (2, 48), (2, 64), (2, 32)]
SHAPE_OVERRIDES = [(w, r, ks, rb) for (w, r) in SHAPES for (ks, rb) in ((32, 2), (32, 3), (32, 4), (64, 2))]


def _small(case, seed=0, key_offset=0.0):
    name, B, H, F, T, d, dt, wb, wa, r, bq, bk = case
    w = workloads.make_workload(name, B, H, F, T, d, dt, wb, wa, r, bq, bk)
    q, k, v = workloads.make_inputs(w, seed=seed)
    if key_offset:
        k = workloads.round_to_bf16(k + np.float32(key_offset)) if dt == "bf16" else k + np.float32(key_offset)
    return w, q, k, v


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("mode", ["auto", "online", "fixed", "fixed_per_row"])
def test_forward_small_parity(dev, case, mode):
    w, q, k, v = _small(case, seed=1, key_offset=1.5)
    _say(f"[fwd-small] {w.name} mode={mode}")
    flags = fs.make_flags("fixed" if mode == "fixed_per_row" else mode, per_row_shift=mode == "fixed_per_row")
    out, bnd, lse = _run(w, q, k, v, dev, flags=flags, lse=True)
    assert bnd.host()["eligible"].all()
    ref, ref_lse = oracle.attention_ref(q, k, v, _geom(w))
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= TOL[w.dtype], err
    lerr = np.abs(lse.cpu().numpy() - ref_lse).max()
    assert lerr <= LSE_TOL[w.dtype], lerr


@pytest.mark.parametrize("i", [2, 5])
def test_forward_dealing_is_bitwise_neutral(dev, config_inputs, i):
    """How the tiles are dealt to the XCDs (whole (frame, head) groups, the
    library's chunks, single tiles, a chunk larger than a group) changes only
    where each tile runs: the outputs are bitwise equal."""
    w = workloads.workload(i)
    q, k, v = config_inputs(i)
    qd, kd, vd = (_to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    dp = fs.device_plan(w, dev)
    bnd = fs.head_bounds(qd, kd, w)
    ref = fs.forward(qd, kd, vd, dp, bnd, flags=fs.make_flags(deal=15))
    for deal in (0, 1, 3, 9):
        _say(f"[deal] workload {i} deal={deal}")
        out = fs.forward(qd, kd, vd, dp, bnd, flags=fs.make_flags(deal=deal))
        torch.cuda.synchronize()
        assert torch.equal(out, ref), deal


_SHAPE_REF = {}


@pytest.mark.parametrize("shape", SHAPE_OVERRIDES, ids=[f"w{a}_r{b}_k{c}_b{d}" for a, b, c, d in SHAPE_OVERRIDES])
def test_forward_launch_shapes(dev, shape):
    """Every built launch shape on a frame span its wave tile divides; several
    leave the frame's last workgroup ragged (idle waves)."""
    waves, rows, kstep, ring = shape
    T = next(t for t in (720, 960, 768) if t % rows == 0)
    case = (f"shapes{T}", 1, 2, 3, T, 128, "bf16", 1, 1, 0, 48, 48)
    w, q, k, v = _small(case, seed=2)
    if T not in _SHAPE_REF:
        _SHAPE_REF[T] = oracle.attention_ref(q, k, v, _geom(w))[0]
    ref = _SHAPE_REF[T]
    _say(f"[fwd-shape] T={T} waves={waves} rows={rows} kstep={kstep} ring={ring}")
    for mode in ("auto", "online"):
        flags = fs.make_flags(mode, waves=waves, rows_per_wave=rows, key_step=kstep, ring=ring)
        assert fs.launch_info((1, 2, 3 * T, 128), fs.BF16, w, flags)[:3] == (waves, rows, kstep)
        out, _, _ = _run(w, q, k, v, dev, flags=flags)
        err = np.abs(out.float().cpu().numpy() - ref).max()
        assert err <= TOL["bf16"], (mode, err)


RAGGED = [(4, 32, 48), (4, 32, 80), (2, 32, 112), (4, 48, 80), (4, 64, 48), (4, 64, 112), (8, 32, 208),
          (2, 64, 16)]


@pytest.mark.parametrize("shape", RAGGED, ids=[f"w{a}_r{b}_T{c}" for a, b, c in RAGGED])
def test_forward_ragged_last_wave(dev, shape):
    """Rows per wave that do not divide the frame span: each frame's last wave
    runs partly past the frame's end (in the last frame, past the sequence's
    end), computes those rows on the frame's last query row and stores only
    its live rows. Every row matches the oracle, on both softmax paths, and a
    sentinel in the output shows nothing outside the live rows is written."""
    waves, rows, T = shape
    case = (f"ragged{T}", 2, 2, 4, T, 128, "bf16", 1, 1, 0, 16, 16)
    w, q, k, v = _small(case, seed=6, key_offset=0.25)
    ref, ref_lse = oracle.attention_ref(q, k, v, _geom(w))
    qd, kd, vd = (_to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    dp = fs.device_plan(w, dev)
    bnd = fs.head_bounds(qd, kd, w)
    for mode in ("auto", "online"):
        _say(f"[fwd-ragged] waves={waves} rows={rows} T={T} mode={mode}")
        flags = fs.make_flags(mode, waves=waves, rows_per_wave=rows)
        assert fs.launch_info(tuple(qd.shape), fs.BF16, w, flags)[:2] == (waves, rows)
        # one extra row on each side of the output and LSE, holding a sentinel
        big = torch.full((w.batch, w.heads, w.seq_len + 2, w.head_dim), 7.0, dtype=torch.bfloat16, device=dev)
        lse_big = torch.full((w.batch * w.heads * w.seq_len + 2,), 7.0, dtype=torch.float32, device=dev)
        out = big[:, :, 1:w.seq_len + 1]
        lse = lse_big[1:-1].view(w.batch, w.heads, w.seq_len)
        fs.forward(qd, kd, vd, dp, bnd, flags=flags, out=out, lse=lse)
        torch.cuda.synchronize()
        err = np.abs(out.float().cpu().numpy() - ref).max()
        assert err <= TOL["bf16"], (mode, err)
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= LSE_TOL["bf16"], mode
        assert (big[:, :, 0] == 7.0).all() and (big[:, :, -1] == 7.0).all()
        assert lse_big[0].item() == 7.0 and lse_big[-1].item() == 7.0


def test_forward_fp32_output_and_strided_layout(dev):
    case = ("strided", 2, 3, 4, 144, 128, "bf16", 1, 1, 0, 48, 48)
    w, q, k, v = _small(case, seed=3)
    ref, _ = oracle.attention_ref(q, k, v, _geom(w))
    out32, _, _ = _run(w, q, k, v, dev, out_dtype=torch.float32)
    assert out32.dtype == torch.float32
    assert np.abs(out32.cpu().numpy() - ref).max() <= 5e-3
    # the same data in a [B, N, H, d] buffer viewed as [B, H, N, d] (no repack)
    def bnhd(x):
        t = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))).to(torch.bfloat16).to(dev)
        return t.permute(0, 2, 1, 3)
    qd, kd, vd = bnhd(q), bnhd(k), bnhd(v)
    assert not qd.is_contiguous()
    dp = fs.device_plan(w, dev)
    bnd = fs.head_bounds(qd, kd, w)
    o = torch.empty((w.batch, w.seq_len, w.heads, w.head_dim), dtype=torch.bfloat16, device=dev).permute(0, 2, 1, 3)
    fs.forward(qd, kd, vd, dp, bnd, out=o)
    torch.cuda.synchronize()
    assert np.abs(o.float().cpu().numpy() - ref).max() <= TOL["bf16"]


# ------------------------------------------------------------------ forward, the five workloads

@pytest.mark.parametrize("i", [1, 2, 3, 4, 5])
def test_forward_workload_parity(dev, config_inputs, i):
    """Full-size workloads in the benchmark's launch configuration (library
    default), every element of O against the fp64 oracle; plus properties
    of every row: finite, and inside the range of V."""
    w = workloads.workload(i)
    _say(f"[fwd] workload {i} {w.name}")
    q, k, v = config_inputs(i)
    out, bnd, _ = _run(w, q, k, v, dev)
    ref, _ = _oracle_full(w, q, k, v)
    err = _max_abs_err(out, ref)
    _say(f"    max abs err {err:.3e} over every element; max |O| {np.abs(ref).max():.3f}; "
         f"eligible heads {int(bnd.host()['eligible'].sum())}/{w.batch * w.heads}")
    assert err <= TOL[w.dtype], err
    o = out.float()
    assert torch.isfinite(o).all()
    vmax = torch.from_numpy(np.abs(v).max(axis=2, keepdims=True)).to(dev)
    assert bool((o.abs() <= vmax * (1 + 2 ** -7) + 1e-6).all())
    # The log-sum-exp output, from a second launch that also writes it: O is
    # bitwise the same, and every row's LSE is within the weights' rounding
    # (LSE_TOL) plus the fp32 rounding of d-term logits, d 2^-24 scale |q| |k|.
    out2, _, lse = _run(w, q, k, v, dev, lse=True)
    assert torch.equal(out2, out)
    _, ref_lse = _oracle_full(w, q, k, v)
    qn = float(np.linalg.norm(q.astype(np.float64), axis=-1).max())
    kn = float(np.linalg.norm(k.astype(np.float64), axis=-1).max())
    tol = LSE_TOL[w.dtype] + w.head_dim * 2.0 ** -24 * qn * kn / math.sqrt(w.head_dim)
    lerr = float(np.abs(lse.cpu().numpy() - ref_lse).max())
    _say(f"    LSE max abs err {lerr:.3e} over every row (tol {tol:.2e})")
    assert np.isfinite(lerr) and lerr <= tol, lerr


def _random_geometries(n, seed):
    """Seeded random test-sized geometries: frames of 16-384 tokens, any
    block sizes dividing them, windows of 0-3 frames on either side, no
    reference frame or spans of 1-2 (global or not), head_dim 64 or 128,
    bf16 or fp32, 1-2 batches and 1-3 heads, plain or offset keys."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        T = 16 * int(rng.integers(1, 25))
        divs = [b for b in range(16, T + 1, 16) if T % b == 0]
        F_ = int(rng.integers(1, 9))
        ref = int(rng.integers(-1, F_))
        rc = int(rng.integers(0, 3)) if ref >= 0 else 0
        if ref + max(1, rc) > F_:
            rc = 0
        gq = int(rng.integers(0, 2)) if ref >= 0 else 0
        out.append((f"rnd{i}", int(rng.integers(1, 3)), int(rng.integers(1, 4)), F_, T, int(rng.choice([64, 128])),
                    "bf16" if rng.random() < 0.75 else "f32", int(rng.integers(0, 4)), int(rng.integers(0, 4)), ref,
                    int(rng.choice(divs)), int(rng.choice(divs)), gq, rc, float(rng.choice([0.0, 1.5])),
                    str(rng.choice(["auto", "online", "fixed"]))))
    return out


RANDOM_GEOMETRIES = _random_geometries(100, 2024)


@pytest.mark.parametrize("case", RANDOM_GEOMETRIES, ids=[c[0] for c in RANDOM_GEOMETRIES])
def test_forward_random_geometries(dev, case):
    """Random geometries (seeded) in the library's default launch: the bound
    records, every element of O and every row's LSE against the oracle.
    "fixed" runs only where every head is eligible (else "auto")."""
    w, q, k, v = _small(case[:12], seed=7, key_offset=case[14])
    w = dataclasses.replace(w, ref_queries_global=case[12], ref_count=case[13])
    _say(f"[fwd-random] {case}")
    g = _geom(w)
    td = _tdtype(w)
    qd, kd, vd = (_to_dev(x, td, dev) for x in (q, k, v))
    bnd = fs.head_bounds(qd, kd, w)
    rec = bnd.host()
    ref_b = oracle.head_bounds_ref(q, k, g)
    for name, rname in (("q_norm_max", "q_max"), ("k_norm_max", "k_max"), ("gap_est", "gap_est")):
        np.testing.assert_allclose(rec[name], ref_b[rname], rtol=1e-5, err_msg=name)
    assert np.array_equal(rec["eligible"].astype(bool), ref_b["eligible"])
    mode = case[15] if case[15] != "fixed" or rec["eligible"].all() else "auto"
    lse = torch.empty((w.batch, w.heads, w.seq_len), dtype=torch.float32, device=dev)
    out = fs.forward(qd, kd, vd, fs.device_plan(w, dev), bnd, flags=fs.make_flags(mode), lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention_ref(q, k, v, g)
    err = float(np.abs(out.float().cpu().numpy() - ref).max())
    assert err <= TOL[w.dtype], err
    qn = float(np.linalg.norm(q.astype(np.float64), axis=-1).max())
    kn = float(np.linalg.norm(k.astype(np.float64), axis=-1).max())
    tol = LSE_TOL[w.dtype] + w.head_dim * 2.0 ** -24 * qn * kn / math.sqrt(w.head_dim)
    lerr = float(np.abs(lse.cpu().numpy() - ref_lse).max())
    assert lerr <= tol, lerr


def test_offsets_past_2_31_elements(dev):
    """Addressing at the largest sizes: 72 heads of 262144 tokens at d = 128
    (16-token frames, each query sees its own frame only), 2.4e9 elements per
    tensor, so the last heads start past 2^31 elements. The records of the
    first and the last head (each computed whole on the host) and the O and
    LSE rows of frames of both heads, near either end of the sequence,
    against the oracle; each frame is its own problem, so a frame's slice is
    checked with a one-frame geometry."""
    B, H, F_, T, d = 1, 72, 16384, 16, 128
    N = F_ * T
    assert B * H * N * d > 2 ** 31
    w = workloads.make_workload("offsets_2_31", B, H, F_, T, d, "bf16", 0, 0, -1, 16, 16)
    _say("[big] drawing 3 x 2.4e9 bf16 inputs on the device")
    q, k, v = (workloads.device_normal((B, H, N, d), s, dev, torch.bfloat16) for s in (31, 32, 33))
    bnd = fs.head_bounds(q, k, w)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _say("[big] forward")
    out = fs.forward(q, k, v, fs.plan_on_device(w, dev), bnd, lse=lse)
    torch.cuda.synchronize()
    rec = bnd.host()
    for h in (0, H - 1):
        qh, kh = (t[:, h:h + 1].float().cpu().numpy() for t in (q, k))
        ref = oracle.head_bounds_ref(qh, kh, _geom(w))
        np.testing.assert_allclose(bnd.key_mean[:, h].cpu().numpy(), ref["mu"][:, 0], rtol=1e-5, atol=1e-6)
        for name, rname in (("q_norm_max", "q_max"), ("k_norm_max", "k_max"), ("gap_est", "gap_est")):
            np.testing.assert_allclose(rec[name][:, h], ref[rname][:, 0], rtol=1e-5, err_msg=f"{name} head {h}")
        assert bool(rec["eligible"][0, h]) == bool(ref["eligible"][0, 0])
    g1 = oracle.MaskGeometry(1, T, 0, 0, -1, 16, 16)
    for h in (0, H - 1):
        for f in (0, 1, F_ // 2, F_ - 2, F_ - 1):
            sl = slice(f * T, (f + 1) * T)
            qs, ks, vs = (t[:, h:h + 1, sl].float().cpu().numpy() for t in (q, k, v))
            ro, rl = oracle.attention_ref(qs, ks, vs, g1)
            assert np.abs(out[:, h:h + 1, sl].float().cpu().numpy() - ro).max() <= TOL["bf16"], (h, f)
            assert np.abs(lse[:, h:h + 1, sl].cpu().numpy() - rl).max() <= LSE_TOL["bf16"], (h, f)
    del q, k, v, out, lse, bnd
    torch.cuda.empty_cache()


def test_whole_path_in_a_captured_graph(dev):
    """Plan (device), bounds and forward captured once in a HIP graph (the
    path records no memset and allocates nothing: every buffer is the
    caller's) and replayed three times; before each replay new inputs are
    copied in eagerly and the device synchronised; every replay's output,
    records and LSE equal an eager run's on the same inputs, bit for bit."""
    w = workloads.make_workload("graph_path", 1, 4, 6, 480, 128, "bf16", 1, 1, 0, 48, 80)
    sets = []
    for seed in (21, 22, 23, 24):
        q, k, v = workloads.make_inputs(w, seed=seed)
        sets.append(tuple(_to_dev(x, torch.bfloat16, dev) for x in (q, k, v)))
    qs, ks, vs = (t.clone() for t in sets[0])
    dp = fs.plan_on_device(w, dev)
    ws = torch.empty(fs.head_bounds_workspace_bytes(qs, w), dtype=torch.uint8, device=dev)
    bnd = fs.head_bounds(qs, ks, w, workspace=ws)
    out = torch.empty_like(qs)
    lse = torch.empty((w.batch, w.heads, w.seq_len), dtype=torch.float32, device=dev)
    fs.forward(qs, ks, vs, dp, bnd, out=out, lse=lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fs.plan_on_device(w, out=dp)
        fs.head_bounds(qs, ks, w, workspace=ws, out=bnd)
        fs.forward(qs, ks, vs, dp, bnd, out=out, lse=lse)
    torch.cuda.synchronize()
    for rep, (q, k, v) in enumerate(sets[1:]):
        _say(f"[graph-path] replay {rep}")
        for dst, src in ((qs, q), (ks, k), (vs, v)):
            dst.copy_(src)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rb = fs.head_bounds(q, k, w)
        rl = torch.empty_like(lse)
        ro = fs.forward(q, k, v, fs.plan_on_device(w, dev), rb, lse=rl)
        torch.cuda.synchronize()
        assert torch.equal(bnd.rec, rb.rec) and torch.equal(bnd.key_mean, rb.key_mean), rep
        assert torch.equal(out, ro) and torch.equal(lse, rl), rep


@pytest.mark.parametrize("where", ["q", "k"])
def test_non_finite_input_stays_in_the_rows_it_touches(dev, where):
    """A NaN at query (or key) 77 of head 1 of four 64-token frames (window
    +-1, reference frame 0): the other heads' records and outputs equal
    those of the same call without it, bit for bit; in head 1 every row that
    does not touch the NaN matches the oracle on the clean inputs. A NaN
    query leaves head 1 eligible (the norm maximum skips it) and only its own
    row non-finite; a NaN key makes the key mean non-finite, so head 1 is not
    eligible and only the rows that attend to frame 1 are non-finite (frame
    3's rows see frames 2, 3 and 0 and stay exact)."""
    w = workloads.make_workload("nan_head", 1, 3, 4, 64, 128, "bf16", 1, 1, 0, 32, 32)
    q, k, v = workloads.make_inputs(w, seed=5)
    qd, kd, vd = (_to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    dp = fs.device_plan(w, dev)
    b0 = fs.head_bounds(qd, kd, w)
    o0 = fs.forward(qd, kd, vd, dp, b0)
    bad = (qd if where == "q" else kd).clone()
    bad[0, 1, 77, 5] = float("nan")
    q1, k1 = (bad, kd) if where == "q" else (qd, bad)
    b1 = fs.head_bounds(q1, k1, w)
    o1 = fs.forward(q1, k1, vd, dp, b1)
    torch.cuda.synchronize()
    assert b0.host()["eligible"].all()
    for h in (0, 2):
        assert torch.equal(b1.rec[0, h], b0.rec[0, h]) and torch.equal(b1.key_mean[0, h], b0.key_mean[0, h])
        assert torch.equal(o1[0, h], o0[0, h])
    ref, _ = oracle.attention_ref(q, k, v, _geom(w))
    got = o1[0, 1].float().cpu().numpy()
    if where == "q":
        assert b1.host()["eligible"][0, 1] == 1
        clean = np.ones(w.seq_len, bool)
        clean[77] = False
        assert not np.isfinite(got[77]).all()
    else:
        assert b1.host()["eligible"][0, 1] == 0
        clean = np.zeros(w.seq_len, bool)
        clean[192:] = True                       # frame 3: frames 2, 3 and the reference frame 0
        assert (~np.isfinite(got[:192])).any(axis=1).all()   # frames 0-2 all attend to key 77
    assert np.isfinite(got[clean]).all()
    assert np.abs(got[clean] - ref[0, 1][clean]).max() <= TOL["bf16"]


def _random_shaped_cases(n, seed):
    """Seeded random bf16 geometries, each with a random launch-shape
    override (waves and rows per wave from every built shape, keys per step
    and ring depth, tile dealing), so that ragged last waves, remainder steps
    and idle waves meet every shape."""
    rng = np.random.default_rng(seed)
    steps = [(32, 2), (32, 3), (32, 4), (64, 2)]
    out = []
    for i in range(n):
        T = 16 * int(rng.integers(1, 21))
        divs = [b for b in range(16, T + 1, 16) if T % b == 0]
        F_ = int(rng.integers(1, 7))
        ref = int(rng.integers(-1, F_))
        rc = int(rng.integers(0, 3)) if ref >= 0 else 0
        if ref + max(1, rc) > F_:
            rc = 0
        waves, rows = SHAPES[int(rng.integers(0, len(SHAPES)))]
        kstep, ring = steps[int(rng.integers(0, len(steps)))]
        out.append((f"shp{i}", int(rng.integers(1, 3)), int(rng.integers(1, 4)), F_, T, int(rng.choice([64, 128])),
                    "bf16", int(rng.integers(0, 3)), int(rng.integers(0, 3)), ref, int(rng.choice(divs)),
                    int(rng.choice(divs)), int(rng.integers(0, 2)) if ref >= 0 else 0, rc, waves, rows, kstep, ring,
                    int(rng.integers(0, 5)), str(rng.choice(["auto", "online", "fixed"]))))
    return out


RANDOM_SHAPED = _random_shaped_cases(48, 4096)


@pytest.mark.parametrize("case", RANDOM_SHAPED, ids=[c[0] for c in RANDOM_SHAPED])
def test_forward_random_geometries_any_launch_shape(dev, case):
    """Every element of O and every LSE row against the oracle for a random
    geometry in a random launch shape ("fixed" only where every head is
    eligible, else "auto")."""
    waves, rows, kstep, ring, deal, mode = case[14:]
    w, q, k, v = _small(case[:12], seed=8, key_offset=1.5)
    w = dataclasses.replace(w, ref_queries_global=case[12], ref_count=case[13])
    _say(f"[fwd-random-shape] {case}")
    qd, kd, vd = (_to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    bnd = fs.head_bounds(qd, kd, w)
    if mode == "fixed" and not bnd.host()["eligible"].all():
        mode = "auto"
    flags = fs.make_flags(mode, waves=waves, rows_per_wave=rows, key_step=kstep, ring=ring, deal=deal)
    assert fs.launch_info(tuple(qd.shape), fs.BF16, w, flags)[:3] == (waves, rows, kstep)
    lse = torch.empty((w.batch, w.heads, w.seq_len), dtype=torch.float32, device=dev)
    out = fs.forward(qd, kd, vd, fs.device_plan(w, dev), bnd, flags=flags, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention_ref(q, k, v, _geom(w))
    err = float(np.abs(out.float().cpu().numpy() - ref).max())
    assert err <= TOL["bf16"], err
    qn = float(np.linalg.norm(q.astype(np.float64), axis=-1).max())
    kn = float(np.linalg.norm(k.astype(np.float64), axis=-1).max())
    tol = LSE_TOL["bf16"] + w.head_dim * 2.0 ** -24 * qn * kn / math.sqrt(w.head_dim)
    assert float(np.abs(lse.cpu().numpy() - ref_lse).max()) <= tol


def test_forward_fp32_workload_deterministic(dev, config_inputs):
    """The fp32 path on the 5 x 48 workload: two runs bitwise equal, in the
    default launch and forced online."""
    w = workloads.workload(1)
    q, k, v = config_inputs(1)
    qd, kd, vd = (_to_dev(x, torch.float32, dev) for x in (q, k, v))
    dp = fs.device_plan(w, dev)
    b1 = fs.head_bounds(qd, kd, w)
    b2 = fs.head_bounds(qd, kd, w)
    outs = [fs.forward(qd, kd, vd, dp, b1, flags=fs.make_flags(m)) for m in ("auto", "auto", "online", "online")]
    torch.cuda.synchronize()
    assert torch.equal(b1.rec, b2.rec) and torch.equal(b1.key_mean, b2.key_mean)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[2], outs[3])


# Mask variants: the reference frames as global tokens in both directions
# (their own queries see every frame), and spans of several reference frames.
MASK_VARIANTS = [
    # (name, B, H, F, T, d, dtype, wb, wa, ref, bq, bk, ref_queries_global, ref_count)
    ("gref_mid", 1, 2, 6, 160, 128, "bf16", 1, 1, 2, 32, 32, 1, 0),
    ("gref0_d64", 2, 2, 5, 96, 64, "bf16", 0, 0, 0, 48, 16, 1, 0),
    ("gref_last_tail", 1, 3, 4, 240, 128, "bf16", 1, 0, 3, 48, 80, 1, 0),
    ("gref_f32", 1, 2, 4, 80, 128, "f32", 1, 0, 3, 16, 80, 1, 0),
    ("span2_mid", 1, 2, 7, 160, 128, "bf16", 1, 1, 3, 32, 32, 0, 2),
    ("span3_first_gref", 1, 2, 8, 96, 128, "bf16", 0, 1, 0, 48, 16, 1, 3),
    ("span2_last_d64", 2, 1, 6, 112, 64, "bf16", 1, 0, 4, 16, 112, 0, 2),
    ("span2_f32", 1, 2, 5, 80, 64, "f32", 1, 0, 2, 16, 80, 0, 2),
]


@pytest.mark.parametrize("case", MASK_VARIANTS, ids=[c[0] for c in MASK_VARIANTS])
@pytest.mark.parametrize("mode", ["auto", "online", "fixed"])
def test_forward_mask_variant_parity(dev, case, mode):
    w, q, k, v = _small(case[:12], seed=4, key_offset=1.5)
    w = dataclasses.replace(w, ref_queries_global=case[12], ref_count=case[13])
    _say(f"[fwd-variant] {w.name} mode={mode}")
    out, bnd, lse = _run(w, q, k, v, dev, flags=fs.make_flags(mode), lse=True)
    g = _geom(w)
    rec = oracle.head_bounds_ref(q, k, g)
    got = bnd.host()
    np.testing.assert_allclose(got["c_max"], rec["c_max"], rtol=1e-4, atol=1e-5 * float(rec["k_max"].max()))
    ref, ref_lse = oracle.attention_ref(q, k, v, g)
    err = np.abs(out.float().cpu().numpy() - ref).max()
    assert err <= TOL[w.dtype], err
    lerr = np.abs(lse.cpu().numpy() - ref_lse).max()
    assert lerr <= LSE_TOL[w.dtype], lerr


@pytest.mark.parametrize("variant", [(1, 0), (0, 2), (1, 3)], ids=["global_ref", "span2", "global_span3"])
def test_forward_mask_variant_full_size(dev, config_inputs, variant):
    """21 frames x 960 tokens with a global reference frame 0 (its rows see
    all 20,160 keys), with reference frames 0-1, and with global reference
    frames 0-2, in the library's default launch: bounds against the oracle,
    and every element of O against it."""
    w = dataclasses.replace(workloads.workload(2), ref_queries_global=variant[0], ref_count=variant[1])
    _say(f"[fwd-variant] {w.name} ref_queries_global={variant[0]} ref_count={variant[1]}")
    q, k, v = config_inputs(2)
    out, bnd, _ = _run(w, q, k, v, dev)
    g = _geom(w)
    rec = oracle.head_bounds_ref(q, k, g)
    got = bnd.host()
    np.testing.assert_allclose(got["c_max"], rec["c_max"], rtol=1e-4, atol=1e-5 * float(rec["k_max"].max()))
    assert np.array_equal(got["eligible"].astype(bool), rec["eligible"])
    ref, _ = _oracle_full(w, q, k, v)
    err = _max_abs_err(out, ref)
    _say(f"    max abs err {err:.3e} over every element")
    assert err <= TOL[w.dtype], err
    assert torch.isfinite(out.float()).all()


def test_online_and_fixed_agree_on_eligible_heads(dev, config_inputs):
    w = workloads.workload(2)
    q, k, v = config_inputs(2)
    on, _, _ = _run(w, q, k, v, dev, flags=fs.make_flags("online"))
    fx, bnd, _ = _run(w, q, k, v, dev, flags=fs.make_flags("fixed"))
    assert bnd.host()["eligible"].all()
    assert (on.float() - fx.float()).abs().max().item() <= TOL["bf16"]


def test_stressed_heads_fall_back_and_stay_finite(dev, config_inputs):
    w = workloads.workload(4)
    q, k, v = config_inputs(4)
    auto, bnd, _ = _run(w, q, k, v, dev)
    elig = bnd.host()["eligible"][0]
    assert [h for h in range(16) if not elig[h]] == list(workloads.STRESSED_HEADS)
    assert torch.isfinite(auto.float()).all()
    # forcing the fixed shift on a stressed head underflows whole rows (0/0):
    # the reason the online fallback exists
    fx, _, _ = _run(w, q, k, v, dev, flags=fs.make_flags("fixed"))
    bad = ~torch.isfinite(fx.float())
    assert bad[0, list(workloads.STRESSED_HEADS)].any()
    ok_heads = [h for h in range(16) if elig[h]]
    assert not bad[0, ok_heads].any()


def test_forward_deterministic(dev, config_inputs):
    w = workloads.workload(2)
    q, k, v = config_inputs(2)
    td = torch.bfloat16
    qd, kd, vd = (_to_dev(x, td, dev) for x in (q, k, v))
    dp = fs.device_plan(w, dev)
    bnd = fs.head_bounds(qd, kd, w)
    a = fs.forward(qd, kd, vd, dp, bnd)
    b = fs.forward(qd, kd, vd, dp, bnd)
    c = fs.forward(qd, kd, vd, dp, bnd, flags=fs.make_flags("online"))
    d = fs.forward(qd, kd, vd, dp, bnd, flags=fs.make_flags("online"))
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(c, d)


def test_binding_rejects_tensors_off_the_operands_gpu(dev):
    """A CPU tensor beside GPU operands (K, V, the output, the workspace, the
    plan or the angle tables) is rejected on the host with status 1, before
    anything is launched."""
    w = workloads.make_workload("devmix", 1, 2, 3, 80, 64, "bf16", 1, 1, 0, 16, 16)
    q = torch.zeros((1, 2, 240, 64), dtype=torch.bfloat16, device=dev)
    qc = q.cpu()
    dp = fs.device_plan(w, dev)
    bnd = fs.head_bounds(q, q, w)
    calls = [
        lambda: fs.head_bounds(q, qc, w),
        lambda: fs.head_bounds(q, q, w, workspace=torch.empty(1 << 20, dtype=torch.uint8)),
        lambda: fs.forward(q, q, qc, dp, bnd),
        lambda: fs.forward(q, q, q, dp, bnd, out=torch.empty_like(qc)),
        lambda: fs.forward(q, q, q, fs.device_plan(w, "cpu"), bnd),
        lambda: fs.produce(q, q, q, w, rope_cos=torch.zeros(240, 32), rope_sin=torch.zeros(240, 32)),
        lambda: fs.prior_art_forward(q, qc, q, w),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(fs.FsattnError) as e:
            call()
        assert e.value.status == 1, i
    torch.cuda.synchronize()


def test_mfma_probe_counts_and_runs(dev):
    """The matrix-unit reference loop reports 2 x its multiply-adds (4 waves x
    iters x 8 MFMAs of 16 x 16 x 32 per workgroup) and completes with finite
    results at a rate below the nominal bf16 peak."""
    wgs, iters = 512, 2000
    fs.mfma_probe(wgs, iters, dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    flops = fs.mfma_probe(wgs, iters, dev)
    b.record()
    torch.cuda.synchronize()
    assert flops == wgs * 4 * iters * 8 * 2 * 16 * 16 * 32
    tflops = flops / (a.elapsed_time(b) * 1e-3) / 1e12
    _say(f"[probe] {tflops:.0f} TFLOP/s")
    assert 0 < tflops < 2516.6 * 1.02


PRIOR_CASES = [
    # (name, B, H, F, T, d, dtype, wb, wa, ref, bq, bk): frames that do not divide 128, a padded
    # sequence end, reference frame outside / inside the window or absent, 16-token frames
    ("pa_240", 1, 2, 5, 240, 128, "bf16", 1, 1, 0, 48, 48),
    ("pa_noref_d64", 2, 1, 4, 96, 64, "bf16", 1, 0, -1, 16, 16),
    ("pa_ref_last", 1, 2, 7, 80, 128, "bf16", 1, 1, 6, 16, 16),
    ("pa_dense", 1, 1, 3, 256, 128, "bf16", 3, 3, 0, 64, 64),
    ("pa_t16", 1, 2, 9, 16, 128, "bf16", 2, 0, 4, 16, 16),
]


@pytest.mark.parametrize("case", PRIOR_CASES, ids=[c[0] for c in PRIOR_CASES])
def test_prior_art_comparator_parity(dev, case):
    """The prior-art comparator (128-token tiles, window and reference passes,
    merge) computes the same attention: every element against the oracle, in
    bf16 and fp32 output."""
    w, q, k, v = _small(case, seed=8, key_offset=0.5)
    ref, _ = oracle.attention_ref(q, k, v, _geom(w))
    qd, kd, vd = (_to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    for odt, tol in ((torch.bfloat16, TOL["bf16"]), (torch.float32, 5e-3)):
        _say(f"[prior-art] {w.name} out={odt}")
        out = fs.prior_art_forward(qd, kd, vd, w, out_dtype=odt)
        torch.cuda.synchronize()
        err = np.abs(out.float().cpu().numpy() - ref).max()
        assert err <= tol, (odt, err)


@pytest.mark.parametrize("i", [2, 5])
def test_prior_art_comparator_on_workloads(dev, config_inputs, i):
    """Full-size workloads: every element of the comparator's output against
    the fp64 oracle."""
    w = workloads.workload(i)
    q, k, v = config_inputs(i)
    qd, kd, vd = (_to_dev(x, torch.bfloat16, dev) for x in (q, k, v))
    _say(f"[prior-art] workload {i}")
    out = fs.prior_art_forward(qd, kd, vd, w)
    torch.cuda.synchronize()
    ref, _ = _oracle_full(w, q, k, v)
    err = _max_abs_err(out, ref)
    _say(f"    max abs err {err:.3e} over every element")
    assert err <= TOL["bf16"], err


# ------------------------------------------------------------------ producer (norm + rotary + layout)

def _packed_views(arrs, dtype, dev):
    """q, k, v (B, H, N, d) packed token-major as one [B, N, 3, H, d] tensor
    (a QKV projection's output) and the three [B, H, N, d] views into it."""
    qkv = torch.from_numpy(np.ascontiguousarray(np.stack(arrs, axis=2).transpose(0, 3, 2, 1, 4)))
    qkv = qkv.to(dtype).to(dev)
    return qkv, [qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3)]


def _produce_tol(dt, ref):
    # bf16: one ulp of the output (2^-7 relative) covers the rounding of an
    # fp32 result that may sit next to a rounding boundary; fp32: 1e-5
    return 2.0 ** -7 * np.abs(ref) + 1e-6 if dt == "bf16" else 1e-5


PRODUCE_CASES = [
    # (name, B, H, F, T, d, dtype, norm, rope, in_place)
    ("bf16_d128", 1, 3, 4, 96, 128, "bf16", True, True, False),
    ("bf16_d64_two_batches", 2, 2, 3, 80, 64, "bf16", True, True, False),
    ("bf16_norm_only", 1, 2, 3, 64, 128, "bf16", True, False, False),
    ("bf16_rope_only", 1, 2, 3, 64, 128, "bf16", False, True, False),
    ("bf16_copy_only", 1, 2, 3, 48, 64, "bf16", False, False, False),
    ("bf16_in_place", 1, 2, 5, 48, 128, "bf16", True, True, True),
    ("f32_d128", 1, 2, 3, 80, 128, "f32", True, True, False),
    ("f32_d64_in_place", 2, 1, 4, 48, 64, "f32", True, True, True),
]


@pytest.mark.parametrize("case", PRODUCE_CASES, ids=[c[0] for c in PRODUCE_CASES])
def test_produce_parity(dev, case):
    name, B, H, F_, T, d, dt, norm, rope, in_place = case
    _say(f"[produce] {name}")
    w = workloads.make_workload(name, B, H, F_, T, d, dt, 1, 1, 0, 16, 16)
    x = workloads.make_producer_inputs(w, seed=5)
    cos, sin = oracle.rope_tables_1d(w.seq_len, d)
    cos, sin = cos.astype(np.float32), sin.astype(np.float32)
    td = _tdtype(w)
    qkv, views = _packed_views((x["q"], x["k"], x["v"]), td, dev)
    gq = torch.from_numpy(x["gamma_q"]).to(dev) if norm else None
    gk = torch.from_numpy(x["gamma_k"]).to(dev) if norm else None
    tc = torch.from_numpy(cos).to(dev) if rope else None
    ts = torch.from_numpy(sin).to(dev) if rope else None
    out = tuple(views) if in_place else None
    q, k, v, bnd = fs.produce(*views, w, gq, gk, 1e-6, tc, ts, out=out)
    torch.cuda.synchronize()
    if in_place:
        assert q.data_ptr() == views[0].data_ptr()
    rq, rk, rv = oracle.produce_ref(x["q"], x["k"], x["v"], x["gamma_q"] if norm else None,
                                    x["gamma_k"] if norm else None, 1e-6, cos if rope else None,
                                    sin if rope else None)
    for got, ref, nm in ((q, rq, "q"), (k, rk, "k")):
        g = got.float().cpu().numpy()
        assert np.all(np.abs(g - ref) <= _produce_tol(dt, ref)), (nm, np.abs(g - ref).max())
    assert np.array_equal(v.float().cpu().numpy(), rv)             # V is copied unchanged
    # the bound records are those of the values written
    ref_b = fs.head_bounds(q, k, w)
    torch.cuda.synchronize()
    assert torch.equal(bnd.rec, ref_b.rec) and torch.equal(bnd.key_mean, ref_b.key_mean)


def _random_produce_cases(n, seed):
    """Seeded random producer geometries: frames of 16-640 tokens (one to
    five bounds chunks, the last one ragged), windows of 0-2 frames, no
    reference frame or spans of 1-2 (global or not), head_dim 64 or 128,
    bf16 or fp32, normalisation and rotation each on or off, in place or
    into new tensors."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        F_ = int(rng.integers(1, 6))
        ref = int(rng.integers(-1, F_))
        rc = int(rng.integers(0, 3)) if ref >= 0 else 0
        if ref + max(1, rc) > F_:
            rc = 0
        out.append((f"prnd{i}", int(rng.integers(1, 3)), int(rng.integers(1, 4)), F_, 16 * int(rng.integers(1, 41)),
                    int(rng.choice([64, 128])), "bf16" if rng.random() < 0.7 else "f32", int(rng.integers(0, 3)),
                    int(rng.integers(0, 3)), ref, int(rng.integers(0, 2)) if ref >= 0 else 0, rc,
                    bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


RANDOM_PRODUCE = _random_produce_cases(24, 77)


@pytest.mark.parametrize("case", RANDOM_PRODUCE, ids=[c[0] for c in RANDOM_PRODUCE])
def test_produce_random_geometries(dev, case):
    """Random producer geometries (seeded): Q and K against produce_ref, V
    copied exactly, the records equal bit for bit to fsattn_head_bounds on
    the outputs, and within rtol 1e-5 of the oracle's on them."""
    name, B, H, F_, T, d, dt, wb, wa, ref, gq, rc, norm, rope, in_place = case
    _say(f"[produce-random] {case}")
    w = workloads.make_workload(name, B, H, F_, T, d, dt, wb, wa, ref, 16, 16,
                                ref_queries_global=gq, ref_count=rc)
    x = workloads.make_producer_inputs(w, seed=9)
    cos, sin = oracle.rope_tables_1d(w.seq_len, d)
    cos, sin = cos.astype(np.float32), sin.astype(np.float32)
    td = _tdtype(w)
    qkv, views = _packed_views((x["q"], x["k"], x["v"]), td, dev)
    gqt = torch.from_numpy(x["gamma_q"]).to(dev) if norm else None
    gkt = torch.from_numpy(x["gamma_k"]).to(dev) if norm else None
    tc = torch.from_numpy(cos).to(dev) if rope else None
    ts = torch.from_numpy(sin).to(dev) if rope else None
    q, k, v, bnd = fs.produce(*views, w, gqt, gkt, 1e-6, tc, ts, out=tuple(views) if in_place else None)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.produce_ref(x["q"], x["k"], x["v"], x["gamma_q"] if norm else None,
                                    x["gamma_k"] if norm else None, 1e-6, cos if rope else None,
                                    sin if rope else None)
    qn, kn = q.float().cpu().numpy(), k.float().cpu().numpy()
    for g, r, nm in ((qn, rq, "q"), (kn, rk, "k")):
        assert np.all(np.abs(g - r) <= _produce_tol(dt, r)), (nm, np.abs(g - r).max())
    assert np.array_equal(v.float().cpu().numpy(), rv)
    ref_b = fs.head_bounds(q, k, w)
    torch.cuda.synchronize()
    assert torch.equal(bnd.rec, ref_b.rec) and torch.equal(bnd.key_mean, ref_b.key_mean)
    got, orc = bnd.host(), oracle.head_bounds_ref(qn, kn, _geom(w))
    for nm, rn in (("q_norm_max", "q_max"), ("k_norm_max", "k_max"), ("gap_est", "gap_est")):
        np.testing.assert_allclose(got[nm], orc[rn], rtol=1e-5, err_msg=nm)
    np.testing.assert_allclose(got["c_max"], orc["c_max"], rtol=1e-4, atol=1e-5 * float(orc["k_max"].max()))
    assert np.array_equal(got["eligible"].astype(bool), orc["eligible"])


def test_produce_then_forward_full_size(dev):
    """6 frames x 8160 tokens, 4 heads, d = 128, bf16 (the RMS-normalised
    workload's shape) from raw token-major projections: fsattn_produce
    (RMSNorm + rotary embedding + layout + bounds), then the forward in the
    library's default launch. Checked: Q, K, V against the oracle on every
    element; the bound records bit for bit against fsattn_head_bounds on the
    outputs and against the oracle; every element of O against the
    oracle's attention on the produced Q, K, V."""
    w = workloads.workload(5)
    _say(f"[produce] {w.name} full size, then forward")
    x = workloads.make_producer_inputs(w, seed=6)
    qkv, views = _packed_views((x["q"], x["k"], x["v"]), torch.bfloat16, dev)
    args = [torch.from_numpy(x[n]).to(dev) for n in ("gamma_q", "gamma_k")]
    tabs = [torch.from_numpy(x[n]).to(dev) for n in ("cos", "sin")]
    q, k, v, bnd = fs.produce(*views, w, args[0], args[1], workloads.RMS_EPS, tabs[0], tabs[1])
    dp = fs.device_plan(w, dev)
    o = fs.forward(q, k, v, dp, bnd)
    ref_b = fs.head_bounds(q, k, w)
    torch.cuda.synchronize()
    assert torch.equal(bnd.rec, ref_b.rec) and torch.equal(bnd.key_mean, ref_b.key_mean)
    rq, rk, rv = oracle.produce_ref(x["q"], x["k"], x["v"], x["gamma_q"], x["gamma_k"], workloads.RMS_EPS,
                                    x["cos"], x["sin"])
    qn, kn, vn = (t.float().cpu().numpy() for t in (q, k, v))
    for g, ref, nm in ((qn, rq, "q"), (kn, rk, "k")):
        assert np.all(np.abs(g - ref) <= _produce_tol("bf16", ref)), (nm, np.abs(g - ref).max())
    assert np.array_equal(vn, rv)
    g = _geom(w)
    rec = oracle.head_bounds_ref(qn, kn, g)
    got = bnd.host()
    np.testing.assert_allclose(got["bound"], rec["bound"], rtol=1e-5)
    assert np.array_equal(got["eligible"].astype(bool), rec["eligible"])
    t0 = time.perf_counter()
    ref_o, _ = oracle.attention_live_ref(qn, kn, vn, g)
    _say(f"    oracle (fp64, every row) {time.perf_counter() - t0:.1f} s")
    err = _max_abs_err(o, ref_o)
    _say(f"    max abs err {err:.3e} over every element")
    assert err <= TOL["bf16"], err


# ------------------------------------------------------------------ degenerate inputs

DEGENERATE = ["q_zero", "keys_equal", "v_constant", "wide_logits"]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("kind", DEGENERATE)
def test_forward_degenerate_inputs(dev, kind, dt):
    """Degenerate cases of the method, in the library's default launch:
    Q = 0 (every logit 0: the bound, gap and shift are 0 and each row is the
    mean of its live V rows); all keys equal (K_max = C_max = 0: the shift is
    exact); V constant (every row is that constant); and logits with a spread
    of tens of nats (the heads fail eligibility and take the online path)."""
    _say(f"[fwd-degenerate] {kind} {dt}")
    w = workloads.make_workload(f"deg_{kind}", 1, 2, 4, 96, 128 if dt == "bf16" else 64, dt, 1, 1, 0, 48, 32)
    q, k, v = workloads.make_inputs(w, seed=8)
    if kind == "q_zero":
        q = np.zeros_like(q)
    elif kind == "keys_equal":
        k = np.broadcast_to(k[:, :, :1, :], k.shape).copy()
    elif kind == "v_constant":
        v = np.broadcast_to(v[:, :, :1, :], v.shape).copy()
    elif kind == "wide_logits":
        q, k = q * np.float32(3.0), k * np.float32(3.0)
        if dt == "bf16":
            q, k = workloads.round_to_bf16(q), workloads.round_to_bf16(k)
    out, bnd, lse = _run(w, q, k, v, dev, lse=True)
    o = out.float().cpu().numpy()
    rec = bnd.host()
    g = _geom(w)
    ref, ref_lse = oracle.attention_ref(q, k, v, g)
    assert np.isfinite(o).all() and np.isfinite(lse.cpu().numpy()).all()
    assert np.abs(o - ref).max() <= TOL[dt], np.abs(o - ref).max()
    # Log-sum-exp bound: LSE_TOL covers the rounding of the weights; with
    # logits of tens of nats the fp32 rounding of the logits themselves also
    # counts: a d-term fp32 dot product is off by at most d * 2^-24 times
    # scale * sum |q_t k_t| <= scale * |q| |k|, so the bound adds that term
    # (negligible for the other inputs here).
    qn = np.linalg.norm(q.astype(np.float64), axis=-1).max()
    kn = np.linalg.norm(k.astype(np.float64), axis=-1).max()
    lse_tol = LSE_TOL[dt] + w.head_dim * 2.0 ** -24 * qn * kn / math.sqrt(w.head_dim)
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= lse_tol
    if kind == "q_zero":
        assert np.all(rec["bound"] == 0) and np.all(rec["gap_est"] == 0) and rec["eligible"].all()
        M = oracle.token_mask(g)
        mean_v = (M.astype(np.float64) @ v[0, 0].astype(np.float64)) / M.sum(axis=1, keepdims=True)
        assert np.abs(o[0, 0] - mean_v).max() <= TOL[dt]
    elif kind == "keys_equal":
        # (exactly 0 for bf16 keys: the sums of equal bf16 values are exact in fp32)
        kn = float(np.linalg.norm(k[0, 0, 0]))
        assert np.all(rec["k_norm_max"] <= 1e-6 * kn) and np.all(rec["c_max"] <= 1e-6 * kn)
        assert rec["eligible"].all()
    elif kind == "v_constant":
        assert np.abs(o - v[:, :, :1, :]).max() <= (2.0 ** -8 if dt == "bf16" else 2e-6) * np.abs(v).max()
    elif kind == "wide_logits":
        assert not rec["eligible"].any(), rec["gap_est"]
