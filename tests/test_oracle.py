"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: hand-derived plans
(tests/golden), closed-form counts, a brute-force token loop with math.exp,
torch's fp64 scaled_dot_product_attention on dense masks, closed forms
(Q = 0, constant V, common key offset, permutations), shift invariance of
the softmax, and Cauchy-Schwarz for the bounds. Mutation tests plant
plausible mistakes in the oracle (on the CPU) and check that a pin fails.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.fsattn_oracle as O
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _geom(t):
    return oracle.MaskGeometry(*t)


# the two attention oracles: dense scores with -inf outside the mask, and the
# same sums taken over each row's live keys only; every attention pin runs on both
ATTN_IMPLS = [oracle.attention_ref, oracle.attention_live_ref]
ATTN_IDS = ["dense", "live_keys"]


def _rand_qkv(rng, B, H, N, d, kscale=1.0):
    q = rng.standard_normal((B, H, N, d))
    k = kscale * rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    return q, k, v


# ------------------------------------------------------------------ plan

def test_plan_matches_hand_derived_golden():
    cases = json.load(open(os.path.join(GOLDEN, "plan_tiny.json")))["cases"]
    for c in cases:
        rp, ci = oracle.plan_bruteforce(_geom(c["mask"]))
        assert rp.tolist() == c["row_ptr"], c["name"]
        assert ci.tolist() == c["col_idx"], c["name"]


def test_plan_sizes_of_workloads_match_hand_counts():
    gold = {w["name"]: w for w in json.load(open(os.path.join(GOLDEN, "workload_plan_sizes.json")))["workloads"]}
    for w in workloads.WORKLOADS:
        g = _geom(w.mask_tuple())
        want = gold[w.name]
        assert [len(oracle.live_frames(g, f)) for f in range(g.F)] == want["live_frames_per_frame"]
        if g.N <= 20160:       # brute force at the larger sizes runs in the slow suite
            rp, ci = oracle.plan_bruteforce(g)
            assert len(rp) - 1 == want["num_q_blocks"]
            assert len(ci) == want["nnz"]


@pytest.mark.slow
def test_plan_sizes_of_large_workloads_bruteforce():
    gold = {w["name"]: w for w in json.load(open(os.path.join(GOLDEN, "workload_plan_sizes.json")))["workloads"]}
    for w in workloads.WORKLOADS:
        g = _geom(w.mask_tuple())
        rp, ci = oracle.plan_bruteforce(g)
        assert len(ci) == gold[w.name]["nnz"]


def test_plan_invariants_random_geometries():
    rng = np.random.default_rng(7)
    for _ in range(40):
        T = 16 * int(rng.integers(1, 7))
        divs = [b for b in range(16, T + 1, 16) if T % b == 0]
        g = oracle.MaskGeometry(int(rng.integers(1, 8)), T, int(rng.integers(0, 4)), int(rng.integers(0, 4)),
                                int(rng.integers(-1, 3)), int(rng.choice(divs)), int(rng.choice(divs)),
                                int(rng.integers(0, 2)), int(rng.integers(0, 3)))
        if g.r + g.nr > g.F:
            g = oracle.MaskGeometry(g.F, g.T, g.wb, g.wa, -1, g.bq, g.bk)
        rp, ci = oracle.plan_bruteforce(g)
        assert rp[0] == 0 and np.all(np.diff(rp) >= 1)     # every row sees its own frame
        for qb in range(len(rp) - 1):
            row = ci[rp[qb]:rp[qb + 1]]
            assert np.all(np.diff(row) > 0)
        # closed form: sum_f |L(f)| * (T/bq) * (T/bk)
        nnz = sum(len(oracle.live_frames(g, f)) for f in range(g.F)) * (T // g.bq) * (T // g.bk)
        assert len(ci) == nnz
        # exhaustive token-level check: a listed block is all-live, an unlisted one all-masked
        M = oracle.token_mask(g)
        for qb in range(len(rp) - 1):
            listed = set(ci[rp[qb]:rp[qb + 1]].tolist())
            for kb in range(g.N // g.bk):
                blk = M[qb * g.bq:(qb + 1) * g.bq, kb * g.bk:(kb + 1) * g.bk]
                assert blk.all() if kb in listed else not blk.any()


def test_invalid_geometry_rejected():
    bad = [
        (3, 48, 1, 1, 0, 32, 16),    # 32 does not divide 48
        (3, 48, 1, 1, 0, 24, 16),    # 24 not a multiple of 16
        (3, 48, 1, 1, 0, 0, 16),
        (3, 48, -1, 1, 0, 16, 16),
        (3, 48, 1, 1, 3, 16, 16),    # reference frame out of range
        (3, 48, 1, 1, -2, 16, 16),
        (3, 48, 1, 1, 0, 16, 16, 2),  # ref_queries_global is 0 or 1
        (3, 48, 1, 1, 2, 16, 16, 0, 2),   # reference span past the last frame
        (3, 48, 1, 1, 0, 16, 16, 0, -1),
    ]
    for t in bad:
        with pytest.raises(ValueError):
            oracle.plan_bruteforce(_geom(t))


def test_partial_block_count_under_coarse_tiles_hand_example():
    # 2 frames x 48 tokens, block-diagonal mask, 32-token tiles over 96 tokens:
    # live tiles (0,0) (0,1) (1,0) (1,1) (1,2) (2,1) (2,2); only (0,0) and (2,2) are full.
    g = oracle.MaskGeometry(2, 48, 0, 0, -1, 16, 16)
    assert oracle.partial_blocks_if_tiled(g, 32) == (5, 7)
    # aligned tiles are never partial
    assert oracle.partial_blocks_if_tiled(g, 48)[0] == 0
    assert oracle.partial_blocks_if_tiled(g, 16)[0] == 0


# ------------------------------------------------------------------ attention

def _bruteforce_attention(q, k, v, F, T, wb, wa, r, scale, rg=0, nr=0):
    """Token-by-token softmax with math.exp; the mask is written as frame
    membership tests, independent of the oracle's vectorised rule."""
    B, H, N, d = q.shape
    refs = list(range(r, r + max(1, nr))) if r >= 0 else []
    out = np.zeros((B, H, N, d))
    lse = np.zeros((B, H, N))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                fi = i // T
                live = []
                for j in range(N):
                    fj = j // T
                    if fj in range(fi - wb, fi + wa + 1) or fj in refs or (rg and fi in refs):
                        live.append(j)
                logits = [scale * sum(q[b, h, i, t] * k[b, h, j, t] for t in range(d)) for j in live]
                mx = max(logits)
                w = [math.exp(x - mx) for x in logits]
                tot = sum(w)
                for t in range(d):
                    out[b, h, i, t] = sum(wj * v[b, h, j, t] for wj, j in zip(w, live)) / tot
                lse[b, h, i] = mx + math.log(tot)
    return out, lse


@pytest.mark.parametrize("geom", [(3, 4, 1, 1, 0), (4, 3, 0, 1, 2), (5, 2, 1, 0, -1), (2, 5, 0, 0, 1),
                                  (4, 3, 0, 0, 2, 1), (5, 2, 1, 0, 0, 1), (6, 2, 0, 0, 1, 0, 3),
                                  (5, 3, 1, 0, 2, 1, 2)])
@pytest.mark.parametrize("attn", ATTN_IMPLS, ids=ATTN_IDS)
def test_attention_matches_bruteforce_loops(attn, geom):
    F, T, wb, wa, r = geom[:5]
    rg = geom[5] if len(geom) > 5 else 0
    nr = geom[6] if len(geom) > 6 else 0
    rng = np.random.default_rng(F * 100 + T)
    q, k, v = _rand_qkv(rng, 1, 2, F * T, 5)
    g = oracle.MaskGeometry(F, T, wb, wa, r, 16, 16, rg, nr)     # blocks unused by attention_ref
    o, lse = attn(q, k, v, g, scale=0.7)
    ob, lb = _bruteforce_attention(q, k, v, F, T, wb, wa, r, 0.7, rg, nr)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


@pytest.mark.parametrize("attn", ATTN_IMPLS, ids=ATTN_IDS)
def test_attention_dense_matches_torch_sdpa(attn):
    import torch
    rng = np.random.default_rng(3)
    F, T, d = 4, 24, 16
    q, k, v = _rand_qkv(rng, 2, 3, F * T, d)
    g = oracle.MaskGeometry(F, T, F, F, 0, 16, 16)       # window covers everything
    o, _ = attn(q, k, v, g)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("attn", ATTN_IMPLS, ids=ATTN_IDS)
def test_attention_windowed_matches_torch_sdpa_with_boolean_mask(attn):
    import torch
    rng = np.random.default_rng(4)
    F, T, d = 6, 16, 8
    q, k, v = _rand_qkv(rng, 1, 2, F * T, d)
    g = oracle.MaskGeometry(F, T, 1, 2, 5, 16, 16)
    o, _ = attn(q, k, v, g, scale=0.3)
    fr = np.arange(F * T) // T
    allowed = np.zeros((F * T, F * T), dtype=bool)
    for i in range(F * T):
        for j in range(F * T):
            allowed[i, j] = (fr[i] - 1 <= fr[j] <= fr[i] + 2) or fr[j] == 5
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(allowed), scale=0.3).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("attn", ATTN_IMPLS, ids=ATTN_IDS)
def test_attention_closed_forms(attn):
    rng = np.random.default_rng(5)
    F, T, d = 5, 16, 8
    g = oracle.MaskGeometry(F, T, 1, 1, 0, 16, 16)
    q, k, v = _rand_qkv(rng, 1, 2, F * T, d)
    # Q = 0: every live key has weight 1/|live|, so O_i is the mean of V over row i's live keys
    o, lse = attn(np.zeros_like(q), k, v, g)
    for i in range(F * T):
        live = [j for j in range(F * T) if j // T in oracle.live_frames(g, i // T)]
        np.testing.assert_allclose(o[:, :, i], v[:, :, live].mean(axis=2), atol=1e-12)
        np.testing.assert_allclose(lse[:, :, i], math.log(len(live)), atol=1e-12)
    # V rows all equal to c: O = c
    c = rng.standard_normal(d)
    o, _ = attn(q, k, np.broadcast_to(c, v.shape), g)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-12)
    # common key offset k_j + c adds q_i . c to every logit of row i: O unchanged
    o0, lse0 = attn(q, k, v, g)
    o1, lse1 = attn(q, k + 3.0 * c, v, g)
    np.testing.assert_allclose(o1, o0, atol=1e-11)
    np.testing.assert_allclose(lse1 - lse0, 3.0 * (q @ c) / math.sqrt(d), atol=1e-10)
    # permuting tokens inside each frame permutes the output rows the same way
    perm = np.concatenate([f * T + rng.permutation(T) for f in range(F)])
    o2, _ = attn(q[:, :, perm], k[:, :, perm], v[:, :, perm], g)
    np.testing.assert_allclose(o2, o0[:, :, perm], atol=1e-12)
    # scaling q by a with scale 1/a is the same softmax
    o3, _ = attn(2.0 * q, k, v, g, scale=0.5 / math.sqrt(d))
    np.testing.assert_allclose(o3, o0, atol=1e-12)


@pytest.mark.parametrize("attn", ATTN_IMPLS, ids=ATTN_IDS)
def test_attention_rows_subset_matches_full(attn):
    rng = np.random.default_rng(6)
    g = oracle.MaskGeometry(4, 32, 1, 1, 0, 16, 16)
    q, k, v = _rand_qkv(rng, 1, 2, 128, 8)
    o, lse = attn(q, k, v, g)
    rows = [0, 5, 31, 32, 77, 127]
    os_, ls_ = attn(q, k, v, g, rows=rows)
    # (a subset changes only the matrix products' blocking: equal to rounding)
    np.testing.assert_allclose(os_, o[:, :, rows], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ls_, lse[:, :, rows], rtol=0, atol=1e-14)


def test_shift_invariance_online_fixed_and_max():
    rng = np.random.default_rng(8)
    g = oracle.MaskGeometry(5, 16, 1, 1, 0, 16, 16)
    q, k, v = _rand_qkv(rng, 1, 2, 80, 8, kscale=2.0)
    k = k + 5.0                                       # large common key component
    o_ref, _ = oracle.attention_ref(q, k, v, g)
    o_on = oracle.attention_online_ref(q, k, v, g, key_block=16)
    np.testing.assert_allclose(o_on, o_ref, rtol=1e-12, atol=1e-13)
    rec = oracle.head_bounds_ref(q, k, g)
    for per_row in (False, True):
        sh = oracle.row_shift_ref(q, rec, per_row=per_row)
        o_fx = oracle.attention_fixed_shift_ref(q, k, v, g, sh)
        np.testing.assert_allclose(o_fx, o_ref, rtol=1e-12, atol=1e-13)
    # an arbitrary (even wrong-side) shift is still exact in fp64 while nothing under/overflows
    o_any = oracle.attention_fixed_shift_ref(q, k, v, g, rng.standard_normal((1, 2, 80)) * 3)
    np.testing.assert_allclose(o_any, o_ref, rtol=1e-12, atol=1e-13)


def test_mean_centring_leaves_output_unchanged():
    rng = np.random.default_rng(9)
    g = oracle.MaskGeometry(4, 16, 1, 1, 0, 16, 16)
    q, k, v = _rand_qkv(rng, 1, 1, 64, 8)
    k = k + rng.standard_normal(8) * 4
    rec = oracle.head_bounds_ref(q, k, g)
    o0, _ = oracle.attention_ref(q, k, v, g)
    o1, _ = oracle.attention_ref(q, k - rec["mu"][:, :, None, :], v, g)
    np.testing.assert_allclose(o1, o0, atol=1e-12)


# ------------------------------------------------------------------ bounds

def test_bounds_hand_example():
    # d = 2, one frame of 16 keys: 8 x (13, 14) and 8 x (7, 6); mean (10, 10),
    # every centred key is +-(3, 4) with norm 5. One query (6, 8) of norm 10,
    # the others zero. scale 1/sqrt(2): bound = 50/sqrt(2); single frame => c_max = 0.
    k = np.zeros((1, 1, 16, 2)); k[0, 0, :8] = (13, 14); k[0, 0, 8:] = (7, 6)
    q = np.zeros((1, 1, 16, 2)); q[0, 0, 3] = (6, 8)
    g = oracle.MaskGeometry(1, 16, 0, 0, -1, 16, 16)
    rec = oracle.head_bounds_ref(q, k, g)
    np.testing.assert_allclose(rec["mu"][0, 0], [10, 10])
    assert rec["q_max"][0, 0] == pytest.approx(10)
    assert rec["k_max"][0, 0] == pytest.approx(5)
    assert rec["bound"][0, 0] == pytest.approx(50 / math.sqrt(2))
    assert rec["c_max"][0, 0] == pytest.approx(0, abs=1e-12)
    # the bound is attained: q = (6,8) is parallel to the centred key (3,4)
    s = oracle.live_logit_stats(q, k, g, rec["mu"])
    assert s.max() == pytest.approx(50 / math.sqrt(2))


def test_bounds_two_frame_window_mean_hand_example():
    # 2 frames x 16 keys in d = 1, no reference frame, window 0 (block diagonal):
    # frame 0 keys all +1, frame 1 keys all -3; mu = -1; every centred key has norm 2;
    # each frame's live set is itself: window means +1 and -3, |mean - mu| = 2 for both.
    k = np.zeros((1, 1, 32, 1)); k[0, 0, :16] = 1.0; k[0, 0, 16:] = -3.0
    q = np.full((1, 1, 32, 1), 0.5)
    g = oracle.MaskGeometry(2, 16, 0, 0, -1, 16, 16)
    rec = oracle.head_bounds_ref(q, k, g, scale=1.0)
    assert rec["mu"][0, 0, 0] == pytest.approx(-1)
    assert rec["k_max"][0, 0] == pytest.approx(2)
    assert rec["c_max"][0, 0] == pytest.approx(2)
    assert rec["bound"][0, 0] == pytest.approx(1.0)
    assert rec["gap_est"][0, 0] == pytest.approx(2.0)
    # with the window covering both frames, the live mean is the global mean: c_max = 0
    g2 = oracle.MaskGeometry(2, 16, 1, 1, -1, 16, 16)
    assert oracle.head_bounds_ref(q, k, g2, scale=1.0)["c_max"][0, 0] == pytest.approx(0, abs=1e-12)


def test_bounds_global_reference_frame_hand_example():
    # 3 frames x 16 keys in d = 1, window 0, reference frame 0: keys 4, 0, 2 per
    # frame; mu = 2, every centred key has norm <= 2 (k_max = 2). Keys only:
    # f0 sees {0} (mean 4), f1 {0,1} (mean 2), f2 {0,2} (mean 3): c_max = 2.
    # Global reference frame: f0 sees all frames (mean 2 = mu): c_max = 1.
    k = np.zeros((1, 1, 48, 1)); k[0, 0, :16] = 4.0; k[0, 0, 32:] = 2.0
    q = np.full((1, 1, 48, 1), 0.5)
    for rg, c_max in ((0, 2.0), (1, 1.0)):
        rec = oracle.head_bounds_ref(q, k, oracle.MaskGeometry(3, 16, 0, 0, 0, 16, 16, rg), scale=1.0)
        assert rec["mu"][0, 0, 0] == pytest.approx(2)
        assert rec["k_max"][0, 0] == pytest.approx(2)
        assert rec["c_max"][0, 0] == pytest.approx(c_max)
        assert rec["gap_est"][0, 0] == pytest.approx(0.5 * (2 + c_max))


def test_bounds_reference_span_hand_example():
    # 4 frames x 16 keys in d = 1, window 0, reference frames 0-1 (span 2):
    # keys 6, 2, 0, -4 per frame; mu = 1, k_max = |-4 - 1| = 5. Frames 0 and 1
    # see {0,1} (mean 4), frame 2 {0,1,2} (mean 8/3), frame 3 {0,1,3} (mean 4/3):
    # c_max = 3. One reference frame 0 instead: f0 {0} (6), f1 {0,1} (4),
    # f2 {0,2} (3), f3 {0,3} (1): c_max = 5.
    k = np.zeros((1, 1, 64, 1))
    for f, val in enumerate((6.0, 2.0, 0.0, -4.0)):
        k[0, 0, 16 * f:16 * (f + 1)] = val
    q = np.full((1, 1, 64, 1), 0.25)
    for nr, c_max in ((2, 3.0), (1, 5.0), (0, 5.0)):
        rec = oracle.head_bounds_ref(q, k, oracle.MaskGeometry(4, 16, 0, 0, 0, 16, 16, 0, nr), scale=1.0)
        assert rec["mu"][0, 0, 0] == pytest.approx(1)
        assert rec["k_max"][0, 0] == pytest.approx(5)
        assert rec["c_max"][0, 0] == pytest.approx(c_max)
        assert rec["gap_est"][0, 0] == pytest.approx(0.25 * (5 + c_max))


def test_bounds_degenerate_cases():
    rng = np.random.default_rng(10)
    g = oracle.MaskGeometry(3, 16, 1, 1, 0, 16, 16)
    q = rng.standard_normal((1, 2, 48, 8))
    k = np.broadcast_to(rng.standard_normal(8), (1, 2, 48, 8)).copy()      # all keys equal
    rec = oracle.head_bounds_ref(q, k, g)
    np.testing.assert_allclose(rec["k_max"], 0, atol=1e-12)
    np.testing.assert_allclose(rec["bound"], 0, atol=1e-12)
    np.testing.assert_allclose(rec["c_max"], 0, atol=1e-12)
    assert rec["eligible"].all()
    rec0 = oracle.head_bounds_ref(np.zeros_like(q), rng.standard_normal((1, 2, 48, 8)), g)
    np.testing.assert_allclose(rec0["bound"], 0)
    np.testing.assert_allclose(rec0["gap_est"], 0)


def test_bounds_translation_invariance():
    rng = np.random.default_rng(11)
    g = oracle.MaskGeometry(4, 16, 1, 1, 0, 16, 16)
    q, k, _ = _rand_qkv(rng, 1, 2, 64, 8)
    c = rng.standard_normal(8) * 10
    r0 = oracle.head_bounds_ref(q, k, g)
    r1 = oracle.head_bounds_ref(q, k + c, g)
    np.testing.assert_allclose(r1["mu"], r0["mu"] + c, atol=1e-12)
    for key in ("k_max", "c_max", "bound", "gap_est"):
        np.testing.assert_allclose(r1[key], r0[key], rtol=1e-11)


def _check_bound_audit(q, k, g, rows=None):
    rec = oracle.head_bounds_ref(q, k, g)
    stats = oracle.live_logit_stats(q, k, g, rec["mu"], rows=rows)     # (B, H, R) centred row maxima
    bound = rec["bound"][:, :, None]
    assert np.all(bound >= stats - 1e-12 * np.abs(stats))              # bound >= every live logit
    row_gaps = bound - stats
    assert np.all(rec["gap_est"][:, :, None] >= row_gaps - 1e-9)      # gap_est >= every row gap
    head_gap = rec["bound"] - stats.max(axis=2)
    assert np.all(rec["gap_est"] >= head_gap - 1e-9)
    return rec, stats


def test_bound_audit_exhaustive_small():
    rng = np.random.default_rng(12)
    for geom in [(5, 16, 1, 1, 0, 0), (6, 16, 2, 0, 3, 0), (4, 32, 0, 0, -1, 0), (7, 16, 1, 1, 0, 0),
                 (5, 16, 1, 1, 2, 1), (6, 16, 0, 1, 0, 1), (7, 16, 0, 0, 2, 0, 3), (6, 16, 1, 0, 4, 1, 2)]:
        F, T, wb, wa, r, rg = geom[:6]
        nr = geom[6] if len(geom) > 6 else 0
        q, k, _ = _rand_qkv(rng, 2, 2, F * T, 8)
        k = k + rng.standard_normal(8) * 3
        _check_bound_audit(q, k, oracle.MaskGeometry(F, T, wb, wa, r, 16, 16, rg, nr))


def test_bound_audit_workload1_exhaustive(config_inputs):
    q, k, _ = config_inputs(1)
    rec, stats = _check_bound_audit(q, k, _geom(workloads.workload(1).mask_tuple()))
    assert rec["eligible"].all()


@pytest.mark.parametrize("i", [2, 3, 5])
def test_bound_audit_workloads_sampled_rows_and_eligibility(config_inputs, i):
    q, k, _ = config_inputs(i)
    w = workloads.workload(i)
    g = _geom(w.mask_tuple())
    rows = np.random.default_rng(i).choice(g.N, 24, replace=False)
    rec, _ = _check_bound_audit(q, k, g, rows=rows)
    assert rec["eligible"].all()
    assert np.all(rec["gap_est"] < 25.0)


def test_workload3_needs_mean_centring(config_inputs):
    """Keys carry a per-head mean offset; the raw (uncentred) bound is above 30
    nats while the centred one qualifies - the reason centring is done."""
    q, k, _ = config_inputs(3)
    g = _geom(workloads.workload(3).mask_tuple())
    rec = oracle.head_bounds_ref(q, k, g)
    scale = 1 / math.sqrt(128)
    raw_kmax = np.sqrt((np.asarray(k, np.float64) ** 2).sum(-1)).max(-1)
    raw_bound = scale * rec["q_max"] * raw_kmax
    assert np.all(raw_bound > 30.0)
    assert rec["eligible"].all()


def test_workload4_stressed_heads_fail_eligibility(config_inputs):
    q, k, _ = config_inputs(4)
    g = _geom(workloads.workload(4).mask_tuple())
    rec = oracle.head_bounds_ref(q, k, g)
    elig = rec["eligible"][0]
    assert [h for h in range(16) if not elig[h]] == list(workloads.STRESSED_HEADS)
    assert np.all(rec["gap_est"][0, list(workloads.STRESSED_HEADS)] > 100.0)
    # for such a head fp32 exp of (logit - shift) underflows to zero for whole rows
    assert np.float32(np.exp(np.float32(-104.0))) == 0.0
    rows = np.arange(0, g.N, 997)
    stats = oracle.live_logit_stats(q[:, 5:6], k[:, 5:6], g, rec["mu"][:, 5:6], rows=rows)
    gaps = rec["bound"][0, 5] - stats[0, 0]
    assert np.any(gaps > 104.0)


# ------------------------------------------------------------------ the fixed shift and the threshold
# ("Unchaining the Softmax": each row starts from a bound on its logits; the
# bound must sit at or above every live logit of the row, and eligibility is
# "bound minus logit max <= 30 nats", decided per head)

def _raw_live_row_max(q, k, g, scale):
    """max over row i's live keys of the raw logit scale * q_i . k_j, by a loop
    over rows with the live keys taken from row_mask (no mean, no bound)."""
    B, H, N, d = q.shape
    out = np.empty((B, H, N))
    for i in range(N):
        live = np.nonzero(oracle.row_mask(g, i))[0]
        for b in range(B):
            for h in range(H):
                out[b, h, i] = max(scale * float(np.dot(q[b, h, i], k[b, h, j])) for j in live)
    return out


def _check_shift_audit(q, k, g):
    """Both shift variants of each row: at least the row's largest raw live
    logit (so no exponential exceeds 1 and none overflows), and at most the
    head's gap estimate above it (so the largest term of an eligible head's
    row is at least e^-30)."""
    d = q.shape[-1]
    scale = 1 / math.sqrt(d)
    rec = oracle.head_bounds_ref(q, k, g)
    rmax = _raw_live_row_max(q, k, g, scale)
    for per_row in (False, True):
        sh = oracle.row_shift_ref(q, rec, per_row=per_row)
        assert np.all(sh >= rmax - 1e-12 * np.abs(rmax)), per_row
        assert np.all(sh - rmax <= rec["gap_est"][:, :, None] + 1e-9), per_row


SHIFT_GEOMS = [(5, 16, 1, 1, 0, 0, 0), (6, 16, 2, 0, 3, 0, 0), (4, 16, 0, 0, -1, 0, 0),
               (5, 16, 1, 1, 2, 1, 0), (7, 16, 0, 0, 2, 0, 3), (3, 16, 2, 2, 0, 0, 0)]


def test_row_shift_bounds_every_raw_live_logit():
    """Exhaustive over every (row, live key) pair of small geometries whose keys
    carry a large common offset (so q_i . mu_h is large and of either sign)."""
    rng = np.random.default_rng(40)
    for F, T, wb, wa, r, rg, nr in SHIFT_GEOMS:
        g = oracle.MaskGeometry(F, T, wb, wa, r, 16, 16, rg, nr)
        q, k, _ = _rand_qkv(rng, 2, 2, F * T, 8)
        k = k + rng.standard_normal(8) * 6.0
        _check_shift_audit(q, k, g)


def test_row_shift_hand_values():
    # the geometry of test_bounds_hand_example: keys 8 x (13, 14) and 8 x (7, 6),
    # mean (10, 10), centred keys +-(3, 4) of norm 5; query row 3 is (6, 8) of
    # norm 10, every other query is 0; scale 1/sqrt(2). bound = 10 * 5 / sqrt(2).
    # Row 3: q . mu = 140, so both shifts are (50 + 140) / sqrt(2) = 190 / sqrt(2),
    # which is its raw logit against (13, 14): 6 * 13 + 8 * 14 = 190. Zero rows:
    # default shift = bound = 50 / sqrt(2), per-row shift = 0 (their logits are 0).
    k = np.zeros((1, 1, 16, 2)); k[0, 0, :8] = (13, 14); k[0, 0, 8:] = (7, 6)
    q = np.zeros((1, 1, 16, 2)); q[0, 0, 3] = (6, 8)
    g = oracle.MaskGeometry(1, 16, 0, 0, -1, 16, 16)
    rec = oracle.head_bounds_ref(q, k, g)
    sq2 = math.sqrt(2)
    sh = oracle.row_shift_ref(q, rec)
    assert sh[0, 0, 3] == pytest.approx(190 / sq2)
    assert np.allclose(np.delete(sh[0, 0], 3), 50 / sq2)
    shr = oracle.row_shift_ref(q, rec, per_row=True)
    assert shr[0, 0, 3] == pytest.approx(190 / sq2)
    assert np.allclose(np.delete(shr[0, 0], 3), 0.0)
    assert _raw_live_row_max(q, k, g, 1 / sq2)[0, 0, 3] == pytest.approx(190 / sq2)


def _threshold_head(scale):
    """One frame of 16 keys in d = 2: 8 x (5, 0) and 8 x (-5, 0), so mu = 0,
    K_max = 5 and C_max = 0; query row 0 is (6, 0) (Q_max = 6), the rest 0.
    gap_est = scale * 6 * 5 exactly (scale 255/256, 1, 257/256 give 29.8828125,
    30 and 30.1171875, all exact in fp32 and fp64)."""
    k = np.zeros((1, 1, 16, 2)); k[0, 0, :8, 0] = 5.0; k[0, 0, 8:, 0] = -5.0
    q = np.zeros((1, 1, 16, 2)); q[0, 0, 0, 0] = 6.0
    return q, k, oracle.MaskGeometry(1, 16, 0, 0, -1, 16, 16)


THRESHOLD_CASES = [(255 / 256, 29.8828125, True), (1.0, 30.0, True), (257 / 256, 30.1171875, False)]


def test_eligibility_threshold_is_30_nats_inclusive():
    for scale, gap, elig in THRESHOLD_CASES:
        q, k, g = _threshold_head(scale)
        rec = oracle.head_bounds_ref(q, k, g, scale=scale)
        assert rec["c_max"][0, 0] == 0.0 and rec["k_max"][0, 0] == 5.0 and rec["q_max"][0, 0] == 6.0
        assert rec["gap_est"][0, 0] == gap
        assert bool(rec["eligible"][0, 0]) is elig, (scale, gap)
    assert oracle.GAP_THRESHOLD_NATS == 30.0


def test_rope_tables_1d_hand_angle():
    # d = 8, base 10^4: pair i of position n turns by n * 10^(-4 * 2i / 8) = n * 10^-i;
    # position 3, pair 1: 0.3 rad; position 5, pair 2: 0.05 rad; position 0: 0
    c, s = oracle.rope_tables_1d(6, 8)
    assert c.shape == (6, 4)
    assert c[3, 1] == pytest.approx(math.cos(0.3), abs=1e-15)
    assert s[3, 1] == pytest.approx(math.sin(0.3), abs=1e-15)
    assert s[5, 2] == pytest.approx(math.sin(0.05), abs=1e-15)
    np.testing.assert_array_equal(c[0], 1.0)
    np.testing.assert_array_equal(s[0], 0.0)


def test_live_flops_closed_form():
    assert oracle.live_flops(_geom(workloads.workload(2).mask_tuple()), 1, 8, 128) == 4 * 128 * 8 * 117 * 960 * 960
    assert oracle.live_flops(_geom(workloads.workload(5).mask_tuple()), 1, 4, 128) == 2727346176000
    # global reference frame 0 of 21 frames with window +-2: frame 0 sees 21
    # frames instead of 3, so 117 - 3 + 21 = 135 frame pairs
    g = _geom(workloads.workload(2).mask_tuple()[:7] + (1,))
    assert oracle.live_flops(g, 1, 8, 128) == 4 * 128 * 8 * 135 * 960 * 960
    # reference frames 0-1 of 21 with window +-2: frames 0..3 see 3, 4, 5, 6
    # frames, 4..18 see 5 + 2, and 19, 20 (window clamped) 4 + 2 and 3 + 2:
    # 18 + 15 * 7 + 11 = 134 frame pairs
    g = _geom(workloads.workload(2).mask_tuple()[:7] + (0, 2))
    assert [len(oracle.live_frames(g, f)) for f in (0, 1, 2, 3, 4, 18, 19, 20)] == [3, 4, 5, 6, 7, 7, 6, 5]
    assert oracle.live_flops(g, 1, 8, 128) == 4 * 128 * 8 * 134 * 960 * 960


# ------------------------------------------------------------------ planted mistakes

def _run_pins_quietly(fns):
    failed = 0
    for fn in fns:
        try:
            fn()
        except AssertionError:
            failed += 1
    return failed


@pytest.mark.parametrize("attn", ATTN_IMPLS, ids=ATTN_IDS)
def test_planted_mistake_dropped_reference_frame_is_caught(monkeypatch, attn):
    def no_ref_rows(g, rows):
        fr = np.arange(g.N) // g.T
        fi = (np.asarray(rows) // g.T)[:, None]
        return (fr[None, :] >= fi - g.wb) & (fr[None, :] <= fi + g.wa)
    monkeypatch.setattr(O, "mask_rows", no_ref_rows)
    assert _run_pins_quietly([test_plan_matches_hand_derived_golden,
                              lambda: test_attention_matches_bruteforce_loops(attn, (3, 4, 1, 1, 0))]) == 2


@pytest.mark.parametrize("attn", ATTN_IMPLS, ids=ATTN_IDS)
def test_planted_mistake_ignored_global_reference_queries_is_caught(monkeypatch, attn):
    def keys_only_rows(g, rows):
        fr = np.arange(g.N) // g.T
        fi = (np.asarray(rows) // g.T)[:, None]
        m = (fr[None, :] >= fi - g.wb) & (fr[None, :] <= fi + g.wa)
        if g.r >= 0:
            m |= fr[None, :] == g.r
        return m
    monkeypatch.setattr(O, "mask_rows", keys_only_rows)
    assert _run_pins_quietly([test_plan_matches_hand_derived_golden,
                              lambda: test_attention_matches_bruteforce_loops(attn, (4, 3, 0, 0, 2, 1))]) == 2


@pytest.mark.parametrize("attn", ATTN_IMPLS, ids=ATTN_IDS)
def test_planted_mistake_single_reference_frame_is_caught(monkeypatch, attn):
    def first_ref_only_rows(g, rows):
        fr = np.arange(g.N) // g.T
        fi = (np.asarray(rows) // g.T)[:, None]
        m = (fr[None, :] >= fi - g.wb) & (fr[None, :] <= fi + g.wa)
        if g.r >= 0:
            m |= fr[None, :] == g.r
            if g.rg:
                m = m | (fi == g.r)
        return m
    monkeypatch.setattr(O, "mask_rows", first_ref_only_rows)
    assert _run_pins_quietly([test_plan_matches_hand_derived_golden,
                              lambda: test_attention_matches_bruteforce_loops(attn, (6, 2, 0, 0, 1, 0, 3))]) == 2


@pytest.mark.parametrize("attn", ATTN_IMPLS, ids=ATTN_IDS)
def test_planted_mistake_exclusive_window_is_caught(monkeypatch, attn):
    def excl_rows(g, rows):
        fr = np.arange(g.N) // g.T
        fi = (np.asarray(rows) // g.T)[:, None]
        m = (fr[None, :] > fi - g.wb) & (fr[None, :] < fi + g.wa)
        if g.r >= 0:
            m |= fr[None, :] == g.r
        return m
    monkeypatch.setattr(O, "mask_rows", excl_rows)
    assert _run_pins_quietly([test_plan_matches_hand_derived_golden,
                              lambda: test_attention_matches_bruteforce_loops(attn, (3, 4, 1, 1, 0))]) == 2


def test_planted_mistake_uncentred_bound_is_caught(monkeypatch):
    real = O.head_bounds_ref

    def uncentred(q, k, g, scale=None, threshold=30.0):
        rec = real(q, k, g, scale, threshold)
        d = np.asarray(q).shape[-1]
        s = 1 / math.sqrt(d) if scale is None else scale
        rec["k_max"] = np.sqrt((np.asarray(k, np.float64) ** 2).sum(-1)).max(-1)
        rec["bound"] = s * rec["q_max"] * rec["k_max"]
        return rec
    monkeypatch.setattr(oracle, "head_bounds_ref", uncentred)
    assert _run_pins_quietly([test_bounds_hand_example, test_bounds_translation_invariance]) == 2


@pytest.mark.parametrize("real", ATTN_IMPLS, ids=ATTN_IDS)
def test_planted_mistake_transposed_operand_is_caught(real):
    def swapped(q, k, v, g, scale=None, rows=None):
        return real(q, v, k, g, scale, rows)            # K and V exchanged
    assert _run_pins_quietly([lambda: test_attention_matches_bruteforce_loops(swapped, (3, 4, 1, 1, 0)),
                              lambda: test_attention_dense_matches_torch_sdpa(swapped)]) == 2


@pytest.mark.parametrize("real", ATTN_IMPLS, ids=ATTN_IDS)
def test_planted_mistake_missing_scale_is_caught(real):
    def unscaled(q, k, v, g, scale=None, rows=None):
        return real(q, k, v, g, 1.0, rows)
    assert _run_pins_quietly([lambda: test_attention_matches_bruteforce_loops(unscaled, (3, 4, 1, 1, 0)),
                              lambda: test_attention_dense_matches_torch_sdpa(unscaled)]) == 2


# ------------------------------------------------------------------ producer (norm + rotary + layout)

def test_rope_hand_examples():
    # d = 4, x = (1, 2, 3, 4): pair 0 is (1, 2), pair 1 is (3, 4)
    x = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 1, 4)
    def rot(a0, a1):
        c = np.array([[math.cos(a0), math.cos(a1)]])
        s = np.array([[math.sin(a0), math.sin(a1)]])
        return oracle.rope_ref(x, c, s).ravel()
    np.testing.assert_allclose(rot(math.pi / 2, 0.0), [-2, 1, 3, 4], atol=1e-15)
    np.testing.assert_allclose(rot(0.0, math.pi / 2), [1, 2, -4, 3], atol=1e-15)
    np.testing.assert_allclose(rot(math.pi, math.pi), [-1, -2, -3, -4], atol=1e-15)
    np.testing.assert_allclose(rot(0.0, 0.0), [1, 2, 3, 4], atol=0)


def test_rope_matches_complex_multiplication():
    rng = np.random.default_rng(30)
    x = rng.standard_normal((2, 3, 7, 16))
    ang = rng.uniform(-4, 4, (7, 8))
    y = oracle.rope_ref(x, np.cos(ang), np.sin(ang))
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)[None, None]
    np.testing.assert_allclose(y[..., 0::2], z.real, atol=1e-13)
    np.testing.assert_allclose(y[..., 1::2], z.imag, atol=1e-13)


def test_rope_preserves_norms_and_depends_on_relative_position():
    rng = np.random.default_rng(31)
    d, n = 8, 9
    c, s = oracle.rope_tables_1d(n, d)
    q = np.broadcast_to(rng.standard_normal(d), (1, 1, n, d)).copy()   # the same vector at every position
    k = np.broadcast_to(rng.standard_normal(d), (1, 1, n, d)).copy()
    rq, rk = oracle.rope_ref(q, c, s)[0, 0], oracle.rope_ref(k, c, s)[0, 0]
    np.testing.assert_allclose(np.linalg.norm(rq, axis=1), np.linalg.norm(q[0, 0], axis=1), rtol=1e-14)
    dots = rq @ rk.T                     # dots[m, j] depends on m - j only
    for m in range(n):
        for j in range(n):
            if m >= 1 and j >= 1:
                assert dots[m, j] == pytest.approx(dots[m - 1, j - 1], abs=1e-12)


def test_rms_norm_matches_torch_and_closed_forms():
    import torch
    rng = np.random.default_rng(32)
    x = rng.standard_normal((2, 3, 5, 16)) * 3
    g = rng.uniform(0.5, 1.5, (3, 16))
    y = oracle.rms_norm_ref(x, g, 1e-6)
    for h in range(3):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x[:, h]), (16,), torch.from_numpy(g[h]), eps=1e-6)
        np.testing.assert_allclose(y[:, h], ref.numpy(), rtol=1e-13, atol=1e-13)
    # gamma = 1, eps = 0: every row has mean square 1
    y1 = oracle.rms_norm_ref(x, np.ones((3, 16)), 0.0)
    np.testing.assert_allclose(np.mean(y1 * y1, axis=-1), 1.0, rtol=1e-13)
    # a constant row c: y = gamma * c / sqrt(c^2 + eps)
    xc = np.full((1, 1, 1, 4), -2.0)
    yc = oracle.rms_norm_ref(xc, np.array([[1.0, 2.0, 3.0, 4.0]]), 0.25)
    np.testing.assert_allclose(yc.ravel(), np.array([1, 2, 3, 4]) * -2.0 / math.sqrt(4.25), rtol=1e-15)


def test_produce_chain_order_and_pass_through():
    rng = np.random.default_rng(33)
    q, k, v = _rand_qkv(rng, 1, 2, 6, 8)
    g = rng.uniform(0.5, 1.5, (2, 8))
    c, s = oracle.rope_tables_1d(6, 8)
    pq, pk, pv = oracle.produce_ref(q, k, v, g, g, 1e-6, c, s)
    np.testing.assert_array_equal(pv, v)
    # norm, then rotation: the rotation keeps each row's norm, which the
    # normalisation fixed at ||gamma * x / rms(x)||
    np.testing.assert_allclose(np.linalg.norm(pq, axis=-1), np.linalg.norm(oracle.rms_norm_ref(q, g, 1e-6), axis=-1),
                               rtol=1e-13)
    # rotating first and normalising second differs unless gamma is uniform
    other = oracle.rms_norm_ref(oracle.rope_ref(q, c, s), g, 1e-6)
    assert np.abs(other - pq).max() > 1e-3
    # no gamma and no tables: the identity
    for a, b in zip(oracle.produce_ref(q, k, v), (q, k, v)):
        np.testing.assert_array_equal(a, b)


def test_planted_mistake_rotate_half_pairing_is_caught(monkeypatch):
    def rotate_half(x, cos, sin):
        x = np.asarray(x, dtype=np.float64)
        h = x.shape[-1] // 2
        c, s = np.asarray(cos)[None, None], np.asarray(sin)[None, None]
        y = np.empty_like(x)
        y[..., :h] = x[..., :h] * c - x[..., h:] * s
        y[..., h:] = x[..., :h] * s + x[..., h:] * c
        return y
    monkeypatch.setattr(oracle, "rope_ref", rotate_half)
    assert _run_pins_quietly([test_rope_hand_examples, test_rope_matches_complex_multiplication]) == 2


def test_planted_mistake_rotation_sign_is_caught(monkeypatch):
    real = O.rope_ref
    def wrong_sign(x, cos, sin):
        y = real(x, cos, sin)
        x = np.asarray(x, dtype=np.float64)
        y[..., 1::2] = -x[..., 0::2] * np.asarray(sin)[None, None] + x[..., 1::2] * np.asarray(cos)[None, None]
        return y
    monkeypatch.setattr(oracle, "rope_ref", wrong_sign)
    assert _run_pins_quietly([test_rope_hand_examples, test_rope_matches_complex_multiplication,
                              test_rope_preserves_norms_and_depends_on_relative_position]) == 3


def test_planted_mistake_norm_without_eps_or_gamma_is_caught(monkeypatch):
    def no_eps(x, gamma, eps):
        x = np.asarray(x, dtype=np.float64)
        return np.asarray(gamma)[None, :, None, :] * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))
    def no_gamma(x, gamma, eps):
        x = np.asarray(x, dtype=np.float64)
        return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    for bad in (no_eps, no_gamma):
        monkeypatch.setattr(oracle, "rms_norm_ref", bad)
        assert _run_pins_quietly([test_rms_norm_matches_torch_and_closed_forms]) == 1


def test_planted_mistake_shift_without_mean_term_is_caught(monkeypatch):
    real = oracle.row_shift_ref

    def no_qmu(q, rec, scale=None, per_row=False, k_max=None):
        zero = dict(rec, mu=np.zeros_like(rec["mu"]))
        return real(q, zero, scale=scale, per_row=per_row, k_max=k_max)
    monkeypatch.setattr(oracle, "row_shift_ref", no_qmu)
    assert _run_pins_quietly([test_row_shift_bounds_every_raw_live_logit, test_row_shift_hand_values]) == 2


def test_planted_mistake_shift_without_scale_on_mean_term_is_caught(monkeypatch):
    def unscaled_qmu(q, rec, scale=None, per_row=False, k_max=None):
        q = np.asarray(q, np.float64)
        scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
        qmu = np.einsum("bhnd,bhd->bhn", q, rec["mu"])
        if per_row:
            return scale * np.sqrt((q * q).sum(-1)) * rec["k_max"][:, :, None] + qmu
        return rec["bound"][:, :, None] + qmu
    monkeypatch.setattr(oracle, "row_shift_ref", unscaled_qmu)
    assert _run_pins_quietly([test_row_shift_bounds_every_raw_live_logit, test_row_shift_hand_values]) == 2


def test_planted_mistake_shift_without_scale_is_caught(monkeypatch):
    real = oracle.row_shift_ref

    def unscaled(q, rec, scale=None, per_row=False, k_max=None):
        q = np.asarray(q, np.float64)
        s = 1.0 / math.sqrt(q.shape[-1]) if scale is None else scale
        return real(q, rec, scale=s, per_row=per_row, k_max=k_max) / s
    monkeypatch.setattr(oracle, "row_shift_ref", unscaled)
    assert _run_pins_quietly([test_row_shift_hand_values]) == 1


@pytest.mark.parametrize("mistake", ["exclusive", "threshold25", "threshold100"])
def test_planted_mistake_threshold_is_caught(monkeypatch, mistake):
    real = oracle.head_bounds_ref

    def bad(q, k, g, scale=None, threshold=oracle.GAP_THRESHOLD_NATS):
        if mistake == "threshold25":
            return real(q, k, g, scale=scale, threshold=25.0)
        if mistake == "threshold100":
            return real(q, k, g, scale=scale, threshold=100.0)
        rec = real(q, k, g, scale=scale, threshold=threshold)
        return dict(rec, eligible=rec["gap_est"] < threshold)
    monkeypatch.setattr(oracle, "head_bounds_ref", bad)
    assert _run_pins_quietly([test_eligibility_threshold_is_30_nats_inclusive]) == 1


def test_planted_mistake_rope_base_is_caught(monkeypatch):
    real = oracle.rope_tables_1d
    monkeypatch.setattr(oracle, "rope_tables_1d", lambda n, d, base=10000.0: real(n, d, base=1000.0))
    assert _run_pins_quietly([test_rope_tables_1d_hand_angle]) == 1
