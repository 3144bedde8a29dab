"""CPU oracle for frame-structured block-sparse attention (fp64, numpy).

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the
HIP library and its Python binding) never calls it, and this module imports
nothing from the product package: the two share no code.

Source: "HeyGen x Google Cloud: Bringing Avatar IV to TPUs" (Google
Developers Blog; a paraphrased copy carries the section headings used below).
  * "Deleting the Mask", Fig. 3: every frame's queries see the keys of a
    window of nearby frames plus one global reference frame; the live regions
    snap to frame boundaries; block sizes that are multiples of 16 and divide
    the frame's token span make every block fully live or fully masked, and
    the reference frame's blocks are just more blocks in one softmax pass.
  * "Unchaining the Softmax", Fig. 4: the running max of the online softmax
    is replaced by a precomputed upper bound on the logits (Cauchy-Schwarz:
    a query's largest logit is at most its norm times the largest key norm);
    keys are mean-centred first, which tightens the bound and leaves the
    softmax unchanged; eligibility is decided per head and heads whose bound
    is too loose use the online softmax; the bound's guarantee is extended to
    windowed masks where each query row sees a different slice of keys.

  * "Layout Is the ABI", Fig. 5: the small operations that produce
    attention's inputs (normalisation, rotary embeddings, projections,
    head packing) are fused into one kernel that writes the layout its
    consumer reads.

Because blocks are exactly full or empty and a softmax is invariant under a
per-row shift, the method's output is, up to rounding, plain softmax
attention under the token-level mask. So the attention oracle is that plain
definition written out in fp64 (dense scores, masked entries set to -inf,
max-subtracted softmax), not the blocked algorithm.

Readings where the pages are silent (each also listed in the design notes):
  R1  softmax scale defaults to 1/sqrt(d)
  R2  the window is inclusive, clamped to [0, F-1], possibly asymmetric
  R3  every query sees the reference frame's keys; reference-frame queries
      see only their own window (the reference frame is not a global query).
      The symmetric reading, where the reference frame's queries see every
      frame as a global token's would, is kept as an option
      (ref_queries_global=1).
  R3b several reference frames: a contiguous span of ref_count frames
      starting at the reference frame (ref_count 0 or 1: the one frame);
      every query sees all of their keys, and under the R3 option the
      queries of every frame of the span are global
  R4  tokens are frame-major: token t belongs to frame t // T
  R5  a plan lists live key blocks in ascending order
  R6  block sizes must be positive multiples of 16 that divide T; anything
      else is an error (no padded fallback)
  R7  one key mean per (batch, head), over all N keys
  R8  default shift for row i: bound_h + scale * q_i . mu_h; variant:
      scale * (|q_i| * K_max + q_i . mu_h)
  R10 eligibility: gap_est = scale * Q_max * (K_max + C_max) <= 30 nats,
      where C_max = max_f |mean of the keys live for frame f - mu_h|; this
      upper-bounds "bound minus logit max" for every row, so it can be
      checked before any logit is computed.
  R14 the fused chain: per-head RMSNorm over d with a gamma per (head,
      dimension), then the rotary embedding, on Q and K; V is only moved.
      The projection is a plain GEMM left to the caller; its output is the
      chain's input, read through strides
  R15 rotary embedding: RoFormer's rotation of dimension pairs (2i, 2i+1),
      with per-token angle tables supplied by the caller (1-D or
      multi-axis positions alike)

Parity status: every function below is pinned by tests that do not reuse
its own arithmetic (brute force over tokens, closed forms, invariants,
a library attention routine, hand-worked values); none is "parity
unpinned". In particular the row shift is pinned by brute force (it is at
least every raw live logit of its row, and at most gap_est above the row's
largest one) and by a hand value, and the eligibility threshold by hand
heads whose gap estimate is just below, exactly at and just above 30 nats.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

GAP_THRESHOLD_NATS = 30.0
LOG2E = 1.4426950408889634


# ---------------------------------------------------------------- geometry

class MaskGeometry:
    """The integers that define the frame-structured mask and its block
    tiling ("Deleting the Mask": window of nearby frames + one reference
    frame; blocks are multiples of 16 dividing the frame span), plus the
    R3 option that makes the reference frame's queries global and the R3b
    span of several reference frames."""

    def __init__(self, num_frames, tokens_per_frame, window_before, window_after,
                 ref_frame, block_q, block_k, ref_queries_global=0, ref_count=0):
        self.F = int(num_frames)
        self.T = int(tokens_per_frame)
        self.wb = int(window_before)
        self.wa = int(window_after)
        self.r = int(ref_frame)
        self.bq = int(block_q)
        self.bk = int(block_k)
        # R3 option: the reference frame's own queries also see every key
        self.rg_arg = int(ref_queries_global)
        self.rg = self.rg_arg if self.r >= 0 else 0
        # R3b: reference frames r .. r + nr - 1 (nr = 0 without a reference frame)
        self.nr_arg = int(ref_count)
        self.nr = max(1, self.nr_arg) if self.r >= 0 else 0

    @classmethod
    def from_tuple(cls, t):
        return cls(*t)

    @property
    def N(self):
        return self.F * self.T

    def validate(self):
        """R6: blocks are positive multiples of 16 dividing T; windows are
        non-negative; the reference frame is -1 (none) or a valid frame."""
        ok = (self.F >= 1 and self.T >= 16 and self.wb >= 0 and self.wa >= 0
              and -1 <= self.r < self.F and self.rg_arg in (0, 1)
              and self.nr_arg >= 0 and self.r + self.nr <= self.F)
        for b in (self.bq, self.bk):
            ok = ok and b > 0 and b % 16 == 0 and self.T % b == 0
        if not ok:
            raise ValueError(f"invalid frame/block geometry {vars(self)}")


def live_frames(g: MaskGeometry, f: int) -> List[int]:
    """Frames whose keys the queries of frame f see (R2, R3, R3b): the
    clamped window [f - wb, f + wa] united with the reference frames, ascending; all
    frames for a reference frame itself under the R3 option."""
    refs = range(g.r, g.r + g.nr)
    if g.rg and f in refs:
        return list(range(g.F))
    s = set(range(max(0, f - g.wb), min(g.F - 1, f + g.wa) + 1))
    s.update(refs)
    return sorted(s)


def token_mask(g: MaskGeometry) -> np.ndarray:
    """Dense boolean mask M[i, j]: query token i may attend to key token j.
    Built from frame indices by integer arithmetic (R2-R4)."""
    fr = np.arange(g.N) // g.T
    fi = fr[:, None]
    fj = fr[None, :]
    m = (fj >= fi - g.wb) & (fj <= fi + g.wa)
    m |= (fj >= g.r) & (fj < g.r + g.nr)
    if g.rg:
        m |= (fi >= g.r) & (fi < g.r + g.nr)
    return m


def mask_rows(g: MaskGeometry, rows) -> np.ndarray:
    """Rows `rows` of token_mask, shape (len(rows), N), without building the
    dense N x N matrix (same integer rule as token_mask)."""
    fr = np.arange(g.N) // g.T
    fi = (np.asarray(rows, dtype=np.int64) // g.T)[:, None]
    m = (fr[None, :] >= fi - g.wb) & (fr[None, :] <= fi + g.wa)
    m |= (fr[None, :] >= g.r) & (fr[None, :] < g.r + g.nr)
    if g.rg:
        m = m | ((fi >= g.r) & (fi < g.r + g.nr))
    return m


def row_mask(g: MaskGeometry, i: int) -> np.ndarray:
    """Row i of token_mask."""
    return mask_rows(g, [i])[0]


# ---------------------------------------------------------------- plan

def plan_bruteforce(g: MaskGeometry) -> Tuple[np.ndarray, np.ndarray]:
    """Live key blocks per query block by enumerating the token-level mask
    over every (query block, key block) pair ("Deleting the Mask": with
    aligned blocks every block is entirely inside or entirely outside the
    mask). Raises if any block is partially live. Returns CSR int32
    (row_ptr[nqb + 1], col_idx[nnz]), key blocks ascending (R5).

    Works frame by frame on the mask rows so that it stays cheap at the
    full sizes (a block row's mask only depends on its tokens)."""
    g.validate()
    nqb, nkb = g.N // g.bq, g.N // g.bk
    row_ptr = np.zeros(nqb + 1, dtype=np.int64)
    cols: List[np.ndarray] = []
    for qb in range(nqb):
        rows = mask_rows(g, np.arange(qb * g.bq, (qb + 1) * g.bq))
        blk = rows.reshape(g.bq, nkb, g.bk)
        live = blk.any(axis=(0, 2))
        full = blk.all(axis=(0, 2))
        if np.any(live & ~full):
            raise AssertionError(f"partial block in query block {qb}")
        c = np.nonzero(live)[0]
        cols.append(c)
        row_ptr[qb + 1] = row_ptr[qb] + len(c)
    col_idx = np.concatenate(cols) if cols else np.zeros(0, np.int64)
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def partial_blocks_if_tiled(g: MaskGeometry, tile: int) -> Tuple[int, int]:
    """(partial, live) block counts if the same mask were tiled with square
    blocks of `tile` tokens and the sequence padded to a multiple of the tile
    (the prior-art tiling of "Deleting the Mask"). Padding tokens are masked."""
    npad = -(-g.N // tile) * tile
    nb = npad // tile
    fr = np.arange(npad) // g.T
    valid = np.arange(npad) < g.N
    partial = live = 0
    for qb in range(nb):
        ri = np.arange(qb * tile, (qb + 1) * tile)
        fi = fr[ri][:, None]
        fj = fr[None, :]
        m = (fj >= fi - g.wb) & (fj <= fi + g.wa)
        m |= (fj >= g.r) & (fj < g.r + g.nr)
        if g.rg:
            m = m | ((fi >= g.r) & (fi < g.r + g.nr))
        m &= valid[ri][:, None] & valid[None, :]
        blk = m.reshape(tile, nb, tile)
        lv = blk.any(axis=(0, 2))
        fl = blk.all(axis=(0, 2))
        live += int(lv.sum())
        partial += int((lv & ~fl).sum())
    return partial, live


# ---------------------------------------------------------------- attention

def attention_ref(q, k, v, g: MaskGeometry, scale: Optional[float] = None,
                  rows: Optional[Sequence[int]] = None, chunk: int = 256):
    """Plain masked softmax attention in fp64.

    q, k, v: arrays (B, H, N, d) (any float dtype; converted exactly to
    fp64). Returns (O, lse) with O (B, H, R, d) fp64 and lse (B, H, R) fp64,
    where R = N or len(rows). lse_i = m_i + ln(l_i) in natural-log units.
    Every row has at least one live key (its own frame), so l_i >= 1."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    assert N == g.N
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    out = np.empty((B, H, R, d), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    for s in range(0, R, chunk):
        ri = rows[s:s + chunk]
        m = mask_rows(g, ri)
        for b in range(B):
            for h in range(H):
                sc = scale * (q[b, h, ri] @ k[b, h].T)
                sc = np.where(m, sc, -np.inf)
                mx = sc.max(axis=1, keepdims=True)
                p = np.exp(sc - mx)
                l = p.sum(axis=1, keepdims=True)
                out[b, h, s:s + chunk] = (p @ v[b, h]) / l
                lse[b, h, s:s + chunk] = mx[:, 0] + np.log(l[:, 0])
    return out, lse


def attention_live_ref(q, k, v, g: MaskGeometry, scale: Optional[float] = None,
                       rows: Optional[Sequence[int]] = None, chunk: int = 1024):
    """The same plain masked softmax attention as attention_ref, in fp64,
    with each row's sums taken over its live keys only: the terms of masked
    keys are exactly zero in the definition, so leaving them out changes
    nothing. A row's live keys depend only on its frame (token_mask is a
    function of the two frame indices), so the rows of one frame share one
    key list, which is read off the mask rows themselves (and checked to be
    the same for every row of the chunk). torch's CPU fp64 matmul and exp
    are used for their threads; this makes full-size workloads affordable.

    Same arguments and results as attention_ref: (O (B, H, R, d),
    lse (B, H, R)) as fp64 numpy arrays."""
    import torch
    q = np.asarray(q); k = np.asarray(k); v = np.asarray(v)
    B, H, N, d = q.shape
    assert N == g.N
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    qt = torch.from_numpy(np.ascontiguousarray(q)).to(torch.float64)
    kt = torch.from_numpy(np.ascontiguousarray(k)).to(torch.float64)
    vt = torch.from_numpy(np.ascontiguousarray(v)).to(torch.float64)
    out = np.empty((B, H, R, d), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    frame_of = rows // g.T
    for f in np.unique(frame_of):
        pos = np.nonzero(frame_of == f)[0]              # positions in `rows` of frame f's rows
        for s in range(0, len(pos), chunk):
            pp = pos[s:s + chunk]
            ri = rows[pp]
            m = mask_rows(g, ri)
            assert (m == m[0]).all()
            live = torch.from_numpy(np.nonzero(m[0])[0])
            for b in range(B):
                for h in range(H):
                    kl = kt[b, h].index_select(0, live)
                    vl = vt[b, h].index_select(0, live)
                    sc = scale * (qt[b, h].index_select(0, torch.from_numpy(ri)) @ kl.T)
                    mx = sc.max(dim=1, keepdim=True).values
                    p = torch.exp(sc - mx)
                    l = p.sum(dim=1, keepdim=True)
                    out[b, h, pp] = ((p @ vl) / l).numpy()
                    lse[b, h, pp] = (mx[:, 0] + torch.log(l[:, 0])).numpy()
    return out, lse


def attention_online_ref(q, k, v, g: MaskGeometry, scale=None, key_block=None):
    """fp64 flash-style online softmax ("Unchaining the Softmax", Fig. 4,
    upper chain): for each query row walk its live keys in blocks, carry a
    running max m, rescale the accumulator and the normaliser by
    exp(m_old - m_new) whenever the max rises. Used only to pin shift
    invariance against attention_ref."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    kb = key_block or g.bk
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                live = np.nonzero(row_mask(g, i))[0]
                m = -np.inf
                l = 0.0
                acc = np.zeros(d)
                for s in range(0, len(live), kb):
                    j = live[s:s + kb]
                    sc = scale * (k[b, h, j] @ q[b, h, i])
                    mn = max(m, sc.max())
                    alpha = math.exp(m - mn) if m != -np.inf else 0.0
                    p = np.exp(sc - mn)
                    l = alpha * l + p.sum()
                    acc = alpha * acc + p @ v[b, h, j]
                    m = mn
                out[b, h, i] = acc / l
    return out


def attention_fixed_shift_ref(q, k, v, g: MaskGeometry, shift, scale=None):
    """fp64 softmax with a caller-given per-row shift in place of the row max
    ("Unchaining the Softmax", Fig. 4, lower chain). shift: (B, H, N). The
    result equals attention_ref whenever exp(logit - shift) does not
    underflow, because softmax is invariant under a per-row shift."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    m = token_mask(g)
    out = np.empty_like(q)
    for b in range(B):
        for h in range(H):
            sc = scale * (q[b, h] @ k[b, h].T)
            p = np.where(m, np.exp(sc - np.asarray(shift)[b, h][:, None]), 0.0)
            out[b, h] = (p @ v[b, h]) / p.sum(axis=1, keepdims=True)
    return out


# ---------------------------------------------------------------- bounds

def head_bounds_ref(q, k, g: MaskGeometry, scale: Optional[float] = None,
                    threshold: float = GAP_THRESHOLD_NATS) -> Dict[str, np.ndarray]:
    """Per-(batch, head) bound record in fp64 ("Unchaining the Softmax").

      mu      key mean over all N keys (R7)                     (B, H, d)
      q_max   max_i |q_i|                                        (B, H)
      k_max   max_j |k_j - mu|                                   (B, H)
      bound   scale * q_max * k_max  (Cauchy-Schwarz bound on every
              mean-centred logit scale * q_i . (k_j - mu))       (B, H)
      c_max   max_f |(mean of keys of the frames live for f) - mu| (B, H)
      gap_est scale * q_max * (k_max + c_max)   (R10)            (B, H)
      eligible gap_est <= threshold                              (B, H) bool
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    mu = k.mean(axis=2)                                          # (B, H, d)
    q_max = np.sqrt((q * q).sum(-1)).max(-1)
    kc = k - mu[:, :, None, :]
    k_max = np.sqrt((kc * kc).sum(-1)).max(-1)
    frame_mean = k.reshape(B, H, g.F, g.T, d).mean(axis=3)      # (B, H, F, d)
    c_max = np.zeros((B, H))
    for f in range(g.F):
        L = live_frames(g, f)
        wmean = frame_mean[:, :, L, :].mean(axis=2)             # equal frame sizes
        c_max = np.maximum(c_max, np.sqrt(((wmean - mu) ** 2).sum(-1)))
    bound = scale * q_max * k_max
    gap_est = scale * q_max * (k_max + c_max)
    return dict(mu=mu, q_max=q_max, k_max=k_max, bound=bound, c_max=c_max,
                gap_est=gap_est, eligible=gap_est <= threshold)


def row_shift_ref(q, rec, scale=None, per_row=False, k_max=None):
    """The fixed shift of each query row in natural-log units (R8):
    default  m_i = bound_h + scale * q_i . mu_h
    per_row  m_i = scale * (|q_i| * k_max_h + q_i . mu_h)."""
    q = np.asarray(q, np.float64)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    qmu = scale * np.einsum("bhnd,bhd->bhn", q, rec["mu"])
    if per_row:
        kmax = rec["k_max"] if k_max is None else k_max
        return scale * np.sqrt((q * q).sum(-1)) * kmax[:, :, None] + qmu
    return rec["bound"][:, :, None] + qmu


def live_logit_stats(q, k, g: MaskGeometry, mu, scale=None, rows=None):
    """Diagnostics for the bound audit: for each (b, h) and each selected
    row, the largest mean-centred live logit max_j scale * q_i.(k_j - mu).
    Returns (B, H, R)."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.empty((B, H, len(rows)))
    for t, i in enumerate(rows):
        m = row_mask(g, int(i))
        for b in range(B):
            for h in range(H):
                kc = k[b, h][m] - mu[b, h]
                out[b, h, t] = (scale * (kc @ q[b, h, i])).max()
    return out


def live_flops(g: MaskGeometry, batch: int, heads: int, head_dim: int) -> int:
    """Live-block FLOPs of one forward: QK^T and PV on live (query, key)
    pairs only, 2*d flops each: 4 * d * B * H * sum_f |L(f)| * T^2."""
    pairs = sum(len(live_frames(g, f)) for f in range(g.F)) * g.T * g.T
    return 4 * head_dim * batch * heads * pairs


# ---------------------------------------------------------------- producer

def rms_norm_ref(x, gamma, eps):
    """Per-row RMS normalisation over the last axis (the "normalization" of
    the chain that produces attention's inputs, "Layout Is the ABI"):
    y = gamma * x / sqrt(mean(x^2) + eps). x: (B, H, N, d); gamma: (H, d)
    or None (no normalisation). R14."""
    x = np.asarray(x, dtype=np.float64)
    if gamma is None:
        return x.copy()
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + float(eps))
    return np.asarray(gamma, dtype=np.float64)[None, :, None, :] * (x / r)


def rope_ref(x, cos, sin):
    """Rotary position embedding (the "rotary embeddings" of the same chain),
    RoFormer's form: dimension pair (2i, 2i+1) of token n is rotated by the
    angle whose cosine and sine are cos[n, i] and sin[n, i]:
        y[2i]   = x[2i] cos - x[2i+1] sin
        y[2i+1] = x[2i] sin + x[2i+1] cos.
    The caller's tables carry the positional scheme (R15). x: (B, H, N, d);
    cos, sin: (N, d/2) or None (no rotation)."""
    x = np.asarray(x, dtype=np.float64)
    if cos is None:
        return x.copy()
    c = np.asarray(cos, dtype=np.float64)[None, None]
    s = np.asarray(sin, dtype=np.float64)[None, None]
    y = np.empty_like(x)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def produce_ref(q_in, k_in, v_in, gamma_q=None, gamma_k=None, eps=1e-6, cos=None, sin=None):
    """The chain that produces attention's inputs ("Layout Is the ABI",
    Fig. 5), without its projection (R14): Q and K are RMS-normalised and
    then rotated; V passes through. Inputs and outputs are (B, H, N, d) in
    fp64; the layout the product writes is a matter of strides."""
    q = rope_ref(rms_norm_ref(q_in, gamma_q, eps), cos, sin)
    k = rope_ref(rms_norm_ref(k_in, gamma_k, eps), cos, sin)
    return q, k, np.asarray(v_in, dtype=np.float64).copy()


def rope_tables_1d(n, d, base=10000.0):
    """RoFormer's tables for 1-D positions 0..n-1: angle n * base^(-2i/d)
    for pair i. Returns (cos, sin), each (n, d/2) fp64."""
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.arange(n, dtype=np.float64)[:, None] * base ** (-2.0 * i / d)[None, :]
    return np.cos(ang), np.sin(ang)
