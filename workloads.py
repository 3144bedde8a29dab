"""Seeded synthetic inputs for frame-structured block-sparse attention.

This module is shared by the CPU oracle, the tests and the benchmark. It only
draws random numbers and shapes them into the five video-shaped workloads; it
holds none of the attention method's arithmetic (no mask, no plan, no bound,
no softmax). Nothing here imports the GPU package or the oracle.

Workloads stand in for the production super-resolution attention described in
"HeyGen x Google Cloud: Bringing Avatar IV to TPUs" (section "Deleting the
Mask"): each frame's queries see a window of neighbouring frames plus one
reference frame, at tens of thousands of tokens. The production activations
are not available, so the inputs are Gaussian with the per-workload modifiers
below (the recipe is restated, with its readings, in the design notes).

Recipe (deterministic):
  1. rng = numpy.random.default_rng(seed)            (seed 0 by default)
  2. Q, then K, then V: rng.standard_normal((B, H, N, d), float32)
  3. the workload's modifiers, in the listed order, drawing from the same rng
  4. bf16 workloads: round to bfloat16 (round-to-nearest-even) once; the
     rounded values are the ground truth for both the oracle and the GPU.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    num_frames: int
    tokens_per_frame: int
    head_dim: int
    dtype: str               # "f32" or "bf16"
    window_before: int
    window_after: int
    ref_frame: int           # -1: no reference frame
    block_q: int
    block_k: int
    modifier: str = "none"   # none | scale_qk | key_offset | stress_keys | rmsnorm_qk
    description: str = ""
    ref_queries_global: int = 0   # 1: the reference frames' queries see every frame
    ref_count: int = 0            # reference frames from ref_frame (0 or 1: one)

    @property
    def seq_len(self) -> int:
        return self.num_frames * self.tokens_per_frame

    def mask_tuple(self):
        """(num_frames, tokens_per_frame, window_before, window_after,
        ref_frame, block_q, block_k, ref_queries_global, ref_count) - the
        nine integers of the mask descriptor, in the C struct's field order."""
        return (self.num_frames, self.tokens_per_frame, self.window_before,
                self.window_after, self.ref_frame, self.block_q, self.block_k,
                self.ref_queries_global, self.ref_count)


# The five workloads. Sizes are one GPU's share of heads at the full
# sequence length.
WORKLOADS = [
    Workload("tiny_f32_5x48", 1, 2, 5, 48, 64, "f32", 1, 1, 0, 16, 16,
             "none", "5 frames x 48 tokens, window +-1 + reference frame 0, blocks 16, fp32"),
    Workload("bf16_21x960", 1, 8, 21, 960, 128, "bf16", 2, 2, 0, 64, 64,
             "scale_qk", "21 frames x 960 tokens, window +-2 + ref 0, blocks 64, Q,K ~ N(0,1)/sqrt(2)"),
    Workload("bf16_9x3600", 1, 5, 9, 3600, 128, "bf16", 1, 1, 0, 48, 240,
             "key_offset", "9 frames x 3600 tokens (45x80 latent), window +-1 + ref 0, "
             "q block 48, k block 240, keys offset by a per-head N(0,4) mean"),
    Workload("bf16_16x1024_dense_stress", 1, 16, 16, 1024, 128, "bf16", 15, 15, 0, 64, 64,
             "stress_keys", "16 frames x 1024 tokens, dense, blocks 64, 0.1% of keys x40 in heads 5 and 10"),
    Workload("bf16_6x8160", 1, 4, 6, 8160, 128, "bf16", 1, 1, 0, 80, 80,
             "rmsnorm_qk", "6 frames x 8160 tokens (68x120 latent), window +-1 + ref 0, blocks 80, "
             "Q,K RMS-normalised with gamma ~ U(0.5, 1.5)"),
]

STRESSED_HEADS = (5, 10)
STRESS_KEYS = 16          # 0.1% of 16,384 keys, rounded
STRESS_FACTOR = 40.0
RMS_EPS = 1e-6


def workload(i: int) -> Workload:
    """Workload by its 1-based number (1..5)."""
    return WORKLOADS[i - 1]


def make_workload(name, batch, heads, num_frames, tokens_per_frame, head_dim,
                  dtype="bf16", window_before=1, window_after=1, ref_frame=0,
                  block_q=16, block_k=16, modifier="none",
                  ref_queries_global=0, ref_count=0) -> Workload:
    """A custom (test-sized) workload with the same recipe."""
    return Workload(name, batch, heads, num_frames, tokens_per_frame, head_dim,
                    dtype, window_before, window_after, ref_frame, block_q,
                    block_k, modifier, ref_queries_global=ref_queries_global,
                    ref_count=ref_count)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32 holding exactly representable values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def make_inputs(w: Workload, seed: int = 0, rows: Optional[int] = None):
    """Return (q, k, v) as float32 numpy arrays of shape (B, H, N, d).

    For bf16 workloads every value is exactly representable in bfloat16.
    ``rows`` is not supported on purpose: inputs are always drawn whole so
    that every consumer sees the same numbers.
    """
    assert rows is None
    rng = np.random.default_rng(seed)
    shape = (w.batch, w.heads, w.seq_len, w.head_dim)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if w.modifier == "none":
        pass
    elif w.modifier == "scale_qk":
        s = np.float32(1.0 / np.sqrt(2.0))
        q *= s
        k *= s
    elif w.modifier == "key_offset":
        mu = np.float32(2.0) * rng.standard_normal((w.batch, w.heads, 1, w.head_dim), dtype=np.float32)
        k += mu
    elif w.modifier == "stress_keys":
        for h in STRESSED_HEADS:
            if h >= w.heads:
                continue
            n_stress = min(STRESS_KEYS, w.seq_len)
            idx = np.sort(rng.choice(w.seq_len, n_stress, replace=False))
            for b in range(w.batch):
                k[b, h, idx, :] *= np.float32(STRESS_FACTOR)
    elif w.modifier == "rmsnorm_qk":
        gq = rng.uniform(0.5, 1.5, (w.heads, w.head_dim)).astype(np.float32)
        gk = rng.uniform(0.5, 1.5, (w.heads, w.head_dim)).astype(np.float32)
        for x, g in ((q, gq), (k, gk)):
            r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + np.float32(RMS_EPS))
            x[...] = g[None, :, None, :] * (x / r)
    else:
        raise ValueError(f"unknown modifier {w.modifier!r}")
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif w.dtype != "f32":
        raise ValueError(w.dtype)
    return q, k, v


def make_producer_inputs(w: Workload, seed: int = 0):
    """Inputs of the input-producing chain (normalisation + rotary embedding)
    at the workload's shape: raw projections q, k, v ~ N(0, 1) as float32
    (B, H, N, d), bf16-representable for bf16 workloads; per-head gammas
    (H, d) ~ U(0.5, 1.5); and rotation tables (N, d/2) as float32 cosines and
    sines of angles ~ U(0, 2 pi). Drawn in that order from one seeded
    generator."""
    rng = np.random.default_rng(seed)
    shape = (w.batch, w.heads, w.seq_len, w.head_dim)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    gq = rng.uniform(0.5, 1.5, (w.heads, w.head_dim)).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, (w.heads, w.head_dim)).astype(np.float32)
    ang = rng.uniform(0.0, 2.0 * np.pi, (w.seq_len, w.head_dim // 2))
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return dict(q=q, k=k, v=v, gamma_q=gq, gamma_k=gk,
                cos=np.cos(ang).astype(np.float32), sin=np.sin(ang).astype(np.float32))


def device_normal(shape, seed: int, device, dtype):
    """Standard-normal values drawn on `device` by torch's seeded generator,
    one [.., N, d] slab per (batch, head) in order, each rounded to `dtype`:
    inputs too large to draw on the host (addressing tests past 2^31
    elements). Both the GPU path and the oracle read the same tensor, the
    oracle through host copies of slices of it."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    B, H = shape[0], shape[1]
    x = torch.empty(shape, dtype=dtype, device=device)
    for b in range(B):
        for h in range(H):
            x[b, h] = torch.randn(shape[2:], generator=g, device=device, dtype=torch.float32).to(dtype)
    return x
