"""Comparison rules between the HIP path and the CPU oracle.

Indices: the GPU's ordered top-k list of every (token, head) must equal the
oracle's, except where the oracle's own fp64 values put a decision within a
relative gap of TIE_REL (1e-6) of its alternative.  There the GPU's list
must still be valid: k distinct slots whose oracle products P = (eps+d1)(eps+d2)
are non-decreasing up to TIE_REL and none worse than the oracle's k-th P by
more than TIE_REL.  Such tokens are counted and reported.

Floats: |gpu - ora| <= rtol * (|ora| + rms(ora)) elementwise, with rtol 1e-4
for fp32 storage and 2e-2 for bf16 storage, on tokens whose selected set
matched the oracle's.
"""
from __future__ import annotations

import numpy as np

import oracle

TIE_REL = 1e-6


def rtol_for(cfg):
    return 1e-4 if cfg.store == "f32" else 2e-2


def close(gpu, ora, rtol, mask=None, what=""):
    gpu = np.asarray(gpu, np.float64)
    ora = np.asarray(ora, np.float64)
    if mask is not None:
        gpu = gpu[mask]
        ora = ora[mask]
    if ora.size == 0:
        return 0.0
    scale = np.abs(ora) + np.sqrt(np.mean(ora ** 2))
    err = np.abs(gpu - ora)
    bad = err > rtol * scale
    worst = float((err / np.maximum(scale, 1e-300)).max())
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} elements beyond rtol {rtol}; worst rel {worst:.3g}"
    return worst


def compare_indices(cfg, q, K1, K2, gpu_idx, ora):
    """Returns (exact_mask[B,T,H], near_tie_count).  Asserts validity."""
    gi = np.asarray(gpu_idx)
    oi = ora["idx"]
    exact = (gi == oi).all(-1)
    near = 0
    if not exact.all():
        Pg = oracle.pair_p(cfg, q, K1, K2, gi)
        Po = ora["P"]
        for pos in zip(*np.nonzero(~exact)):
            pg = Pg[pos]
            slots = gi[pos]
            assert len(set(slots.tolist())) == cfg.k, f"duplicate slots at {pos}: {slots}"
            assert np.all(pg[1:] >= pg[:-1] * (1 - TIE_REL)), f"order beyond near-tie at {pos}"
            assert pg.max() <= Po[pos][-1] * (1 + TIE_REL), f"selection beyond near-tie at {pos}"
            near += 1
    return exact, near


def token_set_match(gpu_idx, ora_idx):
    """[B,T] bool: every head of the token selected the same set of slots."""
    g = np.sort(np.asarray(gpu_idx), -1)
    o = np.sort(np.asarray(ora_idx), -1)
    return (g == o).all(-1).all(-1)
