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


def bf16_ulp(x):
    """Spacing of bf16 values (8 significant bits) at |x|: 2^(e-8) for
    |x| = m 2^e, m in [0.5, 1); the smallest subnormal step at 0."""
    x = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(x)
    return np.where(x > 0, np.ldexp(1.0, np.maximum(e - 8, -133)), np.ldexp(1.0, -133))


def ulp_check(gpu, ora, old, what, arith):
    """State written back to bf16, element by element.  The GPU rounds an
    fp32 result to bf16 and the oracle an fp64 one, so the two agree to one
    bf16 step at the larger of the two values, plus the GPU arithmetic's own
    error before that rounding.  That error is bounded by `arith` times the
    row's scale: |old| + the largest |new - old| of the oracle's write in
    the row (a sum's rounding error follows the size of its terms, which the
    row's largest step shows even where one element's terms cancel).  For
    the value rows `arith` covers fp32 sums; for the sub-keys, the step's
    MFMA product with its operand split into two bf16 parts.  Arrays are
    [..., row length].  Returns (elements that differ, worst in steps)."""
    gpu = np.asarray(gpu, np.float64)
    ora = np.asarray(ora, np.float64)
    old = np.asarray(old, np.float64)
    ulp = np.maximum(bf16_ulp(gpu), bf16_ulp(ora))
    err = np.abs(gpu - ora)
    row = np.abs(ora - old).max(-1, keepdims=True)
    tol = ulp + arith * (np.abs(old) + row)
    bad = err > tol
    steps = err / ulp
    n1 = int((err > 0).sum())
    worst = float(steps.max()) if steps.size else 0.0
    print(f"  {what}: {n1} of {err.size} elements differ (at most {worst:.3g} bf16 steps)")
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / tol, 0)), err.shape)
        detail = f"at {i}: gpu {gpu[i]:.9g} oracle {ora[i]:.9g} old {old[i]:.9g} row step {row[i[:-1]][0]:.3g}"
    else:
        detail = ""
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {err.size} elements beyond one bf16 step and the "
                           f"arithmetic allowance; worst {worst:.3g} steps; {detail}")
    return n1, worst


# Arithmetic allowances of ulp_check: fp32 sums of a value row's reads, and
# the key step's MFMA product (operand split in two bf16 parts, about 16
# significant bits) summed over a chunk's tokens.
ARITH_V = 2.0 ** -16
ARITH_K = 2.0 ** -10
