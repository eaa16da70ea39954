"""GPU: the key step split over tokens.  A chunk's 32-token blocks may be
shared out among several workgroups per 64-key block, whose partial sums a
second kernel adds in a fixed order before it updates K1/K2 and their norms.
Every split (forced with FWPKM_KGRAD_SPLIT, ragged block counts included)
must give the oracle's key step; the default rule splits the single-sequence
long-context shape."""
import os

import numpy as np
import pytest
import torch

import oracle
from parity import close, rtol_for
from sparse_weight_memory_sub_amd import fwpkm
from sparse_weight_memory_sub_amd.workloads import WORKLOADS, FwpkmConfig, make_state, make_tokens

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()
    os.environ.pop("FWPKM_KGRAD_SPLIT", None)


def C(n, H, dq, dv, kh, k, chunk, store="f32", **kw):
    return FwpkmConfig(n=n, heads=H, d_q=dq, d_v=dv, k_half=kh, k=k, chunk=chunk, store=store, **kw)


def _bf16_to_f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy()
    return x.astype(np.float64)


def inputs(cfg, B, Tc, seed):
    q, v, g, _ = make_tokens(cfg, B, Tc + 1, seed, "gauss")
    K1, K2, V = make_state(cfg, B, seed, std=0.5)
    return q, v, g, K1, K2, V


def key_step(cfg, Tc, split, q, v, g, K1, K2, V):
    """One chunk's retrieval and write on the GPU with the given split
    (None: the default rule); returns the GPU's and the oracle's K1, K2."""
    if split is None:
        os.environ.pop("FWPKM_KGRAD_SPLIT", None)
    else:
        os.environ["FWPKM_KGRAD_SPLIT"] = str(split)
    qc, gc, tgt = q[:, :Tc].contiguous(), g[:, :Tc].contiguous(), v[:, 1:Tc + 1].contiguous()
    K1d, K2d, Vd = (x.contiguous().to(DEV) for x in (K1, K2, V))
    r = fwpkm.fwpkm_retrieve(cfg, qc.to(DEV), v[:, :Tc].contiguous().to(DEV), gc.to(DEV), K1d, K2d, Vd)
    fwpkm.fwpkm_chunk_update(cfg, qc.to(DEV), gc.to(DEV), tgt.to(DEV), Tc, r["idx"], r["w"], r["vhat"],
                             K1d, K2d, Vd)
    torch.cuda.synchronize()
    K1o, K2o, _, _ = oracle.chunk_update(cfg, qc, gc, tgt, Tc, r["idx"].cpu().numpy(),
                                         r["w"].cpu().numpy().astype(np.float64),
                                         r["vhat"].cpu().numpy().astype(np.float64),
                                         K1.contiguous(), K2.contiguous(), V.contiguous())
    return (K1d, K2d), (_bf16_to_f64(K1o), _bf16_to_f64(K2o))


CASES = [
    # 200 tokens = 7 blocks of 32, the last ragged: splits 2, 3, 4, 8 give
    # 4+3, 3+3+1, 2+2+2+1 and 1 x 7 blocks
    ("f32_idw_dh32", C(64, 2, 64, 64, 8, 8, chunk=200, lr_k=20.0), 200),
    ("f32_idw_dh64", C(96, 1, 128, 64, 8, 8, chunk=200, lr_k=20.0), 200),
    ("bf16_idw_dh128", C(128, 2, 256, 128, 16, 16, chunk=200, store="bf16", lr_k=20.0), 200),
    ("f32_dot_dh32", C(64, 2, 64, 64, 8, 8, chunk=200, lr_k=20.0, score="dot"), 200),
    ("bf16_dot_dh64", C(128, 1, 128, 64, 8, 8, chunk=200, store="bf16", lr_k=20.0, score="dot"), 200),
]


@pytest.mark.parametrize("split", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_key_step_matches_oracle(case, split):
    name, cfg, Tc = case
    (K1d, K2d), (K1o, K2o) = key_step(cfg, Tc, split, *inputs(cfg, 2, Tc, 71))
    rt = rtol_for(cfg)
    close(K1d.float().cpu().numpy().astype(np.float64), K1o, rt, what=f"{name} split {split} K1")
    close(K2d.float().cpu().numpy().astype(np.float64), K2o, rt, what=f"{name} split {split} K2")


@pytest.mark.parametrize("case", CASES[:3], ids=[c[0] for c in CASES[:3]])
def test_split_result_is_fixed_per_split(case):
    """Each split sums in a fixed order: two runs agree bit for bit, and a
    sequence's keys do not depend on the batch it runs in."""
    name, cfg, Tc = case
    x = inputs(cfg, 2, Tc, 72)
    (a1, a2), _ = key_step(cfg, Tc, 3, *x)
    (b1, b2), _ = key_step(cfg, Tc, 3, *x)
    assert torch.equal(a1, b1) and torch.equal(a2, b2)
    (c1, c2), _ = key_step(cfg, Tc, 3, *(t[1:2] for t in x))
    assert torch.equal(a1[1:2], c1) and torch.equal(a2[1:2], c2)


@pytest.mark.parametrize("split", [2, 3, 8])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_split_carried_norms_equal_recomputed(case, split):
    """forward_seq carries the key norms from one chunk's key step to the next
    chunk's scoring; a run resumed at the chunk boundary recomputes them from
    the keys.  Both runs agree bit for bit."""
    name, cfg, Tc = case
    os.environ["FWPKM_KGRAD_SPLIT"] = str(split)
    B, T = 2, 3 * Tc
    q, v, g, _ = make_tokens(cfg, B, T, 74, "gauss")
    K1, K2, V = make_state(cfg, B, 74, std=0.5)
    qd, vd, gd = (x.to(DEV) for x in (q, v, g))
    Sa = [x.to(DEV) for x in (K1, K2, V)]
    full = fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, *Sa)
    Sb = [x.to(DEV) for x in (K1, K2, V)]
    parts = []
    for t0 in range(0, T, Tc):
        t1 = t0 + Tc
        nxt = vd[:, t1].contiguous() if t1 < T else None
        parts.append(fwpkm.fwpkm_forward_seq(cfg, qd[:, t0:t1].contiguous(), vd[:, t0:t1].contiguous(),
                                             gd[:, t0:t1].contiguous(), *Sb, v_next=nxt)["o"])
    torch.cuda.synchronize()
    assert torch.equal(full["o"], torch.cat(parts, 1))
    for x, y in zip(Sa, Sb):
        assert torch.equal(x, y)


def test_long_shape_default_split_matches_oracle():
    """Long-context layer shape (N=1024^2, 1 head, d_h=256, bf16, C=512,
    one sequence, 32 key workgroups): the default rule splits each key
    block's 16 token blocks eight ways; the keys match the oracle."""
    cfg = WORKLOADS["long"].cfg
    (K1d, K2d), (K1o, K2o) = key_step(cfg, cfg.chunk, None, *inputs(cfg, 1, cfg.chunk, 73))
    rt = rtol_for(cfg)
    close(K1d.float().cpu().numpy().astype(np.float64), K1o, rt, what="long K1")
    close(K2d.float().cpu().numpy().astype(np.float64), K2o, rt, what="long K2")
