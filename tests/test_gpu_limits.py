"""GPU: the boundary's limits.  Retrieval and the chunk write at the largest
per-half top-k (k' = 64) with the largest final top-k its candidate table
holds (k = 59: 249 of 256 pairs with rank product <= k), the most reads per
token (heads * k = 256), the smallest codebook (n = 16, k' = n), and a
top-k wider than k', each along both scoring paths, against the oracle."""
import os

import numpy as np
import pytest
import torch

import oracle
from parity import TIE_REL, close, compare_indices, rtol_for, token_set_match
from sparse_weight_memory_sub_amd import fwpkm
from sparse_weight_memory_sub_amd.workloads import FwpkmConfig, make_state, make_tokens

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()
    os.environ.pop("FWPKM_SCORE_PATH", None)


def C(n, H, dq, dv, kh, k, chunk=64, store="f32", **kw):
    return FwpkmConfig(n=n, heads=H, d_q=dq, d_v=dv, k_half=kh, k=k, chunk=chunk, store=store, **kw)


def as_f64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().float().cpu().numpy().astype(np.float64)
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy().astype(np.float64)
    return x.astype(np.float64)


CASES = [
    # (name, cfg, B, T)
    ("khalf64_k59", C(128, 1, 64, 64, 64, 59, lr_k=20.0), 2, 40),
    ("heads8_k32_bf16", C(128, 8, 64, 64, 32, 32, store="bf16", lr_k=20.0), 1, 33),
    ("n16_khalf16", C(16, 2, 64, 128, 16, 16, lr_k=20.0), 2, 37),
    ("k_wider_than_khalf", C(64, 2, 128, 64, 8, 48, lr_k=20.0), 2, 29),
    ("dot_khalf64_k59", C(128, 1, 64, 64, 64, 59, lr_k=20.0, score="dot"), 2, 40),
]


def test_k_beyond_the_candidate_table_is_refused():
    """k = 64 with k' = 64 needs about 300 candidate pairs: refused on the
    host before any launch."""
    cfg = C(128, 1, 64, 64, 64, 64)
    q, v, g, _ = make_tokens(cfg, 1, 4, 92, "gauss")
    K1, K2, V = make_state(cfg, 1, 92)
    with pytest.raises(fwpkm.FwpkmError, match="candidates"):
        fwpkm.fwpkm_retrieve(cfg, *[x.to(DEV).contiguous() for x in (q, v, g, K1, K2, V)])


@pytest.mark.parametrize("path", ["sweep", "rows"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_limits_retrieve_and_write(case, path):
    name, cfg, B, T = case
    os.environ["FWPKM_SCORE_PATH"] = path
    q, v, g, _ = make_tokens(cfg, B, T + 1, 91, "gauss")
    K1, K2, V = make_state(cfg, B, 91, std=0.5)
    qc, vc, gc = (x[:, :T].contiguous() for x in (q, v, g))
    d = [x.to(DEV).contiguous() for x in (qc, vc, gc, K1, K2, V)]
    r = fwpkm.fwpkm_retrieve(cfg, *d)
    torch.cuda.synchronize()
    ora = oracle.retrieve(cfg, qc, vc, gc, K1, K2, V, tie_rel=TIE_REL)
    gi = r["idx"].cpu().numpy()
    exact, near = compare_indices(cfg, qc, K1, K2, gi, ora)
    print(f"  tokens*heads={exact.size} exact={int(exact.sum())} near_ties={near}")
    assert near <= max(2, 0.1 * exact.size)
    m = token_set_match(gi, ora["idx"])
    close(r["w"].cpu().numpy(), ora["w"], 1e-4, mask=exact, what="w")
    close(r["vhat"].cpu().numpy(), ora["vhat"], 1e-4, mask=m, what="vhat")
    # the write from the GPU's own selection, every token with a target
    tgt = v[:, 1:T + 1].contiguous()
    nr = torch.empty((B, cfg.N), dtype=torch.int32, device=DEV)
    fwpkm.fwpkm_chunk_update(cfg, d[0], d[2], tgt.to(DEV), T, r["idx"], r["w"], r["vhat"], d[3], d[4], d[5],
                             n_read=nr)
    torch.cuda.synchronize()
    K1o, K2o, Vo, nro = oracle.chunk_update(cfg, qc, gc, tgt, T, gi, r["w"].cpu().numpy().astype(np.float64),
                                            r["vhat"].cpu().numpy().astype(np.float64), K1, K2, V)
    assert np.array_equal(nr.cpu().numpy(), nro)
    assert int(nro.sum()) == B * T * cfg.heads * cfg.k
    rt = rtol_for(cfg)
    for got, want, nm in ((d[5], Vo, "V"), (d[3], K1o, "K1"), (d[4], K2o, "K2")):
        close(as_f64(got), as_f64(want), rt, what=f"{name} {path} {nm}")
