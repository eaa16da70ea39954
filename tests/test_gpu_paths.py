"""GPU: the two scoring paths.  Chunks whose token tiles fill the chip use the
two-pass sweep; short chunks (decode, one long sequence) score whole rows and
take their statistics by reductions over the stored rows.  Both must select
the same slots with the same weights, and both must agree with the oracle."""
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
    os.environ.pop("FWPKM_SCORE_PATH", None)


def C(n, H, dq, dv, kh, k, chunk=64, store="f32", **kw):
    return FwpkmConfig(n=n, heads=H, d_q=dq, d_v=dv, k_half=kh, k=k, chunk=chunk, store=store, **kw)


def dev(*ts):
    return [t.to(DEV).contiguous() for t in ts]


def run(path, fn):
    os.environ["FWPKM_SCORE_PATH"] = path
    try:
        out = fn()
        torch.cuda.synchronize()
        return out
    finally:
        del os.environ["FWPKM_SCORE_PATH"]


CASES = [
    ("f32_idw", C(64, 2, 64, 64, 8, 8, chunk=48, lr_k=20.0)),
    ("bf16_idw", C(128, 2, 256, 128, 16, 16, chunk=64, store="bf16", lr_k=20.0)),
    ("f32_dot", C(64, 2, 64, 64, 8, 8, chunk=48, lr_k=20.0, score="dot")),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paths_select_identically(case):
    name, cfg = case
    B, T = 2, 90
    q, v, g, _ = make_tokens(cfg, B, T, 61, "gauss")
    K1, K2, V = make_state(cfg, B, 61, std=0.5)
    d = dev(q, v, g, K1, K2, V)
    a = run("sweep", lambda: fwpkm.fwpkm_retrieve(cfg, *d))
    b = run("rows", lambda: fwpkm.fwpkm_retrieve(cfg, *d))
    for key in ("idx", "w", "o", "vhat"):
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paths_agree_with_oracle_over_a_sequence(case):
    """forward_seq along both paths, each chunk's write checked against the
    oracle from the GPU's own state (chunk-resynchronised)."""
    name, cfg = case
    B, T = 2, 150
    q, v, g, _ = make_tokens(cfg, B, T, 62, "gauss")
    K1, K2, V = make_state(cfg, B, 62, std=0.5)
    rt = rtol_for(cfg)
    for path in ("sweep", "rows"):
        os.environ["FWPKM_SCORE_PATH"] = path
        K1d, K2d, Vd = dev(K1, K2, V)
        for t0 in range(0, T, cfg.chunk):
            t1 = min(T, t0 + cfg.chunk)
            s_K1, s_K2, s_V = (x.cpu() for x in (K1d, K2d, Vd))
            qc, vc, gc = (x[:, t0:t1].contiguous() for x in (q, v, g))
            r = fwpkm.fwpkm_retrieve(cfg, qc.to(DEV), vc.to(DEV), gc.to(DEV), K1d, K2d, Vd)
            n_tgt = (t1 - t0) if t1 < T else (t1 - t0 - 1)
            tgt = v[:, t0 + 1:t0 + 1 + n_tgt].contiguous()
            fwpkm.fwpkm_chunk_update(cfg, qc.to(DEV), gc.to(DEV), tgt.to(DEV), n_tgt, r["idx"], r["w"], r["vhat"],
                                     K1d, K2d, Vd)
            torch.cuda.synchronize()
            K1o, K2o, Vo, _ = oracle.chunk_update(cfg, qc, gc, tgt, n_tgt, r["idx"].cpu().numpy(),
                                                  r["w"].cpu().numpy().astype(np.float64),
                                                  r["vhat"].cpu().numpy().astype(np.float64), s_K1, s_K2, s_V)
            for got, want, nm in ((Vd, Vo, "V"), (K1d, K1o, "K1"), (K2d, K2o, "K2")):
                g64 = got.float().cpu().numpy().astype(np.float64)
                w64 = np.asarray(want)
                if w64.dtype == np.uint16:
                    w64 = torch.from_numpy(w64.view(np.int16)).view(torch.bfloat16).float().numpy()
                close(g64, w64.astype(np.float64), rt, what=f"{path} {nm} chunk@{t0}")
        del os.environ["FWPKM_SCORE_PATH"]


def test_long_workload_uses_rows_and_matches_sweep_selection():
    """The 128K-token single-sequence layer: a chunk of 512 tokens (16 tiles
    of 64 for a 256-CU chip) takes the rows path; its selection equals the
    sweep's."""
    wl = WORKLOADS["long"]
    cfg = wl.cfg
    q, v, g, _ = make_tokens(cfg, 1, 512, wl.seed, "gauss")
    K1, K2, V = make_state(cfg, 1, wl.seed)
    d = dev(q[:, :512], v[:, :512], g[:, :512], K1, K2, V)
    a = run("sweep", lambda: fwpkm.fwpkm_retrieve(cfg, *d))
    b = fwpkm.fwpkm_retrieve(cfg, *d)
    torch.cuda.synchronize()
    for key in ("idx", "w", "o"):
        assert torch.equal(a[key], b[key]), key
