"""GPU: gradient of the retrieval output w.r.t. q, v and g through the C ABI
against the oracle's autograd of the same forward (selection and state fixed)."""
import numpy as np
import pytest
import torch

import oracle
from parity import close
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


def C(n, H, dq, dv, kh, k, store="f32", **kw):
    return FwpkmConfig(n=n, heads=H, d_q=dq, d_v=dv, k_half=kh, k=k, chunk=64, store=store, **kw)


CASES = [
    ("f32_n64_h1", C(64, 1, 64, 64, 8, 8), 2, 37, 0.5),
    ("f32_n128_h2_k12", C(128, 2, 128, 128, 16, 12), 1, 40, 0.5),
    ("f32_k_gt_khalf", C(32, 1, 64, 64, 4, 10), 1, 20, 0.5),
    ("bf16_n128_h4", C(128, 4, 256, 256, 16, 16, store="bf16"), 2, 30, 0.3),
    ("bf16_million_layer", C(1024, 4, 512, 512, 32, 32, store="bf16"), 2, 24, 0.02),
    ("dot_f32_n64_h2", C(64, 2, 64, 64, 8, 8, score="dot"), 2, 30, 0.5),
    ("dot_bf16_n128_h4", C(128, 4, 256, 256, 16, 16, store="bf16", score="dot"), 2, 20, 0.3),
]


def _problem(cfg, B, T, kstd, seed=51):
    q, v, g, _ = make_tokens(cfg, B, T, seed, "gauss")
    K1, K2, V = make_state(cfg, B, seed, std=kstd)
    dO = torch.randn((B, T, cfg.d_v), generator=torch.Generator().manual_seed(seed + 1))
    return q, v, g, K1, K2, V, dO


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_retrieve_backward_parity(case):
    name, cfg, B, T, kstd = case
    q, v, g, K1, K2, V, dO = _problem(cfg, B, T, kstd)
    d = [x.to(DEV).contiguous() for x in (q, v, g, K1, K2, V, dO)]
    r = fwpkm.fwpkm_retrieve(cfg, *d[:6])
    gr = fwpkm.fwpkm_retrieve_backward(cfg, *d[:6], r["idx"], r["w"], d[6])
    torch.cuda.synchronize()
    ora = oracle.retrieve_backward(cfg, q, v, g, K1, K2, V, r["idx"].cpu().numpy(), dO.numpy().astype(np.float64))
    close(gr["dv"].cpu().numpy(), ora["dv"], 1e-5, what="dv")
    close(gr["dg"].cpu().numpy(), ora["dg"], 1e-4, what="dg")
    close(gr["dq"].cpu().numpy(), ora["dq"], 1e-3, what="dq")


def test_retrieve_backward_closed_gate_is_exact():
    cfg = C(64, 2, 64, 128, 8, 8)
    q, v, g, K1, K2, V, dO = _problem(cfg, 2, 20, 0.5)
    g = torch.zeros_like(g)
    d = [x.to(DEV).contiguous() for x in (q, v, g, K1, K2, V, dO)]
    r = fwpkm.fwpkm_retrieve(cfg, *d[:6])
    gr = fwpkm.fwpkm_retrieve_backward(cfg, *d[:6], r["idx"], r["w"], d[6])
    torch.cuda.synchronize()
    assert torch.equal(gr["dv"], d[6])
    assert int(torch.count_nonzero(gr["dq"])) == 0
    # dg = dO . (vhat - v)
    ref = (d[6] * (r["vhat"] - d[1])).sum(-1)
    torch.testing.assert_close(gr["dg"], ref, rtol=1e-5, atol=1e-5)


def _chunked_backward(cfg, q, v, g, K1d, K2d, Vd, dO, passes=1, oracle_check=False):
    """Per chunk: retrieve, retrieve_backward (last pass), chunk_update."""
    B, T = g.shape
    outs = {"dq": [], "dv": [], "dg": [], "o": []}
    for p in range(passes):
        for t0 in range(0, T, cfg.chunk):
            t1 = min(T, t0 + cfg.chunk)
            qc, vc, gc = (x[:, t0:t1].contiguous().to(DEV) for x in (q, v, g))
            if oracle_check and p == passes - 1:
                state = [x.cpu() for x in (K1d, K2d, Vd)]
            r = fwpkm.fwpkm_retrieve(cfg, qc, vc, gc, K1d, K2d, Vd)
            if p == passes - 1:
                dc = dO[:, t0:t1].contiguous().to(DEV)
                gr = fwpkm.fwpkm_retrieve_backward(cfg, qc, vc, gc, K1d, K2d, Vd, r["idx"], r["w"], dc)
                for key in ("dq", "dv", "dg"):
                    outs[key].append(gr[key])
                outs["o"].append(r["o"])
                if oracle_check:
                    torch.cuda.synchronize()
                    ora = oracle.retrieve_backward(cfg, qc.cpu(), vc.cpu(), gc.cpu(), *state, r["idx"].cpu().numpy(),
                                                   dc.cpu().numpy().astype(np.float64))
                    close(gr["dq"].cpu().numpy(), ora["dq"], 1e-3, what=f"dq chunk@{t0}")
                    close(gr["dv"].cpu().numpy(), ora["dv"], 1e-5, what=f"dv chunk@{t0}")
                    close(gr["dg"].cpu().numpy(), ora["dg"], 1e-4, what=f"dg chunk@{t0}")
            n_tgt = (t1 - t0) if t1 < T else (t1 - t0 - 1)
            tgt = v[:, t0 + 1:t0 + 1 + n_tgt].contiguous().to(DEV)
            fwpkm.fwpkm_chunk_update(cfg, qc, gc, tgt, n_tgt, r["idx"], r["w"], r["vhat"], K1d, K2d, Vd)
    return {k: torch.cat(x, 1) for k, x in outs.items()}


@pytest.mark.parametrize("store,passes", [("f32", 1), ("bf16", 2)])
def test_forward_seq_backward_equals_chunked_bitwise(store, passes):
    cfg = FwpkmConfig(n=64, heads=2, d_q=64, d_v=128, k_half=8, k=8, chunk=24, store=store, lr_k=20.0)
    B, T = 2, 100
    q, v, g, K1, K2, V, dO = _problem(cfg, B, T, 0.5, seed=52)
    qd, vd, gd, dOd = (x.to(DEV).contiguous() for x in (q, v, g, dO))
    K1a, K2a, Va = (x.to(DEV).contiguous() for x in (K1, K2, V))
    fw = fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, K1a, K2a, Va, passes=passes)
    K1b, K2b, Vb = (x.to(DEV).contiguous() for x in (K1, K2, V))
    bw = fwpkm.fwpkm_forward_seq_backward(cfg, qd, vd, gd, K1b, K2b, Vb, dOd, passes=passes, want_o=True)
    K1c, K2c, Vc = (x.to(DEV).contiguous() for x in (K1, K2, V))
    ref = _chunked_backward(cfg, q, v, g, K1c, K2c, Vc, dO, passes=passes)
    torch.cuda.synchronize()
    assert torch.equal(bw["o"], fw["o"])
    for x, y in ((K1a, K1b), (K2a, K2b), (Va, Vb), (Vb, Vc), (K1b, K1c)):
        assert torch.equal(x, y)
    for key in ("dq", "dv", "dg"):
        assert torch.equal(bw[key], ref[key]), key


def test_forward_seq_backward_tiny_workload_against_oracle():
    """Each chunk's gradient against the oracle's autograd at the GPU's own
    state before that chunk."""
    from sparse_weight_memory_sub_amd.workloads import WORKLOADS
    wl = WORKLOADS["tiny"]
    cfg = wl.cfg
    T = 256
    q, v, g, _ = make_tokens(cfg, wl.B, wl.T, wl.seed, wl.kind)
    q, v, g = q[:, :T], v[:, :T], g[:, :T]
    K1, K2, V = make_state(cfg, wl.B, wl.seed)
    dO = torch.randn((wl.B, T, cfg.d_v), generator=torch.Generator().manual_seed(9))
    K1d, K2d, Vd = (x.to(DEV).contiguous() for x in (K1, K2, V))
    _chunked_backward(cfg, q, v, g, K1d, K2d, Vd, dO, oracle_check=True)
