"""GPU: row-contribution counts and the addressing metrics (paperlayer.ai D.3)
through the C ABI, against counts of the path's own slot ids and the oracle's
metrics of the same counts."""
import numpy as np
import pytest
import torch

import oracle
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


def C(n, H, dq, dv, kh, k, chunk=64, store="f32", **kw):
    return FwpkmConfig(n=n, heads=H, d_q=dq, d_v=dv, k_half=kh, k=k, chunk=chunk, store=store, **kw)


def dev(*ts):
    return [t.to(DEV).contiguous() for t in ts]


def chunked_idx(cfg, q, v, g, K1d, K2d, Vd):
    """Slot ids of every token from a chunk-by-chunk replay (retrieve + update)."""
    B, T = g.shape
    out = []
    for t0 in range(0, T, cfg.chunk):
        t1 = min(T, t0 + cfg.chunk)
        qc, vc, gc = (x[:, t0:t1].contiguous().to(DEV) for x in (q, v, g))
        r = fwpkm.fwpkm_retrieve(cfg, qc, vc, gc, K1d, K2d, Vd)
        n_tgt = (t1 - t0) if t1 < T else (t1 - t0 - 1)
        tgt = v[:, t0 + 1:t0 + 1 + n_tgt].contiguous().to(DEV)
        fwpkm.fwpkm_chunk_update(cfg, qc, gc, tgt, n_tgt, r["idx"], r["w"], r["vhat"], K1d, K2d, Vd)
        out.append(r["idx"].cpu())
    return torch.cat(out, 1).numpy()


@pytest.mark.parametrize("store,passes", [("f32", 1), ("bf16", 2)])
def test_forward_seq_usage_counts_every_read(store, passes):
    cfg = C(64, 2, 64, 64, 8, 8, chunk=24, store=store)
    B, T = 2, 100
    q, v, g, _ = make_tokens(cfg, B, T, 41, "gauss")
    K1, K2, V = make_state(cfg, B, 41, std=0.5)
    qd, vd, gd, K1a, K2a, Va = dev(q, v, g, K1, K2, V)
    usage = torch.zeros((B, cfg.N), dtype=torch.int32, device=DEV)
    out = fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, K1a, K2a, Va, passes=passes, usage=usage)
    K1b, K2b, Vb = dev(K1, K2, V)
    ref = fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, K1b, K2b, Vb, passes=passes)
    torch.cuda.synchronize()
    assert torch.equal(out["o"], ref["o"]) and torch.equal(Va, Vb)  # counting changes nothing else
    K1c, K2c, Vc = dev(K1, K2, V)
    expect = np.zeros((B, cfg.N), np.int64)
    for _ in range(passes):
        expect += oracle.usage_counts(cfg, chunked_idx(cfg, q, v, g, K1c, K2c, Vc))
    assert np.array_equal(usage.cpu().numpy(), expect)
    m = fwpkm.fwpkm_usage_metrics(cfg, usage, reset=True)
    torch.cuda.synchronize()
    np.testing.assert_allclose(m.cpu().numpy(), oracle.usage_metrics(expect), rtol=1e-12, atol=1e-15)
    assert int(usage.abs().sum()) == 0  # reset starts the next interval
    m2 = fwpkm.fwpkm_usage_metrics(cfg, usage)
    torch.cuda.synchronize()
    assert torch.equal(m2.cpu(), torch.zeros((B, 4), dtype=torch.float64))


def test_stream_usage_equals_forward_seq_usage():
    cfg = C(64, 1, 64, 64, 8, 8, chunk=16)
    B, T = 2, 50
    q, v, g, _ = make_tokens(cfg, B, T, 42, "gauss")
    K1, K2, V = make_state(cfg, B, 42, std=0.5)
    qd, vd, gd, K1a, K2a, Va = dev(q, v, g, K1, K2, V)
    ua = torch.zeros((B, cfg.N), dtype=torch.int32, device=DEV)
    fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, K1a, K2a, Va, usage=ua)
    K1b, K2b, Vb = dev(K1, K2, V)
    ub = torch.zeros((B, cfg.N), dtype=torch.int32, device=DEV)
    st, pos = fwpkm.stream_state(cfg, B, DEV)
    for a, b in zip([0, 1, 2, 9, 16, 17, 33], [1, 2, 9, 16, 17, 33, 50]):
        fwpkm.fwpkm_stream_step(cfg, *dev(q[:, a:b], v[:, a:b], g[:, a:b]), K1b, K2b, Vb, st, pos, usage=ub)
    fwpkm.fwpkm_stream_flush(cfg, K1b, K2b, Vb, st, pos)
    torch.cuda.synchronize()
    assert torch.equal(ua, ub)


def test_usage_metrics_million_workload():
    """The 1M-slot layer at its benchmark batch (16 sequences x 4096 tokens):
    counts sum to every read, metrics equal the oracle's of the same counts."""
    wl = WORKLOADS["million"]
    cfg = wl.cfg
    q, v, g, _ = make_tokens(cfg, wl.B, wl.T, wl.seed, wl.kind)
    K1, K2, V = make_state(cfg, wl.B, wl.seed, device=DEV)
    qd, vd, gd = dev(q, v, g)
    usage = torch.zeros((wl.B, cfg.N), dtype=torch.int32, device=DEV)
    fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, K1, K2, V, usage=usage)
    m = fwpkm.fwpkm_usage_metrics(cfg, usage)
    torch.cuda.synchronize()
    counts = usage.cpu().numpy()
    assert (counts.sum(1) == wl.T * cfg.heads * cfg.k).all()
    ref = oracle.usage_metrics(counts)
    np.testing.assert_allclose(m.cpu().numpy(), ref, rtol=1e-12, atol=1e-15)
    print("  coverage %.4f collision %.4f KLD %.4f" % tuple(ref[:, :3].mean(0)))
