"""GPU: the streaming (decode) entry points through the C ABI.

fwpkm_stream_step / fwpkm_stream_flush must read and write exactly what
fwpkm_forward_seq does over the same tokens, whatever the split into calls
(checked bit for bit), and agree with the oracle's token-by-token reading
(oracle.Stream, pinned to the oracle's chunked pass on the CPU).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from parity import close
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


def problem(cfg, B, T, seed, kind="gauss", kstd=0.5):
    q, v, g, _ = make_tokens(cfg, B, T, seed, kind)
    K1, K2, V = make_state(cfg, B, seed, std=kstd)
    return q, v, g, K1, K2, V


def dev(*ts):
    return [t.to(DEV).contiguous() for t in ts]


def stream_gpu(cfg, q, v, g, K1d, K2d, Vd, cuts, v_next=None, state=None):
    """Stream tokens [cuts[i], cuts[i+1]) per call, then flush."""
    B = g.shape[0]
    if state is None:
        state = fwpkm.stream_state(cfg, B, DEV)
    st, pos = state
    outs, vhs = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        qd, vd, gd = dev(q[:, a:b], v[:, a:b], g[:, a:b])
        r = fwpkm.fwpkm_stream_step(cfg, qd, vd, gd, K1d, K2d, Vd, st, pos, want_vhat=True)
        outs.append(r["o"])
        vhs.append(r["vhat"])
        assert pos.pending == (((b - 1) % cfg.chunk) + 1 if cfg.lookahead else b % cfg.chunk)
    fwpkm.fwpkm_stream_flush(cfg, K1d, K2d, Vd, st, pos, v_next=None if v_next is None else v_next.to(DEV))
    assert pos.pending == 0
    return torch.cat(outs, 1), torch.cat(vhs, 1), state


def cuts_mixed(T, single=30):
    """Token by token at first, then segments that straddle chunk ends."""
    cuts = list(range(single + 1))
    for c in (35, 47, 48, 49, 72, 73, 95):
        if single < c < T:
            cuts.append(c)
    cuts.append(T)
    return cuts


@pytest.mark.parametrize("store,look,v_next,score", [("f32", True, False, "idw"), ("bf16", True, False, "idw"),
                                                     ("f32", False, False, "idw"), ("bf16", True, True, "idw"),
                                                     ("bf16", True, False, "dot")])
def test_stream_equals_forward_seq_bitwise(store, look, v_next, score):
    cfg = C(64, 2, 64, 128, 8, 8, chunk=24, store=store, lr_k=20.0, lookahead=look, score=score)
    B, T = 2, 100
    q, v, g, K1, K2, V = problem(cfg, B, T, seed=31)
    vn = torch.randn((B, cfg.d_v), generator=torch.Generator().manual_seed(6)).to(cfg.torch_dtype) if v_next else None
    qd, vd, gd, K1a, K2a, Va = dev(q, v, g, K1, K2, V)
    ref = fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, K1a, K2a, Va, v_next=None if vn is None else vn.to(DEV),
                                  want_vhat=True)
    K1b, K2b, Vb = dev(K1, K2, V)
    o, vh, _ = stream_gpu(cfg, q, v, g, K1b, K2b, Vb, cuts_mixed(T), v_next=vn)
    torch.cuda.synchronize()
    assert torch.equal(o, ref["o"])
    assert torch.equal(vh, ref["vhat"])
    for a, b in ((K1a, K1b), (K2a, K2b), (Va, Vb)):
        assert torch.equal(a, b)


def test_stream_carries_state_across_sequences_bitwise():
    cfg = C(64, 1, 64, 64, 8, 8, chunk=16, lr_k=10.0)
    B = 2
    q, v, g, K1, K2, V = problem(cfg, B, 90, seed=32)
    qd, vd, gd, K1a, K2a, Va = dev(q, v, g, K1, K2, V)
    a = fwpkm.fwpkm_forward_seq(cfg, qd[:, :50].contiguous(), vd[:, :50].contiguous(), gd[:, :50].contiguous(),
                                K1a, K2a, Va)
    b = fwpkm.fwpkm_forward_seq(cfg, qd[:, 50:].contiguous(), vd[:, 50:].contiguous(), gd[:, 50:].contiguous(),
                                K1a, K2a, Va)
    K1b, K2b, Vb = dev(K1, K2, V)
    state = fwpkm.stream_state(cfg, B, DEV)
    oa, _, _ = stream_gpu(cfg, q[:, :50], v[:, :50], g[:, :50], K1b, K2b, Vb, list(range(51)), state=state)
    ob, _, _ = stream_gpu(cfg, q[:, 50:], v[:, 50:], g[:, 50:], K1b, K2b, Vb, [0, 7, 16, 17, 40], state=state)
    torch.cuda.synchronize()
    assert torch.equal(oa, a["o"]) and torch.equal(ob, b["o"])
    for x, y in ((K1a, K1b), (K2a, K2b), (Va, Vb)):
        assert torch.equal(x, y)


def test_stream_norms_follow_caller_changes():
    """norms_valid = 0 after the caller edits K: the next call recomputes the
    sub-key norms, so its reads equal a frozen-state retrieval."""
    cfg = C(64, 1, 64, 64, 8, 8, chunk=16)
    B = 1
    q, v, g, K1, K2, V = problem(cfg, B, 20, seed=33)
    K1b, K2b, Vb = dev(K1, K2, V)
    st, pos = fwpkm.stream_state(cfg, B, DEV)
    fwpkm.fwpkm_stream_step(cfg, *dev(q[:, :10], v[:, :10], g[:, :10]), K1b, K2b, Vb, st, pos)
    fwpkm.fwpkm_stream_flush(cfg, K1b, K2b, Vb, st, pos)
    assert pos.norms_valid == 1
    K1b.mul_(1.5)
    pos.norms_valid = 0
    r = fwpkm.fwpkm_stream_step(cfg, *dev(q[:, 10:], v[:, 10:], g[:, 10:]), K1b, K2b, Vb, st, pos)
    ref = fwpkm.fwpkm_retrieve(cfg, *dev(q[:, 10:], v[:, 10:], g[:, 10:]), K1b, K2b, Vb)
    torch.cuda.synchronize()
    assert pos.pending == 10 and pos.norms_valid == 1
    assert torch.equal(r["o"], ref["o"])


def test_stream_tiny_workload_against_oracle():
    """Token-by-token decode of the tiny workload against the oracle's run."""
    wl = WORKLOADS["tiny"]
    cfg = wl.cfg
    T = 300
    q, v, g, _ = make_tokens(cfg, wl.B, wl.T, wl.seed, wl.kind)
    q, v, g = q[:, :T], v[:, :T], g[:, :T]
    K1, K2, V = make_state(cfg, wl.B, wl.seed)
    K1d, K2d, Vd = dev(K1, K2, V)
    o, vh, _ = stream_gpu(cfg, q, v, g, K1d, K2d, Vd, list(range(T + 1)))
    torch.cuda.synchronize()
    ora = oracle.forward_seq(cfg, q, v, g, K1, K2, V)
    on = o.cpu().numpy()
    err = np.abs(on - ora["o"]) / (np.abs(ora["o"]) + np.sqrt(np.mean(ora["o"] ** 2)))
    bad_tok = (err > 1e-4).any(-1)
    print(f"  tokens beyond 1e-4: {int(bad_tok.sum())} of {bad_tok.size}; worst {err.max():.3g}")
    assert bad_tok.mean() <= 0.01
    close(Vd.cpu().numpy().astype(np.float64), ora["V"].astype(np.float64), 1e-3, what="final V")
    close(K1d.cpu().numpy().astype(np.float64), ora["K1"].astype(np.float64), 1e-3, what="final K1")


def test_stream_million_layer_decode_bitwise():
    """The 1M-slot layer (4 heads, d_q = d_v = 512, k = 32, C = 512, bf16) at
    two sequences: 600 tokens decoded one per call, across a chunk write,
    equal forward_seq over the same tokens."""
    cfg = WORKLOADS["million"].cfg
    B, T = 2, 600
    q, v, g, _ = make_tokens(cfg, B, T, 3, "clusters")
    K1, K2, V = make_state(cfg, B, 3)
    qd, vd, gd, K1a, K2a, Va = dev(q, v, g, K1, K2, V)
    ref = fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, K1a, K2a, Va, want_vhat=True)
    K1b, K2b, Vb = dev(K1, K2, V)
    o, vh, _ = stream_gpu(cfg, q, v, g, K1b, K2b, Vb, list(range(T + 1)))
    torch.cuda.synchronize()
    assert torch.equal(o, ref["o"]) and torch.equal(vh, ref["vhat"])
    for a, b in ((K1a, K1b), (K2a, K2b), (Va, Vb)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("n,dup", [(64, 4), (256, 256)])
def test_rows_mode_selection_equals_sweep_with_ties(n, dup):
    """Chunks of at most 16 tokens select from whole rows of distances; with
    exact ties (sub-keys repeated `dup` times, all equal for dup = n) both
    selection paths keep the lower sub-key index."""
    cfg = C(n, 2, 64, 64, 8, 8)
    B, T = 2, 40
    q, v, g, K1, K2, V = problem(cfg, B, T, seed=34)
    K1 = K1.clone()
    for i in range(n):
        K1[:, :, i] = K1[:, :, (i // dup) * dup]
    K1d, K2d, Vd = dev(K1, K2, V)
    os.environ["FWPKM_SCORE_PATH"] = "sweep"
    try:
        full = fwpkm.fwpkm_retrieve(cfg, *dev(q, v, g), K1d, K2d, Vd)  # one 40-token chunk: the sweep
    finally:
        del os.environ["FWPKM_SCORE_PATH"]
    for t0 in range(0, T, 8):
        part = fwpkm.fwpkm_retrieve(cfg, *dev(q[:, t0:t0 + 8], v[:, t0:t0 + 8], g[:, t0:t0 + 8]), K1d, K2d, Vd)
        assert torch.equal(part["idx"], full["idx"][:, t0:t0 + 8])
        if dup < n:
            assert torch.equal(part["w"], full["w"][:, t0:t0 + 8])
            assert torch.equal(part["o"], full["o"][:, t0:t0 + 8])
        else:
            # the sweep's overflow path recomputes the equal distances another way
            torch.testing.assert_close(part["w"], full["w"][:, t0:t0 + 8], rtol=1e-5, atol=1e-6)
    # ties between equal sub-keys go to the lower index, as in the oracle
    ora = oracle.retrieve(cfg, q, v, g, K1, K2, V)
    assert np.array_equal(full["idx"].cpu().numpy(), ora["idx"])


@pytest.mark.parametrize("chunk,cuts", [(24, [0, 100]),            # one call over four chunk writes
                                        (1, [0, 1, 2, 5, 9, 10]),  # a write after every token
                                        (7, [0, 7, 14, 15, 30])])  # calls ending exactly on chunk ends
def test_stream_edge_splits_equal_forward_seq(chunk, cuts):
    cfg = C(64, 2, 64, 64, 8, 8, chunk=chunk, lr_k=10.0)
    B, T = 2, cuts[-1]
    q, v, g, K1, K2, V = problem(cfg, B, T, seed=35)
    qd, vd, gd, K1a, K2a, Va = dev(q, v, g, K1, K2, V)
    ref = fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, K1a, K2a, Va, want_vhat=True)
    K1b, K2b, Vb = dev(K1, K2, V)
    o, vh, _ = stream_gpu(cfg, q, v, g, K1b, K2b, Vb, cuts)
    torch.cuda.synchronize()
    assert torch.equal(o, ref["o"]) and torch.equal(vh, ref["vhat"])
    for a, b in ((K1a, K1b), (K2a, K2b), (Va, Vb)):
        assert torch.equal(a, b)


FUSED_CASES = [
    ("f32_idw_h2", C(64, 2, 64, 64, 8, 8, chunk=24)),
    ("bf16_dot_h3", C(128, 3, 128, 128, 16, 16, chunk=24, store="bf16", score="dot")),
    ("f32_h8_k32", C(64, 8, 64, 64, 32, 32, chunk=24)),    # 16 wavefronts: the most the fused kernel takes
    ("f32_h9_k8", C(64, 9, 64, 64, 8, 8, chunk=24)),       # 18 selection wavefronts: two launches
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_decode_fused_selection_and_read_equal_two_launches(case):
    """Decode (one token per call) with its selection and value read fused in
    one workgroup per token against the two-launch form (FWPKM_DECODE=
    unfused): outputs, slot counts and state bit for bit."""
    name, cfg = case
    B, T = 3, 60
    q, v, g, K1, K2, V = problem(cfg, B, T, seed=44)
    res = []
    for form in ("fused", "unfused"):
        if form == "unfused":
            os.environ["FWPKM_DECODE"] = "unfused"
        try:
            K1d, K2d, Vd = dev(K1, K2, V)
            st, pos = fwpkm.stream_state(cfg, B, DEV)
            usage = torch.zeros((B, cfg.N), dtype=torch.int32, device=DEV)
            outs = []
            for t in range(T):
                qd, vd, gd = dev(q[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1])
                r = fwpkm.fwpkm_stream_step(cfg, qd, vd, gd, K1d, K2d, Vd, st, pos, want_vhat=True, usage=usage)
                outs.append(torch.cat([r["o"], r["vhat"]], -1))
            fwpkm.fwpkm_stream_flush(cfg, K1d, K2d, Vd, st, pos)
            torch.cuda.synchronize()
            res.append((torch.cat(outs, 1), usage, K1d, K2d, Vd))
        finally:
            os.environ.pop("FWPKM_DECODE", None)
    for a, b in zip(*res):
        assert torch.equal(a, b)
    assert int(res[0][1].sum()) == B * T * cfg.heads * cfg.k
