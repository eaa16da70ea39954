"""GPU: fwpkm_forward_seq's multi-stream schedule (key path on the caller's
stream; gather and value write on a value stream; for chunks under 2^19
reads on the sweep path, selection and sort on a selection stream; lists
and sort buffers alternating by chunk) gives the same bits as the same call
with every kernel on one stream, along both scoring paths, on both sides
of the read threshold, with and without the addressing step, over a
partial last chunk and two passes, and with read counting."""
import os

import pytest
import torch

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
    for k in ("FWPKM_SCORE_PATH", "FWPKM_SINGLE_STREAM"):
        os.environ.pop(k, None)


def C(**kw):
    base = dict(n=256, heads=2, d_q=128, d_v=64, k_half=16, k=16, chunk=256, store="bf16", lr_k=5.0)
    base.update(kw)
    return FwpkmConfig(**base)


def run(cfg, B, T, passes, seed, single, usage):
    if single:
        os.environ["FWPKM_SINGLE_STREAM"] = "1"
    else:
        os.environ.pop("FWPKM_SINGLE_STREAM", None)
    q, v, g, _ = make_tokens(cfg, B, T, seed, "gauss")
    K1, K2, V = (x.to(DEV).contiguous() for x in make_state(cfg, B, seed, std=0.5))
    qd, vd, gd = (x.to(DEV).contiguous() for x in (q, v, g))
    u = torch.zeros((B, cfg.N), dtype=torch.int32, device=DEV) if usage else None
    out = fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, K1, K2, V, passes=passes, want_vhat=True, usage=u)
    torch.cuda.synchronize()
    res = {"o": out["o"], "vhat": out["vhat"], "K1": K1, "K2": K2, "V": V}
    if usage:
        res["usage"] = u
    return {k: x.cpu() for k, x in res.items()}


CASES = [
    # (name, cfg, B, T, passes, scoring path, count reads)
    ("sweep_addr", C(), 4, 1024, 1, "sweep", False),
    ("sweep_no_addr", C(use_addr=False), 4, 1024, 1, "sweep", False),
    ("sweep_ragged_two_passes", C(), 3, 1000, 2, "sweep", False),
    ("sweep_usage", C(store="f32"), 2, 768, 1, "sweep", True),
    ("rows_addr", C(), 2, 1000, 2, "rows", False),
    ("chosen_path", C(chunk=128), 4, 640, 1, None, False),
    # 4 x 1024 x 4 x 32 = 2^19 reads per chunk: selection stays on the key path
    ("sweep_big_chunks", C(heads=4, d_q=64, k_half=32, k=32, chunk=1024), 4, 2048, 1, "sweep", False),
    # two full chunks at 2^19 reads, then a 512-token chunk under it, twice:
    # the schedule changes at the last chunk and again at the next pass
    ("threshold_crossing", C(heads=4, d_q=64, k_half=32, k=32, chunk=1024), 4, 2560, 2, "sweep", False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_multi_stream_schedule_equals_one_stream(case):
    name, cfg, B, T, passes, path, usage = case
    if path:
        os.environ["FWPKM_SCORE_PATH"] = path
    one = run(cfg, B, T, passes, 61, True, usage)
    many = run(cfg, B, T, passes, 61, False, usage)
    # a second multi-stream call on the same (cached) workspace and streams
    again = run(cfg, B, T, passes, 61, False, usage)
    for k in one:
        assert torch.equal(one[k].view(-1).view(torch.uint8), many[k].view(-1).view(torch.uint8)), f"{name} {k}"
        assert torch.equal(many[k].view(-1).view(torch.uint8), again[k].view(-1).view(torch.uint8)), f"{name} {k}"


@pytest.mark.parametrize("path", ["sweep", "rows"])
def test_caller_side_stream(path):
    """Enqueued on a side stream of the caller (default priority): the
    library's streams fork from and join back to that stream, so work the
    caller orders after it sees the finished state, the same bits as a call
    on the current stream."""
    os.environ["FWPKM_SCORE_PATH"] = path
    cfg, B, T = C(), 3, 1000
    ref = run(cfg, B, T, 1, 62, False, False)
    q, v, g, _ = make_tokens(cfg, B, T, 62, "gauss")
    K1, K2, V = (x.to(DEV).contiguous() for x in make_state(cfg, B, 62, std=0.5))
    qd, vd, gd = (x.to(DEV).contiguous() for x in (q, v, g))
    o = torch.empty((B, T, cfg.d_v), dtype=torch.float32, device=DEV)
    vh = torch.empty_like(o)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, K1, K2, V, o=o, vhat=vh, stream=side)
    # ordered after the call on the side stream only
    with torch.cuda.stream(side):
        got = {"o": o.clone(), "vhat": vh.clone(), "K1": K1.clone(), "K2": K2.clone(), "V": V.clone()}
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for k, x in got.items():
        assert torch.equal(x.cpu().view(-1).view(torch.uint8), ref[k].view(-1).view(torch.uint8)), k


def test_side_stream_workspace_not_reused_early(monkeypatch):
    """A call on a side stream with the workspace and outputs allocated by
    the binding: when the call returns the binding drops its workspace.  A
    block of the same size allocated at once on the current stream (which
    does not wait for the side stream, still busy) must not be any block the
    call uses, or work on the current stream could overwrite it while the
    call still runs.  The blocks are compared by address; nothing is written
    to them."""
    os.environ["FWPKM_SCORE_PATH"] = "sweep"
    cfg, B, T = C(), 4, 2048
    ref = run(cfg, B, T, 1, 63, False, False)
    q, v, g, _ = make_tokens(cfg, B, T, 63, "gauss")
    K1, K2, V = (x.to(DEV).contiguous() for x in make_state(cfg, B, 63, std=0.5))
    qd, vd, gd = (x.to(DEV).contiguous() for x in (q, v, g))
    taken = []
    new = fwpkm._new

    def spy(fresh, shape, dtype, device):
        t = new(fresh, shape, dtype, device)
        taken.append((t.data_ptr(), t.numel() * t.element_size()))
        return t

    monkeypatch.setattr(fwpkm, "_new", spy)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)  # keep the side stream busy past the call's return
    out = fwpkm.fwpkm_forward_seq(cfg, qd, vd, gd, K1, K2, V, stream=side, want_vhat=True)
    assert taken, "the binding allocated nothing"
    later = [torch.empty(nb, dtype=torch.uint8, device=DEV) for _, nb in taken]
    busy = not side.query()
    for t in later:
        for p, nb in taken:
            assert not (p <= t.data_ptr() < p + nb), "a block of the running call was handed out again"
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    print(f"  side stream still busy at the check: {busy}")
    got = {"o": out["o"], "vhat": out["vhat"], "K1": K1, "K2": K2, "V": V}
    for k, x in got.items():
        assert torch.equal(x.cpu().view(-1).view(torch.uint8), ref[k].view(-1).view(torch.uint8)), k
    del later
