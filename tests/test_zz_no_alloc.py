"""GPU: fwpkm_forward_seq_static (the library's static scratch in place of a
workspace) against fwpkm_forward_seq on the same inputs, through the C ABI:
outputs and final state equal bit for bit, on two calls in a row, the second
smaller than the first (the scratch keeps the first call's contents)."""
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


def _inputs(cfg, B, T, seed):
    q, v, g, _ = make_tokens(cfg, B, T, seed, "gauss")
    K1, K2, V = make_state(cfg, B, seed, std=0.5)
    return [x.to(DEV).contiguous() for x in (q, v, g)], [x.to(DEV).contiguous() for x in (K1, K2, V)]


def _bits(x):
    return x.contiguous().view(-1).view(torch.uint8)


@pytest.mark.parametrize("store", ["bf16", "f32"])
def test_static_scratch_equals_workspace_call(store):
    cfg = FwpkmConfig(n=256, heads=2, d_q=128, d_v=128, k_half=16, k=16, chunk=256, store=store)
    for B, T, seed in ((4, 1024, 71), (2, 600, 72)):  # the second call is smaller and ragged
        print(f"  B={B} T={T} {store}", flush=True)
        (q, v, g), state = _inputs(cfg, B, T, seed)
        ref_state = [x.clone() for x in state]
        ref = fwpkm.fwpkm_forward_seq(cfg, q, v, g, *ref_state, passes=2, want_vhat=True)
        got = fwpkm.fwpkm_forward_seq_static(cfg, q, v, g, *state, passes=2, want_vhat=True)
        torch.cuda.synchronize()
        for k in ("o", "vhat"):
            assert torch.equal(_bits(got[k]), _bits(ref[k])), f"{k} B={B} T={T}"
        for nm, a, b in zip(("K1", "K2", "V"), state, ref_state):
            assert torch.equal(_bits(a), _bits(b)), f"{nm} B={B} T={T}"


def test_static_scratch_million_layer_one_chunk_step():
    """The 2^20-slot layer at its full batch of 16 sequences (the largest
    configuration the scratch holds), one chunk per sequence."""
    cfg = FwpkmConfig(n=1024, heads=4, d_q=512, d_v=512, k_half=32, k=32, chunk=512, store="bf16")
    B, T = 16, 512
    (q, v, g), state = _inputs(cfg, B, T, 73)
    ref_state = [x.clone() for x in state]
    ref = fwpkm.fwpkm_forward_seq(cfg, q, v, g, *ref_state)
    got = fwpkm.fwpkm_forward_seq_static(cfg, q, v, g, *state)
    torch.cuda.synchronize()
    assert torch.equal(_bits(got["o"]), _bits(ref["o"]))
    for nm, a, b in zip(("K1", "K2", "V"), state, ref_state):
        assert torch.equal(_bits(a), _bits(b)), nm
