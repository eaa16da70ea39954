"""GPU: the value write over planted slot lists -- long runs of one row,
ragged read counts across sort tiles, and out-of-range slot ids (the read
of no row: they add to no row's sum and no row's read count).  N_read must
be exact and V within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from parity import close, rtol_for
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


def C(n, H, dq, dv, kh, k, chunk, store="f32", **kw):
    return FwpkmConfig(n=n, heads=H, d_q=dq, d_v=dv, k_half=kh, k=k, chunk=chunk, store=store, **kw)


def planted(cfg, B, Tc, seed, hot, bad):
    """Slot lists drawn from `hot` distinct rows per sequence (so runs of
    equal slots are long), a fraction `bad` of them out of range (-1 or
    >= N, which the write skips), softmax-like weights."""
    gen = torch.Generator().manual_seed(seed)
    rows = torch.randint(0, cfg.N, (B, hot), generator=gen)
    pick = torch.randint(0, hot, (B, Tc, cfg.heads, cfg.k), generator=gen)
    idx = torch.gather(rows, 1, pick.view(B, -1)).view(B, Tc, cfg.heads, cfg.k).to(torch.int32)
    flip = torch.rand(idx.shape, generator=gen) < bad
    wild = torch.where(torch.rand(idx.shape, generator=gen) < 0.5, torch.full_like(idx, -1),
                       torch.full_like(idx, cfg.N + 3))
    idx = torch.where(flip, wild, idx)
    w = torch.softmax(torch.randn(idx.shape, generator=gen), -1).float()
    return idx, w


def run(cfg, B, Tc, n_tgt, seed, hot, bad):
    q, v, g, _ = make_tokens(cfg, B, Tc + 1, seed, "gauss")
    K1, K2, V = make_state(cfg, B, seed, std=0.5)
    idx, w = planted(cfg, B, Tc, seed, hot, bad)
    vhat = torch.randn((B, Tc, cfg.d_v), generator=torch.Generator().manual_seed(seed + 1))
    tgt = v[:, 1:n_tgt + 1].contiguous()
    d = [x.to(DEV) for x in (q[:, :Tc].contiguous(), g[:, :Tc].contiguous(), tgt, idx, w, vhat, K1, K2, V)]
    nr = torch.empty((B, cfg.N), dtype=torch.int32, device=DEV)
    fwpkm.fwpkm_chunk_update(cfg, d[0], d[1], d[2], n_tgt, d[3], d[4], d[5], d[6], d[7], d[8], n_read=nr)
    torch.cuda.synchronize()
    return d[8].cpu(), nr.cpu(), (q, g, tgt, idx, w, vhat, K1, K2, V)


CASES = [
    # (name, cfg, B, Tc, n_tgt, hot rows, out-of-range fraction); reads per sequence = n_tgt*H*k
    ("tiny_m504", C(128, 1, 64, 64, 8, 8, chunk=64), 2, 64, 63, 40, 0.0),
    ("ragged_m3192", C(64, 2, 64, 64, 8, 8, chunk=200), 3, 200, 199, 300, 0.05),
    ("hot_rows_m8192", C(64, 4, 64, 64, 8, 16, chunk=128), 2, 128, 128, 7, 0.02),
    ("max_m16384_bf16", C(256, 4, 64, 64, 16, 16, chunk=256, store="bf16"), 2, 256, 256, 5000, 0.01),
    ("over_m16416", C(128, 1, 64, 64, 32, 32, chunk=1024), 2, 513, 513, 2000, 0.01),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_planted_write_matches_oracle(case):
    name, cfg, B, Tc, n_tgt, hot, bad = case
    Vg, nr, (q, g, tgt, idx, w, vhat, K1, K2, V) = run(cfg, B, Tc, n_tgt, 82, hot, bad)
    _, _, Vo, nro = oracle.chunk_update(cfg.replace(use_addr=False), q[:, :Tc].contiguous(), g[:, :Tc].contiguous(),
                                        tgt, n_tgt, idx.numpy(), w.numpy().astype(np.float64),
                                        vhat.numpy().astype(np.float64), K1, K2, V)
    assert np.array_equal(nr.numpy(), nro)
    Vo = np.asarray(Vo)
    if Vo.dtype == np.uint16:
        Vo = torch.from_numpy(Vo.view(np.int16)).view(torch.bfloat16).float().numpy()
    close(Vg.float().numpy().astype(np.float64), Vo.astype(np.float64), rtol_for(cfg), what=f"{name} V")
