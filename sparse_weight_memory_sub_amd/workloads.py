"""Layer configuration and seeded synthetic inputs for the FwPKM hot path.

This module only describes problems and draws random inputs.  It holds none
of the layer's arithmetic, so both the HIP path and the CPU oracle can be fed
the same bits from it.

The workloads stand in for the paper's data (long-context language data and
Needle-in-a-Haystack tasks, none of which is used here) with shapes taken
from the pages: N of about 10^6 slots (gist.science/es, "Memoria esparsa"),
4K-token training sequences and 128K-token contexts (paperlayer.ai 4.1 and
4.3), chunks of 512 tokens (paperlayer.ai 5.2).  Fast-weight state is drawn
as N(0, 0.02^2).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class FwpkmConfig:
    """Shape and hyper-parameters of one FwPKM layer.

    n: sub-keys per codebook (N = n*n slots); heads: H; d_q: per-head query
    dimension (split into two halves of d_q/2); d_v: value dimension;
    k_half: top-k' kept per half; k: final top-k; chunk: C tokens per
    fast-weight write; store: 'f32' or 'bf16' storage of q, v, K1, K2, V.
    """
    n: int
    heads: int
    d_q: int
    d_v: int
    k_half: int
    k: int
    chunk: int
    store: str = "f32"
    idw_eps: float = 1e-3
    lr_v: float = 1.0
    lr_k: float = 1.0
    lookahead: bool = True
    znorm: bool = True
    znorm_eps: float = 1e-5
    use_addr: bool = True
    gate_weight: bool = True  # memorisation MSE weighted by the gate (paperlayer.ai A.5)
    score: str = "idw"        # sub-key scoring: 'idw' (paperlayer.ai A.2) or 'dot' (PKM's product)

    @property
    def N(self) -> int:
        return self.n * self.n

    @property
    def d_h(self) -> int:
        return self.d_q // 2

    def replace(self, **kw) -> "FwpkmConfig":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self):
        return torch.float32 if self.store == "f32" else torch.bfloat16


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: FwpkmConfig
    B: int
    T: int
    passes: int
    seed: int
    kind: str  # 'linear' | 'gauss' | 'clusters' | 'planted' | 'zipf'
    description: str


WORKLOADS = {
    "tiny": Workload(
        "tiny", FwpkmConfig(n=128, heads=1, d_q=64, d_v=64, k_half=8, k=8, chunk=64, store="f32"),
        B=1, T=1024, passes=1, seed=1, kind="linear",
        description="N=128^2, 1 head, d_q=64, d_v=64, k'=k=8, C=64, B=1, T=1024, fp32; "
                    "q, v, gate logits from seeded random linear maps of h~N(0,1)"),
    "mid": Workload(
        "mid", FwpkmConfig(n=512, heads=4, d_q=256, d_v=256, k_half=16, k=16, chunk=256, store="bf16"),
        B=8, T=4096, passes=1, seed=2, kind="gauss",
        description="N=512^2, 4 heads, d_q=256, d_v=256, k'=k=16, C=256, B=8, T=4096, bf16; "
                    "Gaussian q/v, gate = sigmoid(N(0,1.5^2))"),
    "million": Workload(
        "million", FwpkmConfig(n=1024, heads=4, d_q=512, d_v=512, k_half=32, k=32, chunk=512, store="bf16"),
        B=16, T=4096, passes=1, seed=3, kind="clusters",
        description="N=1024^2, 4 heads, d_q=512, d_v=512, k'=k=32, C=512, B=16, T=4096, bf16; "
                    "queries from 4096 Gaussian clusters (sigma 0.3)"),
    "long": Workload(
        "long", FwpkmConfig(n=1024, heads=1, d_q=512, d_v=512, k_half=32, k=32, chunk=512, store="bf16"),
        B=1, T=131072, passes=1, seed=4, kind="planted",
        description="N=1024^2, 1 head, d_q=512, d_v=512, k=32, C=512, B=1, T=131072 of Gaussian "
                    "filler with 64 planted key->value bindings, 1/2/4 passes"),
    "collision": Workload(
        "collision", FwpkmConfig(n=512, heads=4, d_q=256, d_v=256, k_half=16, k=16, chunk=1024, store="bf16"),
        B=4, T=8192, passes=1, seed=5, kind="zipf",
        description="N=512^2, 4 heads, d_q=256, d_v=256, k=16, C=1024, B=4, T=8192, bf16; "
                    "queries from Zipf(1.2) over 256 centres (sigma 0.05)"),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _store(x: torch.Tensor, cfg: FwpkmConfig) -> torch.Tensor:
    """Cast a float32 tensor to the storage dtype (bf16 casts round to nearest even)."""
    return x.to(cfg.torch_dtype).contiguous()


def make_state(cfg: FwpkmConfig, B: int, seed: int, device="cpu", std: float = 0.02):
    """Fast-weight state K1, K2 [B,H,n,d_h] and V [B,N,d_v], N(0, std^2), in the
    storage dtype.  Drawn on `device` (cuda draws use torch's seeded device
    generator, one sequence at a time to bound temporary memory)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed) * 7919 + 17)
    shapeK = (B, cfg.heads, cfg.n, cfg.d_h)
    K1 = _store(torch.randn(shapeK, generator=g, device=dev) * std, cfg)
    K2 = _store(torch.randn(shapeK, generator=g, device=dev) * std, cfg)
    V = torch.empty((B, cfg.N, cfg.d_v), dtype=cfg.torch_dtype, device=dev)
    for b in range(B):
        V[b] = (torch.randn((cfg.N, cfg.d_v), generator=g, device=dev) * std).to(cfg.torch_dtype)
    return K1, K2, V


def make_tokens(cfg: FwpkmConfig, B: int, T: int, seed: int, kind: str = "gauss",
                gate_std: float = 1.5, **kw):
    """Seeded per-token inputs on the CPU: q [B,T,H,d_q], v [B,T,d_v] (storage
    dtype) and the post-sigmoid gate g [B,T] float32.

    kind:
      'gauss'    q, v ~ N(0,1), g = sigmoid(N(0, gate_std^2));
      'linear'   h ~ N(0,1) of width d_model (default 64); q = h Wq, v = h Wv,
                 g = sigmoid(h wg) with W ~ N(0, 1/d_model);
      'clusters' q = c_u + sigma N(0,I), u uniform over n_centres centres
                 c ~ N(0,I) in the H*d_q space (defaults 4096, 0.3);
      'zipf'     like 'clusters' with centre rank r drawn with P(r) ~ r^-s
                 (defaults 256 centres, s = 1.2, sigma 0.05);
      'planted'  Gaussian filler with n_bind bindings (q*, v*) each planted
                 reps times at random non-overlapping positions p: q_p = q*,
                 v_{p+1} = v* (defaults 64, 16).  Returns the plant table too.
    """
    gen = _gen(seed)
    H, dq, dv = cfg.heads, cfg.d_q, cfg.d_v
    extra = {}
    if kind == "linear":
        dm = int(kw.get("d_model", 64))
        h = torch.randn((B, T, dm), generator=gen)
        Wq = torch.randn((dm, H * dq), generator=gen) / math.sqrt(dm)
        Wv = torch.randn((dm, dv), generator=gen) / math.sqrt(dm)
        wg = torch.randn((dm,), generator=gen) / math.sqrt(dm)
        q = (h @ Wq).reshape(B, T, H, dq)
        v = h @ Wv
        g = torch.sigmoid(h @ wg)
    elif kind in ("gauss", "planted"):
        q = torch.randn((B, T, H, dq), generator=gen)
        v = torch.randn((B, T, dv), generator=gen)
        g = torch.sigmoid(torch.randn((B, T), generator=gen) * gate_std)
        if kind == "planted":
            n_bind = int(kw.get("n_bind", 64))
            reps = int(kw.get("reps", 16))
            qs = torch.randn((n_bind, H, dq), generator=gen)
            vs = torch.randn((n_bind, dv), generator=gen)
            # non-overlapping positions p (each uses p and p+1), p+1 < T
            slots = torch.randperm((T - 1) // 2, generator=gen)[: n_bind * reps]
            pos = (slots * 2).reshape(n_bind, reps)
            for b in range(B):
                for i in range(n_bind):
                    for p in pos[i].tolist():
                        q[b, p] = qs[i]
                        v[b, p + 1] = vs[i]
            extra = {"plant_q": qs, "plant_v": vs, "plant_pos": pos}
    elif kind in ("clusters", "zipf"):
        if kind == "clusters":
            nc = int(kw.get("n_centres", 4096))
            sigma = float(kw.get("sigma", 0.3))
            probs = torch.full((nc,), 1.0 / nc)
        else:
            nc = int(kw.get("n_centres", 256))
            sigma = float(kw.get("sigma", 0.05))
            s = float(kw.get("zipf_s", 1.2))
            ranks = torch.arange(1, nc + 1, dtype=torch.float64)
            probs = (ranks ** -s) / (ranks ** -s).sum()
        centres = torch.randn((nc, H * dq), generator=gen)
        u = torch.multinomial(probs.float(), B * T, replacement=True, generator=gen)
        q = (centres[u] + sigma * torch.randn((B * T, H * dq), generator=gen)).reshape(B, T, H, dq)
        v = torch.randn((B, T, dv), generator=gen)
        g = torch.sigmoid(torch.randn((B, T), generator=gen) * gate_std)
        extra = {"centre": u.reshape(B, T)}
    else:
        raise ValueError("unknown token kind %r" % kind)
    return _store(q, cfg), _store(v, cfg), g.float().contiguous(), extra


def planted_recall(vhat_at, plant_v, eps: float = 1e-5):
    """Recall of planted bindings (an evaluation of the 'planted' inputs, not
    part of the layer): vhat_at[b] is the layer's retrieved value at one
    occurrence of binding b's query; binding b counts as recalled when its
    own z-scored value z(v*_b) (per row over d_v, population variance, eps)
    is the closest in cosine of all bindings' values.  Returns (recall,
    argmax per binding, margin per binding: cosine to the closest value
    minus cosine to the runner-up)."""
    pv = plant_v.double()
    z = (pv - pv.mean(-1, keepdim=True)) / torch.sqrt(pv.var(-1, unbiased=False, keepdim=True) + eps)
    zn = z / z.norm(dim=-1, keepdim=True)
    vh = vhat_at.double()
    vh = vh / vh.norm(dim=-1, keepdim=True).clamp_min(1e-300)
    cos = vh @ zn.T
    top = torch.topk(cos, 2, dim=-1)
    arg = top.indices[:, 0]
    hit = arg == torch.arange(pv.shape[0])
    return float(hit.double().mean()), arg.tolist(), (top.values[:, 0] - top.values[:, 1]).tolist()


def make_workload(name: str, device="cpu", state_device=None, B=None, T=None):
    """Inputs of a named workload: dict(q, v, g, K1, K2, V, extra) with the
    per-token tensors on the CPU and the state on `state_device` (default:
    `device`).  B and T may be overridden (smaller samples of the same kind)."""
    wl = WORKLOADS[name]
    B = wl.B if B is None else B
    T = wl.T if T is None else T
    q, v, g, extra = make_tokens(wl.cfg, B, T, wl.seed, wl.kind)
    K1, K2, V = make_state(wl.cfg, B, wl.seed, device=state_device or device)
    dev = torch.device(device)
    return {"cfg": wl.cfg, "B": B, "T": T, "q": q.to(dev), "v": v.to(dev), "g": g.to(dev),
            "K1": K1, "K2": K2, "V": V, "extra": extra}
