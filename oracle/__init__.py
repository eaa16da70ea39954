"""CPU oracle of the FwPKM layer's hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never calls it, and it never calls the product path: the two
share no code.  The arithmetic lives in ``fwpkm_oracle.c`` (plain C, fp64);
this module only compiles it with gcc and marshals numpy arrays through
ctypes.

Configuration objects are duck-typed: anything with the attributes ``n,
heads, d_q, d_v, k_half, k, chunk, store ('f32'|'bf16'), idw_eps, lr_v, lr_k,
lookahead, znorm, znorm_eps, use_addr`` works (optionally ``gate_weight`` and
``score`` ('idw' | 'dot'), default True and 'idw').

Storage-typed arrays (q, v, targets, K1, K2, V) are float32 arrays for
``store='f32'`` and uint16 arrays holding bf16 bit patterns for
``store='bf16'``; torch tensors are accepted and converted.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fwpkm_oracle.c")
_SO = os.path.join(_HERE, "libfwpkm_oracle.so")

_GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libfwpkm_oracle.so``."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        cmd = ["gcc", *_GCC_FLAGS, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int32), ("heads", ctypes.c_int32), ("d_q", ctypes.c_int32),
        ("d_v", ctypes.c_int32), ("k_half", ctypes.c_int32), ("k", ctypes.c_int32),
        ("chunk", ctypes.c_int32), ("store", ctypes.c_int32),
        ("idw_eps", ctypes.c_double), ("lr_v", ctypes.c_double), ("lr_k", ctypes.c_double),
        ("lookahead", ctypes.c_int32), ("znorm", ctypes.c_int32),
        ("znorm_eps", ctypes.c_double), ("use_addr", ctypes.c_int32),
        ("gate_weight", ctypes.c_int32), ("score", ctypes.c_int32),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_SO)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        lib.fwo_retrieve.argtypes = [ctypes.POINTER(_Cfg), i32, i32, P, P, P, P, P, P,
                                     P, P, P, P, P, P, ctypes.c_double]
        lib.fwo_chunk_update.argtypes = [ctypes.POINTER(_Cfg), i32, i32, i32, P, P, P,
                                         P, P, P, P, P, P, P]
        lib.fwo_forward_seq.argtypes = [ctypes.POINTER(_Cfg), i32, i32, i32, P, P, P, P,
                                        P, P, P, P, P, i32]
        lib.fwo_pair_p.argtypes = [ctypes.POINTER(_Cfg), i32, i32, i32, P, P, P, P, P]
        lib.fwo_double_to_bf16.argtypes = [ctypes.c_double]
        lib.fwo_double_to_bf16.restype = ctypes.c_uint16
        lib.fwo_num_threads.restype = ctypes.c_int
        lib.fwo_set_threads.argtypes = [ctypes.c_int]
        lib.fwo_set_threads.restype = None
        for f in (lib.fwo_retrieve, lib.fwo_chunk_update, lib.fwo_forward_seq, lib.fwo_pair_p):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _cfg(c) -> _Cfg:
    store = {"f32": 0, "bf16": 1}[c.store]
    return _Cfg(int(c.n), int(c.heads), int(c.d_q), int(c.d_v), int(c.k_half), int(c.k),
                int(c.chunk), store, float(c.idw_eps), float(c.lr_v), float(c.lr_k),
                int(bool(c.lookahead)), int(bool(c.znorm)), float(c.znorm_eps),
                int(bool(c.use_addr)), int(bool(getattr(c, "gate_weight", True))),
                {"idw": 0, "dot": 1}[getattr(c, "score", "idw")])


def _np(x, dtype):
    """Contiguous numpy copy-or-view of x with the given dtype."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16).numpy().view(np.uint16)
            else:
                x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(x)
    if a.dtype != dtype:
        if dtype == np.uint16:
            raise TypeError("bf16 storage arrays must hold uint16 bit patterns")
        a = a.astype(dtype)
    return a


def _sdt(c):
    return np.float32 if c.store == "f32" else np.uint16


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().fwo_num_threads())


def set_threads(n: int) -> None:
    """Thread count of later oracle calls (the OpenMP default is every core)."""
    _load().fwo_set_threads(int(n))


def double_to_bf16(x: float) -> int:
    return int(_load().fwo_double_to_bf16(float(x)))


def retrieve(c, q, v, g, K1, K2, V, tie_rel: float = 0.0):
    """Frozen-state retrieval of every token.  Returns a dict with o, vhat
    ([B,T,d_v] float64), idx ([B,T,H,k] int32), w and P ([B,T,H,k] float64)
    and tie ([B,T,H] uint8)."""
    lib = _load()
    sdt = _sdt(c)
    q, v, K1, K2, V = (_np(x, sdt) for x in (q, v, K1, K2, V))
    g = _np(g, np.float32)
    B, T = g.shape
    H, k, dv = c.heads, c.k, c.d_v
    o = np.zeros((B, T, dv)); vh = np.zeros((B, T, dv))
    idx = np.zeros((B, T, H, k), np.int32); w = np.zeros((B, T, H, k)); P = np.zeros((B, T, H, k))
    tie = np.zeros((B, T, H), np.uint8)
    cc = _cfg(c)
    rc = lib.fwo_retrieve(ctypes.byref(cc), B, T, _p(q), _p(v), _p(g), _p(K1), _p(K2), _p(V),
                          _p(o), _p(vh), _p(idx), _p(w), _p(P), _p(tie), float(tie_rel))
    if rc != 0:
        raise ValueError("fwo_retrieve rejected its arguments")
    return {"o": o, "vhat": vh, "idx": idx, "w": w, "P": P, "tie": tie}


def chunk_update(c, q, g, tgt, n_tgt, idx, w, vhat, K1, K2, V, want_n_read: bool = True):
    """One chunk's write.  Returns new copies (K1, K2, V, n_read)."""
    lib = _load()
    sdt = _sdt(c)
    q = _np(q, sdt)
    g = _np(g, np.float32)
    B, Tc = g.shape
    tgt = _np(tgt, sdt) if tgt is not None else None
    idx = _np(idx, np.int32)
    w = _np(w, np.float64)
    vhat = _np(vhat, np.float64)
    K1 = _np(K1, sdt).copy(); K2 = _np(K2, sdt).copy(); V = _np(V, sdt).copy()
    N = c.n * c.n
    nr = np.zeros((B, N), np.int32) if want_n_read else None
    cc = _cfg(c)
    rc = lib.fwo_chunk_update(ctypes.byref(cc), B, Tc, int(n_tgt), _p(q), _p(g), _p(tgt),
                              _p(idx), _p(w), _p(vhat), _p(K1), _p(K2), _p(V), _p(nr))
    if rc != 0:
        raise ValueError("fwo_chunk_update rejected its arguments")
    return K1, K2, V, nr


def forward_seq(c, q, v, g, K1, K2, V, passes: int = 1, v_next=None, chunk_limit: int = 0):
    """Whole sequences.  Returns dict(o, vhat, K1, K2, V) with new state copies."""
    lib = _load()
    sdt = _sdt(c)
    q, v = _np(q, sdt), _np(v, sdt)
    g = _np(g, np.float32)
    vn = _np(v_next, sdt) if v_next is not None else None
    K1 = _np(K1, sdt).copy(); K2 = _np(K2, sdt).copy(); V = _np(V, sdt).copy()
    B, T = g.shape
    o = np.zeros((B, T, c.d_v)); vh = np.zeros((B, T, c.d_v))
    cc = _cfg(c)
    rc = lib.fwo_forward_seq(ctypes.byref(cc), B, T, int(passes), _p(q), _p(v), _p(g), _p(vn),
                             _p(K1), _p(K2), _p(V), _p(o), _p(vh), int(chunk_limit))
    if rc != 0:
        raise ValueError("fwo_forward_seq rejected its arguments")
    return {"o": o, "vhat": vh, "K1": K1, "K2": K2, "V": V}


def pair_p(c, q, K1, K2, slots):
    """(eps+d1)(eps+d2) for slots[B,T,H,m] in double."""
    lib = _load()
    sdt = _sdt(c)
    q, K1, K2 = _np(q, sdt), _np(K1, sdt), _np(K2, sdt)
    slots = _np(slots, np.int32)
    B, T, H, m = slots.shape
    P = np.zeros((B, T, H, m))
    cc = _cfg(c)
    rc = lib.fwo_pair_p(ctypes.byref(cc), B, T, m, _p(q), _p(K1), _p(K2), _p(slots), _p(P))
    if rc != 0:
        raise ValueError("fwo_pair_p rejected its arguments")
    return P


def _f64(c, x):
    """Storage array (fp32, or bf16 bit patterns) -> float64 numpy, exactly."""
    a = _np(x, _sdt(c))
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def retrieve_backward(c, q, v, g, K1, K2, V, idx, dO):
    """Gradients of the retrieval output o w.r.t. q, v and g for the upstream
    gradient dO[B,T,d_v], the slot selection idx[B,T,H,k] held fixed (top-k
    is piecewise constant) and the state (K1, K2, V) as given.

    The forward is written out in plain torch (CPU, float64) from the same
    definitions as fwo_retrieve: per head and half d = ||q_half - K_i||^2,
    pair score S = -log(eps + d1) - log(eps + d2) (with dot scoring
    S = q1 . K1_i + q2 . K2_j) of each selected slot
    i*n + j, w = softmax of the k scores, v_hat = (1/H) sum_h sum_j w V[slot],
    o = g v_hat + (1 - g) v; torch autograd takes the gradient.
    Returns dict(dq [B,T,H,d_q], dv [B,T,d_v], dg [B,T], o [B,T,d_v]) float64."""
    import torch
    n, H, dh = c.n, c.heads, c.d_q // 2
    qt = torch.tensor(_f64(c, q), requires_grad=True)
    vt = torch.tensor(_f64(c, v), requires_grad=True)
    gt = torch.tensor(_np(g, np.float32).astype(np.float64), requires_grad=True)
    K1t, K2t, Vt = (torch.tensor(_f64(c, x)) for x in (K1, K2, V))
    it = torch.tensor(_np(idx, np.int32).astype(np.int64))
    G = torch.tensor(np.asarray(dO, dtype=np.float64))
    B, T = gt.shape
    k = it.shape[-1]
    bi = torch.arange(B).view(B, 1, 1, 1).expand(B, T, H, k)
    hi = torch.arange(H).view(1, 1, H, 1).expand(B, T, H, k)
    qh = qt.view(B, T, H, 2, dh)
    k1 = K1t[bi, hi, it // n]  # [B,T,H,k,dh]
    k2 = K2t[bi, hi, it % n]
    if getattr(c, "score", "idw") == "dot":
        S = (qh[:, :, :, None, 0, :] * k1).sum(-1) + (qh[:, :, :, None, 1, :] * k2).sum(-1)
    else:
        d1 = ((qh[:, :, :, None, 0, :] - k1) ** 2).sum(-1)
        d2 = ((qh[:, :, :, None, 1, :] - k2) ** 2).sum(-1)
        S = -torch.log(c.idw_eps + d1) - torch.log(c.idw_eps + d2)
    w = torch.softmax(S, dim=-1)
    rows = Vt[bi, it]  # [B,T,H,k,d_v]
    vhat = (w[..., None] * rows).sum(3).mean(2)
    o = gt[..., None] * vhat + (1.0 - gt[..., None]) * vt
    (o * G).sum().backward()
    return {"dq": qt.grad.numpy(), "dv": vt.grad.numpy(), "dg": gt.grad.numpy(), "o": o.detach().numpy()}


def usage_counts(c, idx):
    """Row contributions ([layer] D.3): the number of reads of every value
    row, per sequence, from slot ids idx[B, T, H, k] -> [B, n*n] int64."""
    idx = np.asarray(idx)
    B = idx.shape[0]
    out = np.zeros((B, c.n * c.n), np.int64)
    for b in range(B):
        np.add.at(out[b], idx[b].reshape(-1).astype(np.int64), 1)
    return out


def usage_metrics(counts):
    """Addressing metrics ([layer] D.3) of row contributions counts[B, N]:
    per sequence (coverage, collision, KLD, reads) as float64 [B, 4].
    coverage = share of rows read at least once; collision = share of reads
    that land on a row read more than once; KLD = KL(u || uniform) with
    u = counts / reads, natural log.  No reads gives zeros."""
    counts = np.asarray(counts, dtype=np.float64)
    B, N = counts.shape
    res = np.zeros((B, 4))
    for b in range(B):
        c = counts[b]
        S = c.sum()
        if S == 0:
            continue
        u = c[c > 0] / S
        res[b] = [np.count_nonzero(c) / N, c[c > 1].sum() / S, float(np.sum(u * np.log(u * N))), S]
    return res


class Stream:
    """Streaming (inference) reading of the layer, token by token.

    [layer] A.1: a prediction never waits for its own lookahead target;
    inference collects (q_t, target) pairs until a chunk of C is full, then
    writes it.  [layer] E.1: the memory state carries over from one
    sequence to the next.  Steps, per arriving token x_j:

      1. with lookahead, v_j completes the pending token before it;
      2. a pending chunk that is complete (C tokens, each with its target)
         is written (chunk_update) before anything else reads the state;
      3. x_j is read against the current state (retrieve) and joins the
         pending chunk, with target v_j when lookahead is off.

    flush() ends the sequences: the pending tokens are written, the last
    one pairing with v_next when given, else without a target.  Plain
    Python over single tokens: for small cases only.
    """

    def __init__(self, c, K1, K2, V):
        sdt = _sdt(c)
        self.c = c
        self.K1 = _np(K1, sdt).copy()
        self.K2 = _np(K2, sdt).copy()
        self.V = _np(V, sdt).copy()
        self.pend = []  # per pending token: dict(q, g, idx, w, vhat, tgt)

    def _write(self, n_tgt):
        c, P = self.c, self.pend
        q = np.stack([e["q"] for e in P], axis=1)
        g = np.stack([e["g"] for e in P], axis=1)
        idx = np.stack([e["idx"] for e in P], axis=1)
        w = np.stack([e["w"] for e in P], axis=1)
        vh = np.stack([e["vhat"] for e in P], axis=1)
        tgt = np.stack([e["tgt"] for e in P[:n_tgt]], axis=1) if n_tgt > 0 else None
        self.K1, self.K2, self.V, _ = chunk_update(c, q, g, tgt, n_tgt, idx, w, vh, self.K1, self.K2, self.V,
                                                   want_n_read=False)
        self.pend = []

    def step(self, q, v, g):
        """q[B,T,H,d_q], v[B,T,d_v], g[B,T] -> dict(o, vhat) of the T tokens."""
        c = self.c
        sdt = _sdt(c)
        q, v = _np(q, sdt), _np(v, sdt)
        g = _np(g, np.float32)
        B, T = g.shape
        o = np.zeros((B, T, c.d_v))
        vh = np.zeros((B, T, c.d_v))
        for j in range(T):
            if c.lookahead and self.pend:
                self.pend[-1]["tgt"] = v[:, j]
            if len(self.pend) == c.chunk:
                self._write(c.chunk)
            r = retrieve(c, q[:, j:j + 1], v[:, j:j + 1], g[:, j:j + 1], self.K1, self.K2, self.V)
            o[:, j] = r["o"][:, 0]
            vh[:, j] = r["vhat"][:, 0]
            self.pend.append({"q": q[:, j], "g": g[:, j], "idx": r["idx"][:, 0], "w": r["w"][:, 0],
                              "vhat": r["vhat"][:, 0], "tgt": None if c.lookahead else v[:, j]})
            if not c.lookahead and len(self.pend) == c.chunk:
                self._write(c.chunk)
        return {"o": o, "vhat": vh}

    def flush(self, v_next=None):
        c = self.c
        if not self.pend:
            return
        n_tgt = len(self.pend)
        if c.lookahead:
            if v_next is not None:
                self.pend[-1]["tgt"] = _np(v_next, _sdt(c))
            else:
                n_tgt -= 1
        self._write(n_tgt)
