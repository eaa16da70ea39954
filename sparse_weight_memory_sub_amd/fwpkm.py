"""Thin ctypes binding of libfwpkm.so (include/fwpkm.h).

The functions keep the C entry points' names.  They only check and marshal
torch tensors (device pointers, the current HIP stream, a workspace from the
torch allocator); every step of the layer runs in the library's HIP kernels.
Nothing here falls back to another implementation: if the library or a GPU
is missing, the call raises.
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

from .workloads import FwpkmConfig

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfwpkm.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, -1, -2, -3, -4
_STATUS = {OK: "FWPKM_OK", EINVAL: "FWPKM_EINVAL", EUNSUPPORTED: "FWPKM_EUNSUPPORTED",
           EWORKSPACE: "FWPKM_EWORKSPACE", EHIP: "FWPKM_EHIP"}

EXPORTS = ("fwpkm_abi_version", "fwpkm_last_error", "fwpkm_workspace_bytes",
           "fwpkm_retrieve", "fwpkm_chunk_update", "fwpkm_forward_seq",
           "fwpkm_retrieve_backward", "fwpkm_forward_seq_backward", "fwpkm_forward_seq_usage",
           "fwpkm_usage_metrics",
           "fwpkm_stream_state_bytes", "fwpkm_stream_step", "fwpkm_stream_flush",
           "fwpkm_forward_seq_static", "fwpkm_release_streams", "fwpkm_timing_enable", "fwpkm_timing_read")

# kernel families of fwpkm_timing_read, in fwpkm_kernel order
KERNELS = ("knorm", "score_select", "gather", "resid", "sort", "scatter", "pbar",
           "score_stats", "score_rowstat", "kgrad", "fill", "select", "qt", "pend", "usage", "backward")


class FwpkmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class Cfg(ctypes.Structure):
    _fields_ = [
        ("n", ctypes.c_int32), ("heads", ctypes.c_int32), ("d_q", ctypes.c_int32),
        ("d_v", ctypes.c_int32), ("k_half", ctypes.c_int32), ("k", ctypes.c_int32),
        ("chunk", ctypes.c_int32), ("store", ctypes.c_int32),
        ("idw_eps", ctypes.c_float), ("lr_v", ctypes.c_float), ("lr_k", ctypes.c_float),
        ("lookahead", ctypes.c_int32), ("znorm", ctypes.c_int32),
        ("znorm_eps", ctypes.c_float), ("use_addr", ctypes.c_int32),
        ("gate_weight", ctypes.c_int32), ("score", ctypes.c_int32),
    ]


class StreamPos(ctypes.Structure):
    """fwpkm_stream_pos: host-side position of a decode stream."""
    _fields_ = [("pending", ctypes.c_int32), ("norms_valid", ctypes.c_int32)]


@functools.lru_cache(maxsize=256)
def _cfg(c: FwpkmConfig) -> Cfg:
    """A shared, never modified fwpkm_cfg of the configuration, for the calls."""
    return cfg_struct(c)


def cfg_struct(c: FwpkmConfig) -> Cfg:
    return Cfg(int(c.n), int(c.heads), int(c.d_q), int(c.d_v), int(c.k_half), int(c.k), int(c.chunk),
               {"f32": 0, "bf16": 1}[c.store], float(c.idw_eps), float(c.lr_v), float(c.lr_k),
               int(bool(c.lookahead)), int(bool(c.znorm)), float(c.znorm_eps), int(bool(c.use_addr)),
               int(bool(c.gate_weight)), {"idw": 0, "dot": 1}[c.score])


_lib = None


def load(path: str = LIB_PATH):
    """Load libfwpkm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m sparse_weight_memory_sub_amd.build`")
        lib = ctypes.CDLL(path)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        C = ctypes.POINTER(Cfg)
        lib.fwpkm_abi_version.restype = i32
        lib.fwpkm_last_error.restype = ctypes.c_char_p
        lib.fwpkm_workspace_bytes.argtypes = [C, i32, i32, ctypes.POINTER(sz)]
        lib.fwpkm_retrieve.argtypes = [C, i32, i32, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        lib.fwpkm_chunk_update.argtypes = [C, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        lib.fwpkm_forward_seq.argtypes = [C, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, sz, P]
        SP = ctypes.POINTER(StreamPos)
        lib.fwpkm_stream_state_bytes.argtypes = [C, i32, ctypes.POINTER(sz)]
        lib.fwpkm_stream_step.argtypes = [C, i32, i32, P, P, P, P, P, P, P, P, P, P, SP, P, sz, P]
        lib.fwpkm_forward_seq_usage.argtypes = [C, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        lib.fwpkm_usage_metrics.argtypes = [C, i32, P, P, i32, P, sz, P]
        lib.fwpkm_retrieve_backward.argtypes = [C, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P, P]
        lib.fwpkm_forward_seq_backward.argtypes = [C, i32, i32, i32, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        lib.fwpkm_stream_flush.argtypes = [C, i32, P, P, P, P, P, SP, P, sz, P]
        lib.fwpkm_forward_seq_static.argtypes = [C, i32, i32, i32, P, P, P, P, P, P, P, P, P, P]
        lib.fwpkm_release_streams.argtypes = []
        lib.fwpkm_timing_enable.argtypes = [i32]
        lib.fwpkm_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        for f in (lib.fwpkm_workspace_bytes, lib.fwpkm_retrieve, lib.fwpkm_chunk_update, lib.fwpkm_forward_seq,
                  lib.fwpkm_stream_state_bytes, lib.fwpkm_stream_step, lib.fwpkm_stream_flush,
                  lib.fwpkm_forward_seq_usage, lib.fwpkm_usage_metrics, lib.fwpkm_retrieve_backward,
                  lib.fwpkm_forward_seq_backward, lib.fwpkm_release_streams, lib.fwpkm_forward_seq_static,
                  lib.fwpkm_timing_enable, lib.fwpkm_timing_read):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(rc: int):
    if rc != OK:
        raise FwpkmError(rc, load().fwpkm_last_error().decode())


def abi_version() -> int:
    return int(load().fwpkm_abi_version())


def release_streams() -> None:
    """Destroy the streams and events fwpkm_forward_seq made for this thread."""
    _check(load().fwpkm_release_streams())


def timing_enable(on: bool = True) -> None:
    """Bracket every kernel family launch with HIP events (resets totals when on)."""
    _check(load().fwpkm_timing_enable(1 if on else 0))


def timing_read() -> dict:
    """{family: (total_ms, launches)} of the launches timed since timing_enable(True)."""
    out = {}
    for i, name in enumerate(KERNELS):
        ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
        _check(load().fwpkm_timing_read(i, ctypes.byref(ms), ctypes.byref(n)))
        out[name] = (float(ms.value), int(n.value))
    return out


def workspace_bytes(cfg: FwpkmConfig, B: int, T: int) -> int:
    # the size follows the scoring path and the key step's token split, which
    # FWPKM_SCORE_PATH and FWPKM_KGRAD_SPLIT can override
    return _workspace_bytes(cfg, int(B), int(T), os.environ.get("FWPKM_SCORE_PATH", ""),
                            os.environ.get("FWPKM_KGRAD_SPLIT", ""))


@functools.lru_cache(maxsize=256)
def _workspace_bytes(cfg: FwpkmConfig, B: int, T: int, path: str, ksplit: str) -> int:
    out = ctypes.c_size_t(0)
    c = _cfg(cfg)
    _check(load().fwpkm_workspace_bytes(ctypes.byref(c), int(B), int(T), ctypes.byref(out)))
    return int(out.value)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _new(fresh, shape, dtype, device):
    """A tensor this binding allocates for a call (listed in `fresh`)."""
    t = torch.empty(shape, dtype=dtype, device=device)
    fresh.append(t)
    return t


def _mine(stream, fresh):
    """Tensors this binding allocated (on torch's current stream) for a call
    enqueued on another `stream`: tell the caching allocator that `stream`
    uses them, so a block freed when the call returns (the workspace) or
    later (an output) is not handed to new work before `stream` is done
    with it."""
    if stream is None or not fresh:
        return
    ts = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    if ts.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return
    for t in fresh:
        t.record_stream(ts)


def _workspace(cfg, B, T, ws, device, fresh):
    """The caller's workspace (the library checks its size), or a new one
    (listed in `fresh`)."""
    if ws is None:
        ws = _new(fresh, (max(workspace_bytes(cfg, B, T), 256),), torch.uint8, device)
    return ws, ws.numel() * ws.element_size()


def fwpkm_retrieve(cfg: FwpkmConfig, q, v, g, K1, K2, V, o=None, vhat=None, idx=None, w=None,
                   ws=None, stream=None, want=("vhat", "idx", "w")):
    """Frozen-state retrieval.  Returns dict(o, vhat, idx, w) (outputs are
    allocated when not given and wanted)."""
    sd = cfg.torch_dtype
    B, T = g.shape
    H, dq, dv, k = cfg.heads, cfg.d_q, cfg.d_v, cfg.k
    dev = g.device
    _dev(q, "q", sd, (B, T, H, dq)); _dev(v, "v", sd, (B, T, dv)); _dev(g, "g", torch.float32, (B, T))
    _dev(K1, "K1", sd, (B, H, cfg.n, dq // 2)); _dev(K2, "K2", sd, (B, H, cfg.n, dq // 2))
    _dev(V, "V", sd, (B, cfg.N, dv))
    fresh = []
    o = _new(fresh, (B, T, dv), torch.float32, dev) if o is None else o
    if vhat is None and "vhat" in want:
        vhat = _new(fresh, (B, T, dv), torch.float32, dev)
    if idx is None and "idx" in want:
        idx = _new(fresh, (B, T, H, k), torch.int32, dev)
    if w is None and "w" in want:
        w = _new(fresh, (B, T, H, k), torch.float32, dev)
    _dev(o, "o", torch.float32, (B, T, dv))
    if vhat is not None: _dev(vhat, "vhat", torch.float32, (B, T, dv))
    if idx is not None: _dev(idx, "idx", torch.int32, (B, T, H, k))
    if w is not None: _dev(w, "w", torch.float32, (B, T, H, k))
    ws, wsb = _workspace(cfg, B, T, ws, dev, fresh)
    c = _cfg(cfg)
    _check(load().fwpkm_retrieve(ctypes.byref(c), B, T, _ptr(q), _ptr(v), _ptr(g), _ptr(K1), _ptr(K2), _ptr(V),
                                 _ptr(o), _ptr(vhat), _ptr(idx), _ptr(w), _ptr(ws), wsb, _stream(stream)))
    _mine(stream, fresh)
    return {"o": o, "vhat": vhat, "idx": idx, "w": w}


def fwpkm_retrieve_backward(cfg: FwpkmConfig, q, v, g, K1, K2, V, idx, w, dO, dq=None, dv=None, dg=None,
                            stream=None):
    """Gradient of fwpkm_retrieve's o w.r.t. q, v and g for upstream dO, the
    selection idx / w and the state held fixed.  Returns dict(dq, dv, dg)."""
    sd = cfg.torch_dtype
    B, T = g.shape
    H, dqd, dvd, k = cfg.heads, cfg.d_q, cfg.d_v, cfg.k
    dev = g.device
    _dev(q, "q", sd, (B, T, H, dqd)); _dev(v, "v", sd, (B, T, dvd)); _dev(g, "g", torch.float32, (B, T))
    _dev(K1, "K1", sd, (B, H, cfg.n, dqd // 2)); _dev(K2, "K2", sd, (B, H, cfg.n, dqd // 2))
    _dev(V, "V", sd, (B, cfg.N, dvd))
    _dev(idx, "idx", torch.int32, (B, T, H, k)); _dev(w, "w", torch.float32, (B, T, H, k))
    _dev(dO, "dO", torch.float32, (B, T, dvd))
    fresh = []
    dq = _new(fresh, (B, T, H, dqd), torch.float32, dev) if dq is None else dq
    dv = _new(fresh, (B, T, dvd), torch.float32, dev) if dv is None else dv
    dg = _new(fresh, (B, T), torch.float32, dev) if dg is None else dg
    _dev(dq, "dq", torch.float32, (B, T, H, dqd)); _dev(dv, "dv", torch.float32, (B, T, dvd))
    _dev(dg, "dg", torch.float32, (B, T))
    c = _cfg(cfg)
    _check(load().fwpkm_retrieve_backward(ctypes.byref(c), B, T, _ptr(q), _ptr(v), _ptr(g), _ptr(K1), _ptr(K2),
                                          _ptr(V), _ptr(idx), _ptr(w), _ptr(dO), _ptr(dq), _ptr(dv), _ptr(dg),
                                          _stream(stream)))
    _mine(stream, fresh)
    return {"dq": dq, "dv": dv, "dg": dg}


def fwpkm_chunk_update(cfg: FwpkmConfig, q, g, tgt, n_tgt: int, idx, w, vhat, K1, K2, V, n_read=None,
                       ws=None, stream=None):
    """One chunk's write; K1, K2, V are updated in place.  Returns n_read (or None)."""
    sd = cfg.torch_dtype
    B, Tc = g.shape
    H, dq, dv, k = cfg.heads, cfg.d_q, cfg.d_v, cfg.k
    _dev(q, "q", sd, (B, Tc, H, dq)); _dev(g, "g", torch.float32, (B, Tc))
    if n_tgt > 0:
        _dev(tgt, "tgt", sd, (B, n_tgt, dv))
    _dev(idx, "idx", torch.int32, (B, Tc, H, k)); _dev(w, "w", torch.float32, (B, Tc, H, k))
    _dev(vhat, "vhat", torch.float32, (B, Tc, dv))
    _dev(K1, "K1", sd, (B, H, cfg.n, dq // 2)); _dev(K2, "K2", sd, (B, H, cfg.n, dq // 2))
    _dev(V, "V", sd, (B, cfg.N, dv))
    if n_read is not None:
        _dev(n_read, "n_read", torch.int32, (B, cfg.N))
    fresh = []
    ws, wsb = _workspace(cfg, B, Tc, ws, g.device, fresh)
    c = _cfg(cfg)
    _check(load().fwpkm_chunk_update(ctypes.byref(c), B, Tc, int(n_tgt), _ptr(q), _ptr(g),
                                     _ptr(tgt) if n_tgt > 0 else None, _ptr(idx), _ptr(w), _ptr(vhat),
                                     _ptr(K1), _ptr(K2), _ptr(V), _ptr(n_read), _ptr(ws), wsb, _stream(stream)))
    _mine(stream, fresh)
    return n_read


def fwpkm_forward_seq(cfg: FwpkmConfig, q, v, g, K1, K2, V, passes: int = 1, v_next=None, o=None, vhat=None,
                      ws=None, stream=None, want_vhat: bool = False, usage=None):
    """Whole sequences, chunk-causal, `passes` times; K1, K2, V updated in place.
    With `usage` ([B, N] int32) the reads are also counted
    (fwpkm_forward_seq_usage).  Returns dict(o, vhat) of the last pass."""
    sd = cfg.torch_dtype
    B, T = g.shape
    H, dq, dv = cfg.heads, cfg.d_q, cfg.d_v
    dev = g.device
    _dev(q, "q", sd, (B, T, H, dq)); _dev(v, "v", sd, (B, T, dv)); _dev(g, "g", torch.float32, (B, T))
    if v_next is not None:
        _dev(v_next, "v_next", sd, (B, dv))
    _dev(K1, "K1", sd, (B, H, cfg.n, dq // 2)); _dev(K2, "K2", sd, (B, H, cfg.n, dq // 2))
    _dev(V, "V", sd, (B, cfg.N, dv))
    fresh = []
    o = _new(fresh, (B, T, dv), torch.float32, dev) if o is None else o
    _dev(o, "o", torch.float32, (B, T, dv))
    if vhat is None and want_vhat:
        vhat = _new(fresh, (B, T, dv), torch.float32, dev)
    if vhat is not None:
        _dev(vhat, "vhat", torch.float32, (B, T, dv))
    ws, wsb = _workspace(cfg, B, T, ws, dev, fresh)
    c = _cfg(cfg)
    if usage is None:
        _check(load().fwpkm_forward_seq(ctypes.byref(c), B, T, int(passes), _ptr(q), _ptr(v), _ptr(g),
                                        _ptr(v_next), _ptr(K1), _ptr(K2), _ptr(V), _ptr(o), _ptr(vhat), _ptr(ws),
                                        wsb, _stream(stream)))
    else:
        _dev(usage, "usage", torch.int32, (B, cfg.N))
        _check(load().fwpkm_forward_seq_usage(ctypes.byref(c), B, T, int(passes), _ptr(q), _ptr(v), _ptr(g),
                                              _ptr(v_next), _ptr(K1), _ptr(K2), _ptr(V), _ptr(o), _ptr(vhat),
                                              _ptr(usage), _ptr(ws), wsb, _stream(stream)))
    _mine(stream, fresh)
    return {"o": o, "vhat": vhat}


def fwpkm_forward_seq_static(cfg: FwpkmConfig, q, v, g, K1, K2, V, passes: int = 1, v_next=None, o=None,
                             vhat=None, stream=None, want_vhat: bool = False):
    """fwpkm_forward_seq with the library's static scratch in place of a
    workspace (the library allocates nothing; outputs not given are
    allocated here, by torch).  Returns dict(o, vhat) of the last pass."""
    sd = cfg.torch_dtype
    B, T = g.shape
    H, dq, dv = cfg.heads, cfg.d_q, cfg.d_v
    dev = g.device
    _dev(q, "q", sd, (B, T, H, dq)); _dev(v, "v", sd, (B, T, dv)); _dev(g, "g", torch.float32, (B, T))
    if v_next is not None:
        _dev(v_next, "v_next", sd, (B, dv))
    _dev(K1, "K1", sd, (B, H, cfg.n, dq // 2)); _dev(K2, "K2", sd, (B, H, cfg.n, dq // 2))
    _dev(V, "V", sd, (B, cfg.N, dv))
    fresh = []
    o = _new(fresh, (B, T, dv), torch.float32, dev) if o is None else o
    _dev(o, "o", torch.float32, (B, T, dv))
    if vhat is None and want_vhat:
        vhat = _new(fresh, (B, T, dv), torch.float32, dev)
    if vhat is not None:
        _dev(vhat, "vhat", torch.float32, (B, T, dv))
    c = _cfg(cfg)
    _check(load().fwpkm_forward_seq_static(ctypes.byref(c), B, T, int(passes), _ptr(q), _ptr(v), _ptr(g),
                                           _ptr(v_next), _ptr(K1), _ptr(K2), _ptr(V), _ptr(o), _ptr(vhat),
                                           _stream(stream)))
    _mine(stream, fresh)
    return {"o": o, "vhat": vhat}


def fwpkm_forward_seq_backward(cfg: FwpkmConfig, q, v, g, K1, K2, V, dO, passes: int = 1, v_next=None,
                               want_o: bool = False, ws=None, stream=None):
    """Gradients of forward_seq's o w.r.t. q, v, g by replay from the state
    forward_seq started with (K1, K2, V are rewritten as the forward did).
    Returns dict(dq, dv, dg, o)."""
    sd = cfg.torch_dtype
    B, T = g.shape
    H, dqd, dvd = cfg.heads, cfg.d_q, cfg.d_v
    dev = g.device
    _dev(q, "q", sd, (B, T, H, dqd)); _dev(v, "v", sd, (B, T, dvd)); _dev(g, "g", torch.float32, (B, T))
    if v_next is not None:
        _dev(v_next, "v_next", sd, (B, dvd))
    _dev(K1, "K1", sd, (B, H, cfg.n, dqd // 2)); _dev(K2, "K2", sd, (B, H, cfg.n, dqd // 2))
    _dev(V, "V", sd, (B, cfg.N, dvd))
    _dev(dO, "dO", torch.float32, (B, T, dvd))
    fresh = []
    dq = _new(fresh, (B, T, H, dqd), torch.float32, dev)
    dv = _new(fresh, (B, T, dvd), torch.float32, dev)
    dg = _new(fresh, (B, T), torch.float32, dev)
    o = _new(fresh, (B, T, dvd), torch.float32, dev) if want_o else None
    ws, wsb = _workspace(cfg, B, T, ws, dev, fresh)
    c = _cfg(cfg)
    _check(load().fwpkm_forward_seq_backward(ctypes.byref(c), B, T, int(passes), _ptr(q), _ptr(v), _ptr(g),
                                             _ptr(v_next), _ptr(K1), _ptr(K2), _ptr(V), _ptr(dO), _ptr(dq),
                                             _ptr(dv), _ptr(dg), _ptr(o), _ptr(ws), wsb, _stream(stream)))
    _mine(stream, fresh)
    return {"dq": dq, "dv": dv, "dg": dg, "o": o}


def fwpkm_usage_metrics(cfg: FwpkmConfig, usage, reset: bool = False, metrics=None, ws=None, stream=None):
    """Addressing metrics of the counted interval: [B, 4] float64 tensor of
    (coverage, collision, KLD, reads) per sequence; reset zeroes usage."""
    B = usage.shape[0]
    _dev(usage, "usage", torch.int32, (B, cfg.N))
    fresh = []
    if metrics is None:
        metrics = _new(fresh, (B, 4), torch.float64, usage.device)
    _dev(metrics, "metrics", torch.float64, (B, 4))
    if ws is None:
        ws = _new(fresh, (2048 * B,), torch.uint8, usage.device)
    c = _cfg(cfg)
    _check(load().fwpkm_usage_metrics(ctypes.byref(c), B, _ptr(usage), _ptr(metrics), 1 if reset else 0, _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)))
    _mine(stream, fresh)
    return metrics


@functools.lru_cache(maxsize=256)
def stream_state_bytes(cfg: FwpkmConfig, B: int) -> int:
    out = ctypes.c_size_t(0)
    c = _cfg(cfg)
    _check(load().fwpkm_stream_state_bytes(ctypes.byref(c), int(B), ctypes.byref(out)))
    return int(out.value)


def stream_state(cfg: FwpkmConfig, B: int, device) -> tuple:
    """A fresh (state, pos) pair for fwpkm_stream_step: device state of
    stream_state_bytes() bytes and a StreamPos with nothing pending."""
    state = torch.empty(max(stream_state_bytes(cfg, B), 256), dtype=torch.uint8, device=device)
    return state, StreamPos(0, 0)


def fwpkm_stream_step(cfg: FwpkmConfig, q, v, g, K1, K2, V, state, pos: StreamPos, o=None, vhat=None,
                      ws=None, stream=None, want_vhat: bool = False, usage=None):
    """T new tokens of a decode stream; K1, K2, V updated by the chunk writes
    the call triggers, pos advanced.  Returns dict(o, vhat)."""
    sd = cfg.torch_dtype
    B, T = g.shape
    H, dq, dv = cfg.heads, cfg.d_q, cfg.d_v
    dev = g.device
    _dev(q, "q", sd, (B, T, H, dq)); _dev(v, "v", sd, (B, T, dv)); _dev(g, "g", torch.float32, (B, T))
    _dev(K1, "K1", sd, (B, H, cfg.n, dq // 2)); _dev(K2, "K2", sd, (B, H, cfg.n, dq // 2))
    _dev(V, "V", sd, (B, cfg.N, dv))
    _dev(state, "state", torch.uint8, (state.numel(),))
    if state.numel() < stream_state_bytes(cfg, B):
        raise ValueError("state is smaller than stream_state_bytes()")
    fresh = []
    o = _new(fresh, (B, T, dv), torch.float32, dev) if o is None else o
    _dev(o, "o", torch.float32, (B, T, dv))
    if vhat is None and want_vhat:
        vhat = _new(fresh, (B, T, dv), torch.float32, dev)
    if vhat is not None:
        _dev(vhat, "vhat", torch.float32, (B, T, dv))
    if usage is not None:
        _dev(usage, "usage", torch.int32, (B, cfg.N))
    ws, wsb = _workspace(cfg, B, cfg.chunk, ws, dev, fresh)
    c = _cfg(cfg)
    _check(load().fwpkm_stream_step(ctypes.byref(c), B, T, _ptr(q), _ptr(v), _ptr(g), _ptr(K1), _ptr(K2), _ptr(V),
                                    _ptr(o), _ptr(vhat), _ptr(usage), _ptr(state), ctypes.byref(pos), _ptr(ws), wsb,
                                    _stream(stream)))
    _mine(stream, fresh)
    return {"o": o, "vhat": vhat}


def fwpkm_stream_flush(cfg: FwpkmConfig, K1, K2, V, state, pos: StreamPos, v_next=None, ws=None, stream=None):
    """End of the stream's sequences: writes the pending tokens."""
    sd = cfg.torch_dtype
    B = V.shape[0]
    H, dq, dv = cfg.heads, cfg.d_q, cfg.d_v
    _dev(K1, "K1", sd, (B, H, cfg.n, dq // 2)); _dev(K2, "K2", sd, (B, H, cfg.n, dq // 2))
    _dev(V, "V", sd, (B, cfg.N, dv))
    _dev(state, "state", torch.uint8, (state.numel(),))
    if v_next is not None:
        _dev(v_next, "v_next", sd, (B, dv))
    fresh = []
    ws, wsb = _workspace(cfg, B, cfg.chunk, ws, V.device, fresh)
    c = _cfg(cfg)
    _check(load().fwpkm_stream_flush(ctypes.byref(c), B, _ptr(v_next), _ptr(K1), _ptr(K2), _ptr(V), _ptr(state),
                                     ctypes.byref(pos), _ptr(ws), wsb, _stream(stream)))
    _mine(stream, fresh)
