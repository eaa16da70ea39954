"""Host-only checks of the C-ABI library (no GPU needed).

The library loads on a machine without a GPU; every call here returns from
argument validation before anything touches HIP.
"""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_weight_memory_sub_amd import fwpkm
from sparse_weight_memory_sub_amd.workloads import WORKLOADS, FwpkmConfig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fwpkm.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fwpkm.LIB_PATH), reason="libfwpkm.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fwpkm_[a-z_]+)\s*\(", src)))


def test_header_declares_exactly_the_exports():
    assert _declared() == sorted(fwpkm.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = fwpkm.load()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fwpkm.LIB_PATH], capture_output=True, text=True).stdout
    syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in _declared():
        assert name in syms, name


def test_abi_version_and_empty_error():
    assert fwpkm.abi_version() == 3
    assert fwpkm.load().fwpkm_last_error() is not None


GOOD = FwpkmConfig(n=64, heads=2, d_q=64, d_v=64, k_half=8, k=8, chunk=32)


def _rc(fn, *args):
    return getattr(fwpkm.load(), fn)(*args)


def _ws_rc(cfg, B=2, T=10):
    c = fwpkm.cfg_struct(cfg)
    out = ctypes.c_size_t(0)
    return _rc("fwpkm_workspace_bytes", ctypes.byref(c), B, T, ctypes.byref(out)), out.value


@pytest.mark.parametrize("change,code", [
    (dict(n=0), fwpkm.EINVAL),
    (dict(n=46341), fwpkm.EINVAL),          # n*n overflows int32
    (dict(d_q=63), fwpkm.EINVAL),           # odd
    (dict(k_half=65), fwpkm.EINVAL),        # k' > n
    (dict(k=65), fwpkm.EINVAL),             # k > k'^2
    (dict(heads=0), fwpkm.EINVAL),
    (dict(chunk=0), fwpkm.EINVAL),
    (dict(idw_eps=0.0), fwpkm.EINVAL),
    (dict(idw_eps=float("nan")), fwpkm.EINVAL),
    (dict(lr_v=float("inf")), fwpkm.EINVAL),
    (dict(store="bf16"), fwpkm.OK),
    (dict(n=48), fwpkm.OK),
    (dict(n=40), fwpkm.EUNSUPPORTED),       # n % 16
    (dict(n=2048, k_half=8), fwpkm.EUNSUPPORTED),
    (dict(d_q=96), fwpkm.EUNSUPPORTED),     # d_q/2 = 48
    (dict(d_v=96), fwpkm.EUNSUPPORTED),
    (dict(k_half=64, k=64), fwpkm.EUNSUPPORTED),  # 280 product candidates
    (dict(k_half=48, k=48), fwpkm.OK),
])
def test_config_validation(change, code):
    rc, _ = _ws_rc(GOOD.replace(**change))
    assert rc == code, fwpkm.load().fwpkm_last_error()
    if code != fwpkm.OK:
        assert fwpkm.load().fwpkm_last_error().decode()


def test_workspace_bytes_sizes():
    rc, z = _ws_rc(GOOD, B=0, T=10)
    assert rc == 0 and z == 0
    rc, a = _ws_rc(GOOD, B=2, T=10)
    rc2, b = _ws_rc(GOOD, B=2, T=100)
    rc3, c = _ws_rc(GOOD, B=4, T=100)
    assert rc == rc2 == rc3 == 0
    assert 0 < a < b < c
    assert a % 256 == 0
    for name, wl in WORKLOADS.items():
        rc, nb = _ws_rc(wl.cfg, B=wl.B, T=wl.T)
        assert rc == 0, (name, fwpkm.load().fwpkm_last_error())
        assert nb < (1 << 34), name   # a few GiB at most


def _null():
    return ctypes.c_void_p(0)


def test_entry_points_reject_before_launch():
    c = fwpkm.cfg_struct(GOOD)
    N = ctypes.c_void_p
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    # missing required pointers
    rc = _rc("fwpkm_retrieve", ctypes.byref(c), 1, 4, None, fake, fake, fake, fake, fake, fake, None, None, None,
             fake, 1 << 30, None)
    assert rc == fwpkm.EINVAL
    # workspace too small / NULL / misaligned
    rc = _rc("fwpkm_retrieve", ctypes.byref(c), 1, 4, fake, fake, fake, fake, fake, fake, fake, None, None, None,
             fake, 16, None)
    assert rc == fwpkm.EWORKSPACE
    rc = _rc("fwpkm_retrieve", ctypes.byref(c), 1, 4, fake, fake, fake, fake, fake, fake, fake, None, None, None,
             None, 1 << 30, None)
    assert rc == fwpkm.EWORKSPACE
    rc = _rc("fwpkm_retrieve", ctypes.byref(c), 1, 4, fake, fake, fake, fake, fake, fake, fake, None, None, None,
             ctypes.c_void_p(0x1010), 1 << 30, None)
    assert rc == fwpkm.EWORKSPACE
    # bad sizes
    rc = _rc("fwpkm_retrieve", ctypes.byref(c), -1, 4, fake, fake, fake, fake, fake, fake, fake, None, None, None,
             fake, 1 << 30, None)
    assert rc == fwpkm.EINVAL
    rc = _rc("fwpkm_chunk_update", ctypes.byref(c), 1, 4, 5, fake, fake, fake, fake, fake, fake, fake, fake, fake,
             None, fake, 1 << 30, None)
    assert rc == fwpkm.EINVAL  # n_tgt > Tc
    rc = _rc("fwpkm_chunk_update", ctypes.byref(c), 1, 4, 2, fake, fake, None, fake, fake, fake, fake, fake, fake,
             None, fake, 1 << 30, None)
    assert rc == fwpkm.EINVAL  # tgt missing
    rc = _rc("fwpkm_forward_seq", ctypes.byref(c), 1, 4, 0, fake, fake, fake, None, fake, fake, fake, fake, None,
             fake, 1 << 30, None)
    assert rc == fwpkm.EINVAL  # passes = 0
    rc = _rc("fwpkm_forward_seq", ctypes.byref(c), 1, 4, 1, fake, fake, fake, None, fake, fake, fake, None, None,
             fake, 1 << 30, None)
    assert rc == fwpkm.EINVAL  # o missing
    # NULL cfg
    rc = _rc("fwpkm_forward_seq", None, 1, 4, 1, fake, fake, fake, None, fake, fake, fake, fake, None,
             fake, 1 << 30, None)
    assert rc == fwpkm.EINVAL
    assert "cfg" in fwpkm.load().fwpkm_last_error().decode()


def test_empty_calls_are_noops():
    c = fwpkm.cfg_struct(GOOD)
    for B, T in ((0, 5), (3, 0)):
        assert _rc("fwpkm_retrieve", ctypes.byref(c), B, T, None, None, None, None, None, None, None, None, None,
                   None, None, 0, None) == fwpkm.OK
        assert _rc("fwpkm_chunk_update", ctypes.byref(c), B, T, 0, None, None, None, None, None, None, None, None,
                   None, None, None, 0, None) == fwpkm.OK
        assert _rc("fwpkm_forward_seq", ctypes.byref(c), B, T, 1, None, None, None, None, None, None, None, None,
                   None, None, 0, None) == fwpkm.OK


def test_stream_state_bytes_cover_the_pending_chunk():
    c = fwpkm.cfg_struct(GOOD)
    out = ctypes.c_size_t(0)
    assert _rc("fwpkm_stream_state_bytes", ctypes.byref(c), 3, ctypes.byref(out)) == fwpkm.OK
    B, C, H, n, dq, dv, k = 3, GOOD.chunk, GOOD.heads, GOOD.n, GOOD.d_q, GOOD.d_v, GOOD.k
    es = 4  # f32 storage
    # norms, then q, g, targets, slot ids, weights and vhat of C tokens per sequence
    floor = B * H * 2 * n * 4 + B * C * (H * dq * es + 4 + dv * es + 2 * H * k * 4 + dv * 4)
    assert floor <= out.value <= floor + 7 * 256
    assert _rc("fwpkm_stream_state_bytes", ctypes.byref(c), 0, ctypes.byref(out)) == fwpkm.OK
    assert out.value == 0
    assert _rc("fwpkm_stream_state_bytes", ctypes.byref(c), -1, ctypes.byref(out)) == fwpkm.EINVAL


def test_stream_entry_points_reject_before_launch():
    c = fwpkm.cfg_struct(GOOD)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    pos = fwpkm.StreamPos(0, 0)

    def step(B, T, q, o, state, p, ws, wsb):
        return _rc("fwpkm_stream_step", ctypes.byref(c), B, T, q, fake, fake, fake, fake, fake, o, None, None,
                   state, p, ws, wsb, None)

    assert step(1, 1, fake, fake, fake, None, fake, 1 << 30) == fwpkm.EINVAL          # pos NULL
    assert step(1, 1, None, fake, fake, ctypes.byref(pos), fake, 1 << 30) == fwpkm.EINVAL  # q missing
    assert step(1, 1, fake, None, fake, ctypes.byref(pos), fake, 1 << 30) == fwpkm.EINVAL  # o missing
    assert step(1, 1, fake, fake, None, ctypes.byref(pos), fake, 1 << 30) == fwpkm.EINVAL  # state missing
    assert step(1, 1, fake, fake, ctypes.c_void_p(0x1010), ctypes.byref(pos), fake, 1 << 30) == fwpkm.EINVAL
    assert step(1, 1, fake, fake, fake, ctypes.byref(pos), fake, 16) == fwpkm.EWORKSPACE
    assert step(1, -1, fake, fake, fake, ctypes.byref(pos), fake, 1 << 30) == fwpkm.EINVAL
    for bad in (-1, GOOD.chunk + 1):
        p = fwpkm.StreamPos(bad, 0)
        assert step(1, 1, fake, fake, fake, ctypes.byref(p), fake, 1 << 30) == fwpkm.EINVAL
        assert "pending" in fwpkm.load().fwpkm_last_error().decode()
    # empty calls are no-ops and leave the position alone
    p = fwpkm.StreamPos(5, 0)
    assert step(0, 1, None, None, None, ctypes.byref(p), None, 0) == fwpkm.OK
    assert step(2, 0, None, None, None, ctypes.byref(p), None, 0) == fwpkm.OK
    assert (p.pending, p.norms_valid) == (5, 0)
    # a flush with nothing pending launches nothing
    p = fwpkm.StreamPos(0, 0)
    assert _rc("fwpkm_stream_flush", ctypes.byref(c), 2, None, None, None, None, fake, ctypes.byref(p), None, 0,
               None) == fwpkm.OK
    p = fwpkm.StreamPos(3, 0)
    assert _rc("fwpkm_stream_flush", ctypes.byref(c), 2, None, None, fake, fake, fake, ctypes.byref(p), fake,
               1 << 30, None) == fwpkm.EINVAL  # K1 missing
    assert p.pending == 3


def test_usage_entry_points_reject_before_launch():
    c = fwpkm.cfg_struct(GOOD)
    fake = ctypes.c_void_p(0x1000)
    assert _rc("fwpkm_usage_metrics", ctypes.byref(c), 2, None, fake, 1, fake, 4096, None) == fwpkm.EINVAL
    assert _rc("fwpkm_usage_metrics", ctypes.byref(c), 2, fake, None, 0, fake, 4096, None) == fwpkm.EINVAL
    assert _rc("fwpkm_usage_metrics", ctypes.byref(c), -1, fake, fake, 0, fake, 4096, None) == fwpkm.EINVAL
    assert _rc("fwpkm_usage_metrics", ctypes.byref(c), 2, fake, fake, 0, fake, 4095, None) == fwpkm.EWORKSPACE
    assert _rc("fwpkm_usage_metrics", ctypes.byref(c), 0, None, None, 0, None, 0, None) == fwpkm.OK
    # forward_seq_usage validates like forward_seq (o missing)
    assert _rc("fwpkm_forward_seq_usage", ctypes.byref(c), 1, 4, 1, fake, fake, fake, None, fake, fake, fake, None,
               None, fake, fake, 1 << 30, None) == fwpkm.EINVAL


def test_retrieve_backward_rejects_before_launch():
    c = fwpkm.cfg_struct(GOOD)
    fake = ctypes.c_void_p(0x1000)
    args = [fake] * 12
    assert _rc("fwpkm_retrieve_backward", ctypes.byref(c), 1, 4, *args[:11], None, None) == fwpkm.EINVAL  # dg missing
    assert _rc("fwpkm_retrieve_backward", ctypes.byref(c), -1, 4, *args, None) == fwpkm.EINVAL
    assert _rc("fwpkm_retrieve_backward", ctypes.byref(c), 0, 4, *([None] * 12), None) == fwpkm.OK


def test_forward_seq_backward_rejects_before_launch():
    c = fwpkm.cfg_struct(GOOD)
    fake = ctypes.c_void_p(0x1000)
    # dq missing
    assert _rc("fwpkm_forward_seq_backward", ctypes.byref(c), 1, 4, 1, fake, fake, fake, None, fake, fake, fake,
               fake, None, fake, fake, None, fake, 1 << 30, None) == fwpkm.EINVAL
    assert _rc("fwpkm_forward_seq_backward", ctypes.byref(c), 1, 4, 0, fake, fake, fake, None, fake, fake, fake,
               fake, fake, fake, fake, None, fake, 1 << 30, None) == fwpkm.EINVAL  # passes = 0


def _raw_ws(cfg, B, T):
    c = fwpkm.cfg_struct(cfg)
    out = ctypes.c_size_t(0)
    assert _rc("fwpkm_workspace_bytes", ctypes.byref(c), B, T, ctypes.byref(out)) == fwpkm.OK
    return out.value


def test_debug_overrides_need_the_debug_switch(monkeypatch):
    """FWPKM_SCORE_PATH=rows sizes the workspace for whole rows of distances,
    but only while FWPKM_DEBUG is "1"."""
    cfg = FwpkmConfig(n=256, heads=4, d_q=128, d_v=64, k_half=16, k=16, chunk=256)
    B, T = 8, 1024
    monkeypatch.delenv("FWPKM_SCORE_PATH", raising=False)
    monkeypatch.setenv("FWPKM_DEBUG", "1")
    base = _raw_ws(cfg, B, T)
    monkeypatch.setenv("FWPKM_SCORE_PATH", "rows")
    assert _raw_ws(cfg, B, T) > base
    monkeypatch.setenv("FWPKM_DEBUG", "0")
    assert _raw_ws(cfg, B, T) == base
    monkeypatch.delenv("FWPKM_DEBUG")
    assert _raw_ws(cfg, B, T) == base


def test_release_streams_with_nothing_to_release():
    assert _rc("fwpkm_release_streams") == fwpkm.OK
    assert _rc("fwpkm_release_streams") == fwpkm.OK


def test_static_scratch_refuses_calls_beyond_it():
    """fwpkm_forward_seq_static returns FWPKM_EWORKSPACE, before touching the
    GPU, for a call needing more than FWPKM_STATIC_SCRATCH_BYTES."""
    wl = WORKLOADS["million"]
    c = fwpkm.cfg_struct(wl.cfg)
    P = ctypes.c_void_p(256)
    rc = _rc("fwpkm_forward_seq_static", ctypes.byref(c), 2 * wl.B, wl.T, 1, P, P, P, None, P, P, P, P, None, None)
    assert rc == fwpkm.EWORKSPACE
    msg = fwpkm.load().fwpkm_last_error().decode()
    assert "static scratch holds 536870912" in msg, msg
