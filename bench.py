"""Benchmark of the FwPKM layer hot path on one MI355X.

A step is one fwpkm_forward_seq over one batch of the workload: every chunk
of every sequence read (scoring, top-k, gather, gated output) and then
written (value rows and sub-key codebooks), in causal order.  Inputs are
seeded synthetic data already resident in HBM; the fast-weight state carries
over from step to step, as it does across sequences of a stream.

Prints one JSON line: tokens/s of the whole job, the roofline of the
dominant kernel (its algorithmic bytes or flops per launch over its average
launch time, measured with HIP events on the library's stream), and the CPU
oracle timed on a bounded sample of the same workload.

    python bench.py [--workload million] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FwPKM layer tokens/s (retrieve+chunk update) on one GPU; gather/scatter HBM GB/s"
HBM_PEAK_GBS = 8000.0                 # MI355X HBM3E, GB/s
MFMA_PEAK_TFS = {"bf16": 2500.0, "f32": 157.3}  # dense MFMA, TFLOP/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="million", choices=("million", "mid", "collision", "long", "tiny"),
                    help="workload shape (default: the million-slot layer)")
    ap.add_argument("--passes", type=int, default=None, help="passes over each sequence (default: the workload's)")
    ap.add_argument("--cpu-seqs", type=int, default=None, help="sequences of the oracle sample (default 5)")
    ap.add_argument("--cpu-chunks", type=int, default=None, help="chunks per sequence of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-only", action="store_true",
                    help="only the timed steps (for profilers): no kernel timing pass, no CPU baseline")
    ap.add_argument("--decode", action="store_true",
                    help="time streaming decode (one token per call per sequence) instead of forward_seq")
    ap.add_argument("--decode-tokens", type=int, default=1024, help="timed decode tokens per sequence")
    ap.add_argument("--score", choices=("idw", "dot"), default=None,
                    help="sub-key scoring variant (default: the workload's, IDW)")
    ap.add_argument("--no-gate-weight", action="store_true",
                    help="memorisation error without the gate weighting (an ablation)")
    ap.add_argument("--backward", action="store_true",
                    help="time fwpkm_forward_seq_backward (replayed pass with gradients w.r.t. q, v, g)")
    ap.add_argument("--usage", action="store_true",
                    help="time forward_seq with row-contribution counting and the addressing metrics")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print per-kernel tables of a rocprofv3 --kernel-trace CSV output directory and exit")
    ap.add_argument("--last-call", action="store_true",
                    help="with --summarize-trace: only the last forward_seq call of the trace (from its sub-key "
                         "norms on), with each stream's gaps and the chunk period")
    ap.add_argument("--decode-calls", nargs=2, type=int, metavar=("FIRST", "COUNT"),
                    help="with --summarize-trace: the library's kernels of decode calls FIRST .. FIRST+COUNT-1 "
                         "(calls counted by their scoring launches), per call")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="HBM bytes per kernel from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE CSV output directories "
                         "of a --profile-only run with one kernel at a time; writes profiles/<family>_<workload>_pmc.json "
                         "and prints a table")
    ap.add_argument("--summarize-mfma", metavar="DIR",
                    help="MFMA work and busy fraction per scoring, row-statistic and key-step kernel from a rocprofv3 "
                         "--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F32 "
                         "GRBM_GUI_ACTIVE CSV output directory; prints a table")
    ap.add_argument("--prequeue", action="store_true",
                    help="also time one step queued whole behind a sleep kernel before the GPU starts it "
                         "(the device-side time, without the host's enqueue pace)")
    ap.add_argument("--ceiling", action="store_true",
                    help="measure the HBM rates of random 1 KiB value rows (read; read-modify-write at several "
                         "depths, from registers and staged in LDS) and of a sequential copy")
    return ap.parse_args()


def algorithmic(cfg, B, Tc, n_tgt, U, passes_write_o=True):
    """Algorithmic bytes / flops of one launch of each kernel family for one
    chunk step of B sequences (Tc tokens, n_tgt with targets, U unique rows
    written per sequence)."""
    es = 2 if cfg.store == "bf16" else 4
    H, k, dv, n, dh = cfg.heads, cfg.k, cfg.d_v, cfg.n, cfg.d_h
    tok = B * Tc
    M = B * n_tgt * H * k
    gather = tok * (H * k * dv * es      # selected value rows
                    + H * k * 8          # slot ids and weights
                    + dv * es + 4        # residual-path value and gate
                    + dv * es            # lookahead target
                    + 4 * dv             # residual r written
                    + (4 * dv if passes_write_o else 0))  # o written
    scatter = (B * U * dv * es * 2       # read-modify-write of each written row
               + B * n_tgt * dv * 4      # residual rows (read once)
               + M * 12)                 # sorted slot, entry, weight per read
    score_flops = 2.0 * tok * H * 2 * n * dh        # q.K for both halves
    kgrad_flops = 2.0 * 2 * B * H * 2 * n * Tc * dh  # distance recompute + a^T q
    return {"gather": gather, "scatter": scatter, "score_select": score_flops,
            "score_rowstat": score_flops, "kgrad": kgrad_flops}


def layer_bytes_per_token(cfg, U):
    """Algorithmic HBM bytes per token of the whole layer step (retrieval and
    chunk write), with U unique value rows written per chunk and sequence:
    the compulsory traffic the roofline of the layer's tokens/s is priced on."""
    es = 2 if cfg.store == "bf16" else 4
    H, k, dv, dq, n, C = cfg.heads, cfg.k, cfg.d_v, cfg.d_q, cfg.n, cfg.chunk
    retrieve = (H * k * dv * es          # selected value rows
                + H * dq * es            # q
                + dv * es + 4            # v and the gate
                + 4 * dv + 4 * dv        # o, and v_hat / residual
                + 8 * H * k              # slot ids and weights
                + H * n * dq * es / C)   # both codebooks, read once per chunk
    update = (4 * dv + dv * es           # residual and target in
              + 2 * U * dv * es / C      # read-modify-write of the written rows
              + 16 * H * k               # sorted read list
              + H * dq * es              # q again for the key step
              + 2 * H * n * dq * es / C) # codebooks read and written
    return retrieve + update


def src_hash(*names):
    h = hashlib.sha256()
    for nm in names:
        with open(os.path.join(ROOT, "sparse_weight_memory_sub_amd", "csrc", nm), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SRC = {"gather": ("k_gather.hip", "gather.h", "rows.h", "fwpkm_internal.h"),
              "scatter": ("k_scatter.hip", "fwpkm_internal.h"),
              "score_select": ("k_score.hip", "mfma_frag.h", "fwpkm_internal.h"),
              "score_rowstat": ("k_score.hip", "mfma_frag.h", "fwpkm_internal.h"),
              "kgrad": ("k_addr.hip", "mfma_frag.h", "fwpkm_internal.h")}


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter summaries, when
    they were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path) or kernel not in KERNEL_SRC:
        return None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    if d.get("src_hash") != src_hash(*KERNEL_SRC[kernel]):
        return None
    return d.get("hbm_bytes_per_launch")


def decode_bench(args, cfg, wl, B, q, v, g, K1, K2, V):
    """Streaming decode: every call reads one new token of each of the B
    sequences (fwpkm_stream_step with T = 1); a chunk write fires every C
    tokens.  Prints one JSON line."""
    import torch
    from sparse_weight_memory_sub_amd import fwpkm

    dev = q.device
    stream = torch.cuda.current_stream()
    st, pos = fwpkm.stream_state(cfg, B, dev)
    ws = torch.empty(fwpkm.workspace_bytes(cfg, B, cfg.chunk), dtype=torch.uint8, device=dev)
    T = q.shape[1]
    o = torch.empty((B, 1, cfg.d_v), dtype=torch.float32, device=dev)
    cursor = [0]

    # per-token inputs made contiguous once, outside the timed region
    q = torch.stack([q[:, t:t + 1].contiguous() for t in range(T)])  # [T][B][1][H][d_q]
    v = torch.stack([v[:, t:t + 1].contiguous() for t in range(T)])
    g = torch.stack([g[:, t:t + 1].contiguous() for t in range(T)])

    def tokens(n):
        for _ in range(n):
            t = cursor[0] % T
            cursor[0] += 1
            fwpkm.fwpkm_stream_step(cfg, q[t], v[t], g[t], K1, K2, V, st, pos, o=o, ws=ws, stream=stream)

    tokens(args.warmup * cfg.chunk // 4 + 1)
    torch.cuda.synchronize()
    K = args.decode_tokens

    def timed(events):
        fwpkm.timing_enable(events)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        start.record(stream)
        tokens(K)
        stop.record(stream)
        enq = time.perf_counter() - h0
        torch.cuda.synchronize()
        wall = time.perf_counter() - h0
        fwpkm.timing_enable(False)
        return start.elapsed_time(stop), wall * 1e3, enq * 1e3

    ms, wall_ms, enq_ms = timed(False)
    value = B * K / (ms / 1e3)
    log(f"decode: {K} tokens x {B} sequences in {ms:.2f} ms ({ms / K * 1e3:.1f} us per call), "
        f"{value:.4g} tokens/s; host wall {wall_ms:.2f} ms, of which enqueueing {enq_ms:.2f} ms")
    ms_ev, _, _ = timed(True)
    tk = fwpkm.timing_read()
    es = 2 if cfg.store == "bf16" else 4
    # algorithmic bytes of one read call: both codebooks once, the selected
    # value rows, the token's q, v and the output row
    kbytes = B * cfg.heads * 2 * cfg.n * cfg.d_h * es
    gbytes = B * (cfg.heads * cfg.k * (cfg.d_v * es + 8) + cfg.d_v * (es + 8) + 4)
    kernels = {}
    for name, (t_ms, n) in tk.items():
        if n:
            kernels[name] = {"avg_ms": t_ms / n, "launches": n, "per_call_ms": t_ms / K}
    sel = kernels.get("score_select")
    roof = None
    if sel:
        ach = kbytes / (sel["avg_ms"] / 1e3) / 1e9
        roof = {"kernel": "score_select", "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "traffic": None, "bytes_per_launch": kbytes,
                "avg_launch_ms": sel["avg_ms"]}
    result = {
        "metric": "FwPKM streaming decode tokens/s (one token per call per sequence, chunk writes included)",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.store, "data": "synthetic",
        "config": {"workload": f"{wl.name}-decode", "n_slots": cfg.N, "heads": cfg.heads, "d_q": cfg.d_q,
                   "d_v": cfg.d_v, "k_half": cfg.k_half, "k": cfg.k, "chunk": cfg.chunk, "batch": B,
                   "tokens_per_call": 1, "storage": cfg.store},
        "host_wall_ms_per_step": wall_ms / K,
        "host_enqueue_ms_per_step": enq_ms / K,
        "ms_per_step_with_kernel_events": ms_ev / K,
        "read_call_algorithmic_bytes": kbytes + gbytes,
        "roofline": roof, "kernels": kernels,
    }
    print(json.dumps(result), flush=True)


def usage_bench(args, cfg, wl, B, T, q, v, g, K1, K2, V):
    """forward_seq with row-contribution counts, and the addressing metrics
    every 32K tokens of each sequence (paperlayer.ai D.3).  Prints one JSON
    line."""
    import torch
    from sparse_weight_memory_sub_amd import fwpkm

    dev = q.device
    stream = torch.cuda.current_stream()
    o = torch.empty((B, T, cfg.d_v), dtype=torch.float32, device=dev)
    ws = torch.empty(fwpkm.workspace_bytes(cfg, B, T), dtype=torch.uint8, device=dev)
    usage = torch.zeros((B, cfg.N), dtype=torch.int32, device=dev)
    metrics = torch.empty((B, 4), dtype=torch.float64, device=dev)
    mws = torch.empty(2048 * B, dtype=torch.uint8, device=dev)
    interval = max(1, 32768 // T)  # steps per 32K tokens of a sequence

    def run(n, count):
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(n):
            fwpkm.fwpkm_forward_seq(cfg, q, v, g, K1, K2, V, o=o, ws=ws, stream=stream,
                                    usage=usage if count else None)
            if count and (i + 1) % interval == 0:
                fwpkm.fwpkm_usage_metrics(cfg, usage, reset=True, metrics=metrics, ws=mws, stream=stream)
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / n

    run(args.warmup, True)
    usage.zero_()
    steps = max(args.steps, interval)
    ms_plain = run(steps, False)
    ms_count = run(steps, True)
    usage.zero_()  # the timing pass below is exactly one interval
    fwpkm.timing_enable(True)
    run(interval, True)
    fwpkm.timing_enable(False)
    ms_u, n_u = fwpkm.timing_read()["usage"]
    m = metrics.cpu().numpy()
    value = B * T / (ms_count / 1e3)
    log(f"usage counting: {ms_count:.3f} ms/step against {ms_plain:.3f} without; metrics every {interval} steps")
    result = {
        "metric": "FwPKM layer tokens/s with row-contribution counting and addressing metrics every 32K tokens",
        "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": ms_count, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.store, "data": "synthetic",
        "config": {"workload": f"{wl.name}-usage", "n_slots": cfg.N, "heads": cfg.heads, "k": cfg.k,
                   "batch": B, "seq_len": T, "interval_tokens": interval * T},
        "ms_per_step_without_counting": ms_plain,
        "usage_kernels_ms_per_step": ms_u / interval,
        "usage_launches_per_step": n_u / interval,
        "metrics_mean": {"coverage": float(m[:, 0].mean()), "collision": float(m[:, 1].mean()),
                         "kld": float(m[:, 2].mean()), "reads": float(m[:, 3].mean())},
    }
    print(json.dumps(result), flush=True)


def backward_bench(args, cfg, wl, B, T, q, v, g, K1, K2, V):
    """fwpkm_forward_seq_backward: the pass replayed with each chunk's gradient
    of o w.r.t. q, v and g.  Prints one JSON line."""
    import torch
    from sparse_weight_memory_sub_amd import fwpkm

    dev = q.device
    stream = torch.cuda.current_stream()
    ws = torch.empty(fwpkm.workspace_bytes(cfg, B, T), dtype=torch.uint8, device=dev)
    dO = torch.randn((B, T, cfg.d_v), generator=torch.Generator().manual_seed(7)).to(dev)

    def step():
        fwpkm.fwpkm_forward_seq_backward(cfg, q, v, g, K1, K2, V, dO, ws=ws, stream=stream)

    for _ in range(args.warmup):
        step()

    def timed(events):
        fwpkm.timing_enable(events)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        fwpkm.timing_enable(False)
        return start.elapsed_time(stop) / args.steps

    ms = timed(False)
    ms_ev = timed(True)
    tk = fwpkm.timing_read()
    es = 2 if cfg.store == "bf16" else 4
    H, k, dv, dq, dh = cfg.heads, cfg.k, cfg.d_v, cfg.d_q, cfg.d_h
    per_tok = (H * k * (dv * es + 8)          # selected value rows, slot ids and weights
               + H * dq * es + dv * es + 4    # q, v, g
               + 4 * dv                       # dO
               + 4 * H * dq + 4 * dv + 4)     # dq, dv, dg written
    Tc = min(cfg.chunk, T)
    bwt, bwn = tk["backward"]
    avg = bwt / bwn
    # plus the codebooks once per launch (the selected sub-key rows are reread from L2)
    nbytes = B * Tc * per_tok + B * H * 2 * cfg.n * dh * es
    ach = nbytes / (avg / 1e3) / 1e9
    kernels = {name: {"avg_ms": t / n, "launches": n} for name, (t, n) in tk.items() if n}
    log(f"forward_seq_backward: {ms:.3f} ms/step; backward kernel {avg * 1e3:.1f} us per chunk, {ach:.0f} GB/s")
    result = {
        "metric": "FwPKM replayed pass with gradients w.r.t. q, v, g: tokens/s",
        "value": B * T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.store, "data": "synthetic",
        "config": {"workload": f"{wl.name}-backward", "n_slots": cfg.N, "heads": H, "d_q": dq, "d_v": dv,
                   "k": k, "chunk": cfg.chunk, "batch": B, "seq_len": T},
        "ms_per_step_with_kernel_events": ms_ev,
        "roofline": {"kernel": "backward", "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ach / HBM_PEAK_GBS, "traffic": None, "bytes_per_launch": nbytes,
                     "avg_launch_ms": avg},
        "kernels": kernels,
    }
    print(json.dumps(result), flush=True)


def ceiling_bench(args):
    """Rates HBM sustains for the value rows' access patterns: 16 sequences'
    value tables of 2^20 rows of 1 KiB (16 GiB), with 62080 distinct random
    rows per table, the rows the 2^20-slot layer writes per chunk (about a
    GB).  Sorted: each table's rows in ascending order, 64 consecutive rows
    per wavefront (the value write's order); shuffled: the same rows in
    random order (the gather's).  Prints one JSON line."""
    import ctypes

    import torch

    path = os.path.join(ROOT, "sparse_weight_memory_sub_amd", "probe", "libfwpkm_probe.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is missing: build it with `python -m sparse_weight_memory_sub_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32 = ctypes.c_void_p, ctypes.c_int
    lib.fwpkm_probe_rows.argtypes = [i32, i32, P, i32, i32, P, P, P, i32, ctypes.POINTER(i32)]
    lib.fwpkm_probe_copy.argtypes = [P, P, ctypes.c_size_t, P]
    dev = torch.device("cuda:0")
    seqs, rows_per, U, per = 16, 1 << 20, 62080, 64
    base = torch.empty(seqs * rows_per * 1024, dtype=torch.uint8, device=dev)
    gen = torch.Generator().manual_seed(11)
    sorted_rows = torch.cat([torch.randperm(rows_per, generator=gen)[:U].sort().values + s * rows_per
                             for s in range(seqs)]).to(torch.int32)
    shuffled = sorted_rows[torch.randperm(sorted_rows.numel(), generator=gen)]
    nrows = sorted_rows.numel()
    assert int(sorted_rows.max()) < base.numel() // 1024 and int(sorted_rows.min()) >= 0
    lists = {"sorted": sorted_rows.to(dev), "shuffled": shuffled.to(dev)}
    waves = (nrows + per - 1) // per
    out = torch.empty(waves * 64, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(fn, reps=5):
        for _ in range(2):
            fn()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(reps):
            fn()
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / reps

    def rows_fn(mode, R, lst):
        def f():
            rc = lib.fwpkm_probe_rows(mode, R, ctypes.c_void_p(lst.data_ptr()), nrows, per,
                                      ctypes.c_void_p(base.data_ptr()), ctypes.c_void_p(out.data_ptr()), sp, 0,
                                      None)
            if rc != 0:
                raise RuntimeError(f"probe launch failed: hip error {rc}")
        return f

    names = {0: "read", 1: "rmw", 2: "rmw-pipelined", 3: "rmw-lds"}
    depths = {0: (1, 2, 4, 8, 16), 1: (1, 2, 4, 8, 16), 2: (1, 2, 4, 8), 3: (4, 8, 16, 32)}
    table = []
    for order in ("sorted", "shuffled"):
        for mode in (0, 1, 2, 3):
            for R in depths[mode]:
                regs = ctypes.c_int(0)
                lib.fwpkm_probe_rows(mode, R, None, 0, per, None, None, None, 1, ctypes.byref(regs))
                ms = timed(rows_fn(mode, R, lists[order]))
                nbytes = nrows * 1024 * (1 if mode == 0 else 2)
                gbs = nbytes / (ms / 1e3) / 1e9
                table.append({"order": order, "pattern": names[mode], "rows_in_flight": R, "vgprs": regs.value,
                              "ms": ms, "GB/s": gbs})
                log(f"{order:8s} {names[mode]:14s} R={R:2d} vgprs={regs.value:3d}: {ms * 1e3:7.1f} us, {gbs:7.1f} GB/s")
    half = 1 << 30

    def copy():
        rc = lib.fwpkm_probe_copy(ctypes.c_void_p(base.data_ptr()), ctypes.c_void_p(base.data_ptr() + half), half, sp)
        if rc != 0:
            raise RuntimeError(f"copy launch failed: hip error {rc}")

    ms = timed(copy)
    copy_gbs = 2 * half / (ms / 1e3) / 1e9
    log(f"sequential copy of 1 GiB: {ms * 1e3:.1f} us, {copy_gbs:.1f} GB/s (read + write)")
    best = {}
    for r in table:
        key = (r["order"], "read" if r["pattern"] == "read" else "rmw")
        if key not in best or r["GB/s"] > best[key]["GB/s"]:
            best[key] = r
    result = {"metric": "HBM GB/s of random 1 KiB value rows (ceilings of the value-row kernels)",
              "value": best[("sorted", "rmw")]["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": 5, "warmup": 2,
              "higher_is_better": True, "data": "synthetic",
              "config": {"workload": "value-row-ceiling", "tables": seqs, "rows_per_table": rows_per,
                         "row_bytes": 1024, "rows_touched_per_table": U, "rows_per_wavefront": per,
                         "footprint_bytes": base.numel()},
              "sequential_copy_GBs": copy_gbs,
              "best": {f"{k[0]}-{k[1]}": v for k, v in best.items()}, "table": table}
    print(json.dumps(result), flush=True)


# kernel families of the library's timing (fwpkm_timing_read), by kernel name
def kernel_family(name):
    import re
    n = name.replace("(anonymous namespace)", "").split("(")[0]
    if "k_scatter" in n or "k_fixup" in n:
        return "scatter"
    if "k_gather" in n:
        return "gather"
    if "k_sort_" in n:
        return "sort"
    m = re.search(r"k_score<\s*\d+\s*,\s*\d+\s*,\s*\d+\s*,\s*(\d+)", n)
    if m:
        mode = int(m.group(1))
        return "score_rowstat" if mode == 4 else ("score_select" if mode & 1 else "score_stats")
    for key, fam in (("k_kgrad", "kgrad"), ("k_select", "select"), ("k_qt", "qt"), ("k_pbar", "pbar"),
                     ("k_knorm", "knorm"), ("k_rows", "score_select"), ("k_row_", "score_rowstat")):
        if key in n:
            return fam
    return None


def _rocprof_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {directory}")
    return rows


def _short_kernel(name):
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("fwpkm::", "")


def _call_timeline(rows):
    """The last call's kernels (from its last k_knorm on): span, time with
    any kernel running, per-stream kernel time and gaps, chunk period."""
    rows = sorted(rows, key=lambda r: int(r["Start_Timestamp"]))
    kn = [i for i, r in enumerate(rows) if "k_knorm" in r["Kernel_Name"]]
    seg = rows[kn[-1]:] if kn else rows
    iv = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in seg)
    busy, (cs, ce) = 0, iv[0]
    for a, b in iv[1:]:
        if a > ce:
            busy += ce - cs
            cs, ce = a, b
        else:
            ce = max(ce, b)
    busy += ce - cs
    span = max(b for _, b in iv) - iv[0][0]
    lines = ["", f"Last call: {len(seg)} kernels over {span / 1e6:.3f} ms, some kernel running for "
             f"{busy / 1e6:.3f} ms.", "", "| stream (queue) | kernels | kernel time ms | gaps ms | median gap us |",
             "|---|---|---|---|---|"]
    byq = {}
    for r in seg:
        byq.setdefault(r["Queue_Id"], []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r))
    for q, L in sorted(byq.items()):
        L.sort(key=lambda x: x[0])
        gaps = sorted(b[0] - a[1] for a, b in zip(L, L[1:]))
        med = gaps[len(gaps) // 2] / 1e3 if gaps else 0.0
        lines.append(f"| {q} | {len(L)} | {sum(e - s for s, e, _ in L) / 1e6:.3f} | {sum(gaps) / 1e6:.3f} | {med:.1f} |")
    sel = [int(r["Start_Timestamp"]) for r in seg if "k_select" in r["Kernel_Name"] and "ovf" not in r["Kernel_Name"]]
    if len(sel) > 1:
        per = [(b - a) / 1e3 for a, b in zip(sel, sel[1:])]
        lines += ["", f"Chunk period (one selection launch to the next): mean {sum(per) / len(per):.1f} us, "
                  f"min {min(per):.1f}, max {max(per):.1f}."]
    return seg, lines


def summarize_trace(directory, last_call=False):
    """Per-kernel dispatch counts and mean durations of the library's kernels
    in a rocprofv3 kernel trace, and the per-chunk-step time of each kernel
    family (one gather launch per chunk step of B sequences, or two
    half-batch ones).  last_call: the last forward_seq call only, with its
    streams' gaps."""
    rows = _rocprof_rows(directory, "kernel_trace.csv")
    rows = [r for r in rows if "fwpkm::" in r["Kernel_Name"]]
    extra = []
    if last_call:
        rows, extra = _call_timeline(rows)
    per = {}
    for r in rows:
        name = r["Kernel_Name"]
        if "fwpkm::" not in name:
            continue  # the input generation's and the row-count measurement's kernels
        dt = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.setdefault(name, []).append(dt)
    lines = ["| kernel | dispatches | avg us | total ms |", "|---|---|---|---|"]
    for name, ts in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        short = _short_kernel(name)
        lines.append(f"| `{short}` | {len(ts)} | {sum(ts) / len(ts):.1f} | {sum(ts) / 1e3:.2f} |")
    fam = {}
    for name, ts in per.items():
        f = kernel_family(name)
        if f:
            fam[f] = fam.get(f, 0.0) + sum(ts)
    steps = sum(1 for r in rows if "k_select<" in r["Kernel_Name"] or "k_select_gather" in r["Kernel_Name"]
                or "k_select_rows" in r["Kernel_Name"])
    if steps:
        lines += ["", f"Per chunk step ({steps} selections):", "", "| family | us per chunk step |", "|---|---|"]
        for f, t in sorted(fam.items(), key=lambda kv: -kv[1]):
            lines.append(f"| {f} | {t / steps:.1f} |")
    print("\n".join(lines + extra))


def summarize_decode_calls(directory, first, count):
    """Kernel time and launch spacing of decode calls first .. first+count-1
    of a rocprofv3 kernel trace of `bench.py --decode`; each call starts with
    one whole-row scoring launch (k_rows)."""
    rows = sorted((r for r in _rocprof_rows(directory, "kernel_trace.csv") if "fwpkm::" in r["Kernel_Name"]),
                  key=lambda r: int(r["Start_Timestamp"]))
    starts = [i for i, r in enumerate(rows) if "k_rows<" in r["Kernel_Name"]]
    if len(starts) <= first + count:
        raise SystemExit(f"the trace has {len(starts)} calls; {first + count + 1} needed")
    a, b = starts[first], starts[first + count]
    win = rows[a:b]
    per = {}
    for r in win:
        per.setdefault(_short_kernel(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    tot = sum(sum(v) for v in per.values())
    wall = (int(rows[b]["Start_Timestamp"]) - int(win[0]["Start_Timestamp"])) / 1e3
    lines = [f"Calls {first} .. {first + count - 1}: {tot / count:.1f} us of kernels per call, "
             f"calls {wall / count:.1f} us apart.", "",
             "| kernel | launches | avg us | us per decode call |", "|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {len(v)} | {sum(v) / len(v):.2f} | {sum(v) / count:.2f} |")
    print("\n".join(lines))


def summarize_pmc(fetch_dir, write_dir, workload):
    """HBM bytes per kernel family launch from FETCH_SIZE and WRITE_SIZE
    passes (KiB per dispatch), scaled by what the same counters read for the
    calibration kernel of --profile-only (torch.neg over 2^28 float32: 1 GiB
    read, 1 GiB written).  Assumes one launch per family per chunk step (one
    kernel at a time, full batches)."""
    def per_kernel(directory, counter):
        vals = {}
        for r in _rocprof_rows(directory, "counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Dispatch_Id"], r["Kernel_Name"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return vals
    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    gib_kib = float(1 << 20)
    def calib(vals):
        c = [v for (_, n), v in vals.items() if "neg" in n]
        if not c:
            raise SystemExit("no calibration dispatch (torch.neg) in the counter output")
        return gib_kib / (sum(c) / len(c))
    fs, wsc = calib(fetch), calib(write)
    def family_totals(vals):
        tot, steps = {}, 0
        for (_, n), v in vals.items():
            f = kernel_family(n)
            if f:
                tot[f] = tot.get(f, 0.0) + v
            if "k_select<" in n:
                steps += 1
        return tot, steps
    ft, steps = family_totals(fetch)
    wt, steps_w = family_totals(write)
    if not steps or steps != steps_w:
        raise SystemExit(f"chunk steps differ between the passes ({steps}, {steps_w})")
    print(f"fetch scale {fs:.4f}, write scale {wsc:.4f}; {steps} chunk steps")
    print("| family | FETCH_SIZE KiB/step (raw) | WRITE_SIZE KiB/step (raw) | HBM bytes/step (scaled) |")
    print("|---|---|---|---|")
    for f in sorted(ft):
        fk, wk = ft[f] / steps, wt.get(f, 0.0) / steps
        hbm = (fk * fs + wk * wsc) * 1024
        print(f"| {f} | {fk:.0f} | {wk:.0f} | {hbm / 1e6:.1f} MB |")
        if f in KERNEL_SRC:
            out = {"kernel": f, "workload": workload, "src_hash": src_hash(*KERNEL_SRC[f]),
                   "hbm_bytes_per_launch": hbm, "fetch_scale": fs, "write_scale": wsc,
                   "fetch_kib_raw": fk, "write_kib_raw": wk,
                   "command": "FWPKM_DEBUG=1 FWPKM_SINGLE_STREAM=1 rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) "
                              "--output-format csv -d <dir> -o run -- python3 -u bench.py --profile-only "
                              f"--workload {workload} --steps 2 --warmup 1"}
            with open(os.path.join(ROOT, "profiles", f"{f}_{workload}_pmc.json"), "w") as fh:
                json.dump(out, fh, indent=1)


def summarize_mfma(directory):
    """Matrix-core work of the scoring, row-statistic and key-step kernels
    from one rocprofv3 --pmc pass of SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_INSTS_VALU_MFMA_MOPS_F32 and
    GRBM_GUI_ACTIVE: per kernel, the executed MFMA flops per dispatch (MOPS
    x 512, recomputes included), their rate over the dispatch's duration
    against the dense bf16 peak, and the MFMA-busy fraction
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs).
    Counter values are summed over the instances rocprofv3 reports."""
    acc, disp, dur = {}, {}, {}
    for r in _rocprof_rows(directory, "counter_collection.csv"):
        n = r["Kernel_Name"]
        if not any(k in n for k in ("k_score<", "k_kgrad<", "k_rows<")):
            continue
        k = _short_kernel(n)
        c = acc.setdefault(k, {})
        c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        seen = disp.setdefault(k, set())
        if r["Dispatch_Id"] not in seen:
            seen.add(r["Dispatch_Id"])
            dur[k] = dur.get(k, 0.0) + (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    print("| kernel | dispatches | avg us | executed GFLOP / dispatch | TFLOP/s | % of bf16 peak | MFMA busy % |")
    print("|---|---|---|---|---|---|---|")
    for k in sorted(acc, key=lambda k: -dur[k]):
        n, c = len(disp[k]), acc[k]
        us = dur[k] / n
        flops = (c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0)) * 512 / n
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (c["GRBM_GUI_ACTIVE"] / 8 * 1024)
        tfs = flops / (us * 1e-6) / 1e12
        print(f"| `{k}` | {n} | {us:.1f} | {flops / 1e9:.2f} | {tfs:.0f} | {100 * tfs / MFMA_PEAK_TFS['bf16']:.1f} "
              f"| {100 * busy:.1f} |")


GOLDEN_RECALL = os.path.join(ROOT, "tests", "golden", "long_recall.json")


def planted_recall_report(cfg, wl, passes, q, v, g, start_state, extra):
    """One fwpkm_forward_seq of `passes` passes from the workload's initial
    state; recall of the planted bindings at their first and last occurrence
    in the last pass, beside the CPU oracle's recall for the same inputs and
    pass count (stored by tests/golden/make_long_recall.py, when it was made
    for this workload)."""
    import torch
    from sparse_weight_memory_sub_amd import fwpkm
    from sparse_weight_memory_sub_amd.workloads import planted_recall

    K1, K2, V = (x.clone() for x in start_state)
    out = fwpkm.fwpkm_forward_seq(cfg, q, v, g, K1, K2, V, passes=passes, want_vhat=True)
    torch.cuda.synchronize()
    pv, pos = extra["plant_v"], extra["plant_pos"]
    vh = out["vhat"][0]
    first = vh[pos.min(1).values.to(vh.device)].cpu()
    last = vh[pos.max(1).values.to(vh.device)].cpu()
    rf, af, _ = planted_recall(first, pv)
    rl, al, _ = planted_recall(last, pv)
    rep = {"passes": passes, "bindings": int(pv.shape[0]), "reps": int(pos.shape[1]),
           "gpu_first": rf, "gpu_last": rl, "oracle_first": None, "oracle_last": None,
           "definition": "share of bindings whose v_hat at the binding's first (last) occurrence in the last "
                         "pass is closest in cosine to its own z-scored value among all bindings' values"}
    try:
        gold = json.load(open(GOLDEN_RECALL))
        ok = gold.get("T") == wl.T and gold.get("seed") == wl.seed and str(passes) in gold["passes"]
    except (OSError, ValueError, KeyError):
        ok = False
    if ok:
        gp = gold["passes"][str(passes)]
        rep["oracle_first"], rep["oracle_last"] = gp["recall_first"], gp["recall_last"]
        rep["agree_first"] = sum(a == b for a, b in zip(af, gp["argmax_first"]))
        rep["agree_last"] = sum(a == b for a, b in zip(al, gp["argmax_last"]))
    log(f"recall after {passes} pass(es): GPU first {rf:.4f} last {rl:.4f}; oracle first "
        f"{rep['oracle_first']} last {rep['oracle_last']}")
    return rep


def prequeued_step(torch, step, stream):
    """One step enqueued in full while a sleep kernel holds the stream, then
    timed on the device from the sleep's end: the GPU-side time of the step
    with every launch already queued, so the host's enqueue pace (several
    microseconds per launch and per cross-stream event) cannot show.  Valid
    when the host finished enqueueing before the sleep ended (the sleep is
    timed from a calibration launch, hence the 10% margin).  The step starts
    right after a long single-wave kernel, so the clocks may still be
    ramping: this is a diagnostic beside `value`, not a replacement."""
    cycles = 1 << 26
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    torch.cuda._sleep(cycles)
    b.record(stream)
    torch.cuda.synchronize()
    per_cycle_ms = a.elapsed_time(b) / cycles
    host_est_ms = None
    for _ in range(2):
        sleep_ms = max(200.0, 4.0 * (host_est_ms or 0.0))
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(sleep_ms / per_cycle_ms))
        start.record(stream)
        h0 = time.perf_counter()
        step()
        host_ms = (time.perf_counter() - h0) * 1e3
        stop.record(stream)
        torch.cuda.synchronize()
        host_est_ms = host_ms
        if host_ms < 0.9 * sleep_ms:
            break
    return {"ms_per_step": start.elapsed_time(stop), "host_enqueue_ms": host_ms, "sleep_ms": sleep_ms,
            "valid": host_ms < 0.9 * sleep_ms}


def main():
    args = parse()
    if args.summarize_trace:
        if args.decode_calls:
            summarize_decode_calls(args.summarize_trace, *args.decode_calls)
        else:
            summarize_trace(args.summarize_trace, args.last_call)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.workload)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the FwPKM layer benchmark runs on one GPU; --gpus must be 1",
                          "requested_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from sparse_weight_memory_sub_amd import fwpkm
    from sparse_weight_memory_sub_amd.workloads import WORKLOADS, make_state, make_tokens

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if args.ceiling:
        ceiling_bench(args)
        return
    wl = WORKLOADS[args.workload]
    cfg, B, T = wl.cfg, wl.B, wl.T
    if args.score or args.no_gate_weight:
        cfg = cfg.replace(score=args.score or cfg.score, gate_weight=not args.no_gate_weight and cfg.gate_weight)
        wl = wl.__class__(**{**wl.__dict__, "cfg": cfg,
                             "name": wl.name + ("-dot" if cfg.score == "dot" else "")
                             + ("-nogate" if not cfg.gate_weight else "")})
    passes = args.passes or wl.passes
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    q, v, g, extra = make_tokens(cfg, B, T, wl.seed, wl.kind)
    planted = wl.kind == "planted"
    # the planted workload's state is drawn on the host, as the oracle's
    # recall run draws it, so the two recalls start from the same bits
    K1, K2, V = make_state(cfg, B, wl.seed, device="cpu" if planted else dev)
    K1, K2, V = (x.to(dev) for x in (K1, K2, V))
    q, v, g = q.to(dev), v.to(dev), g.to(dev)
    log(f"workload {wl.name}: B={B} T={T} N={cfg.N} H={cfg.heads} d_q={cfg.d_q} d_v={cfg.d_v} "
        f"k={cfg.k} C={cfg.chunk} {cfg.store}; inputs ready in {time.time() - t0:.1f}s")

    if args.decode:
        decode_bench(args, cfg, wl, B, q, v, g, K1, K2, V)
        return
    if args.usage:
        usage_bench(args, cfg, wl, B, T, q, v, g, K1, K2, V)
        return
    if args.backward:
        backward_bench(args, cfg, wl, B, T, q, v, g, K1, K2, V)
        return

    want_cpu = not (args.no_cpu_baseline or args.profile_only)
    if want_cpu:
        ns = min(args.cpu_seqs or 5, B)
        pristine = [x[:ns].cpu() for x in (K1, K2, V)]
    start_state = [x.clone() for x in (K1, K2, V)] if planted and not args.profile_only else None

    o = torch.empty((B, T, cfg.d_v), dtype=torch.float32, device=dev)
    ws = torch.empty(fwpkm.workspace_bytes(cfg, B, T), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        fwpkm.fwpkm_forward_seq(cfg, q, v, g, K1, K2, V, passes=passes, o=o, ws=ws, stream=stream)

    if args.profile_only:
        # Counter scale for the profile passes: an elementwise kernel of known
        # traffic (reads 1 GiB, writes 1 GiB).
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration done (3 x torch.neg over 2^28 float32)")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")

    def timed(events):
        """K steps bracketed by synchronisation and stream events; with
        `events` the library also brackets every kernel family launch."""
        fwpkm.timing_enable(events)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            step()
        stop.record(stream)
        torch.cuda.synchronize()
        fwpkm.timing_enable(False)
        return start.elapsed_time(stop) / args.steps

    ms_step = timed(events=False)
    tokens_step = B * T * passes
    value = tokens_step / (ms_step / 1e3)
    log(f"{args.steps} steps: {ms_step:.3f} ms/step, {value:.4g} tokens/s")

    result = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.store, "data": "synthetic",
        "config": {"workload": wl.name, "n_slots": cfg.N, "heads": cfg.heads, "d_q": cfg.d_q, "d_v": cfg.d_v,
                   "k_half": cfg.k_half, "k": cfg.k, "chunk": cfg.chunk, "batch": B, "seq_len": T,
                   "score": cfg.score, "gate_weight": cfg.gate_weight,
                   "passes": passes, "storage": cfg.store, "accumulate": "f32", "state": "carried across steps"},
    }
    if args.prequeue:
        result["prequeued"] = prequeued_step(torch, step, stream)
        log(f"prequeued: {result['prequeued']}")
    if args.profile_only:
        print(json.dumps(result), flush=True)
        return
    # the same K steps again with every kernel family launch bracketed by HIP
    # events; while timing is on the library runs one kernel at a time, so
    # each duration is the kernel's own (the overlapped schedule above is what
    # `value` measures)
    ms_ev = timed(events=True)
    tk = fwpkm.timing_read()
    result["ms_per_step_with_kernel_events"] = ms_ev
    log(f"with kernel events: {ms_ev:.3f} ms/step")

    # --- unique rows written per chunk, measured on sampled chunks ---
    nchunks = (T + cfg.chunk - 1) // cfg.chunk
    Us = []
    Ks = [x.clone() for x in (K1, K2, V)]
    for c in sorted({0, nchunks // 2, nchunks - 1}):
        c0, c1 = c * cfg.chunk, min(T, (c + 1) * cfg.chunk)
        r = fwpkm.fwpkm_retrieve(cfg, q[:, c0:c1].contiguous(), v[:, c0:c1].contiguous(), g[:, c0:c1].contiguous(),
                                 *Ks, want=("idx",))
        n_t = (c1 - c0) if c1 < T else (c1 - c0 - 1)
        idx = r["idx"][:, :n_t].reshape(B, -1)
        Us.append(float(sum(torch.unique(idx[b]).numel() for b in range(B))) / B)
    del Ks
    U = sum(Us) / len(Us)
    n_tgt = cfg.chunk  # all but the sequence's last chunk
    alg = algorithmic(cfg, B, min(cfg.chunk, T), n_tgt, U)
    kernels = {}
    for name, (ms, n) in tk.items():
        if n == 0:
            continue
        avg = ms / n
        entry = {"avg_ms": avg, "launches": n, "share": ms / sum(x[0] for x in tk.values())}
        if name in ("gather", "scatter"):
            entry["algorithmic_bytes"] = alg[name]
            entry["GB/s"] = alg[name] / (avg / 1e3) / 1e9
            entry["frac_hbm_peak"] = entry["GB/s"] / HBM_PEAK_GBS
        elif name in ("score_select", "score_rowstat", "kgrad"):
            entry["algorithmic_flops"] = alg[name]
            entry["TFLOP/s"] = alg[name] / (avg / 1e3) / 1e12
            entry["frac_mfma_peak"] = entry["TFLOP/s"] / MFMA_PEAK_TFS[cfg.store]
        kernels[name] = entry
    # dominant kernel: the family with the largest share of kernel time
    dom = max((k for k in kernels if "algorithmic_bytes" in kernels[k] or "algorithmic_flops" in kernels[k]),
              key=lambda k: kernels[k]["share"])
    d = kernels[dom]
    if "algorithmic_bytes" in d:
        result["roofline"] = {"kernel": dom, "bound": "hbm", "achieved": d["GB/s"], "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": d["frac_hbm_peak"], "traffic": traffic_from_profiles(dom, wl.name),
                              "bytes_per_launch": d["algorithmic_bytes"], "avg_launch_ms": d["avg_ms"]}
    else:
        peak = MFMA_PEAK_TFS[cfg.store]
        result["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": d["TFLOP/s"], "peak": peak,
                              "unit": "TFLOP/s", "frac": d["frac_mfma_peak"],
                              "traffic": traffic_from_profiles(dom, wl.name),
                              "flops_per_launch": d["algorithmic_flops"], "avg_launch_ms": d["avg_ms"]}
    bpt = layer_bytes_per_token(cfg, U)
    roof_tps = HBM_PEAK_GBS * 1e9 / bpt
    result["roofline"]["layer_bytes_per_token"] = bpt
    result["roofline"]["layer_roofline_tokens_per_s"] = roof_tps
    result["roofline"]["layer_frac"] = value / roof_tps
    result["kernels"] = kernels
    result["unique_rows_per_chunk_seq"] = U
    result["reads_per_chunk_seq"] = n_tgt * cfg.heads * cfg.k
    rl = result["roofline"]
    log(f"dominant kernel {dom}: {rl['achieved']:.1f} {rl['unit']} ({100 * rl['frac']:.1f}% of peak); U={U:.0f}; "
        f"layer {value:.4g} of {roof_tps:.4g} tokens/s at {bpt:.0f} B/token ({100 * rl['layer_frac']:.1f}%)")

    # --- planted bindings: recall after `passes` passes from the initial state ---
    if start_state is not None:
        result["recall"] = planted_recall_report(cfg, wl, passes, q, v, g, start_state, extra)
        del start_state

    # --- CPU oracle on a bounded sample of the same workload ---
    if want_cpu:
        import oracle
        ns = min(args.cpu_seqs or 5, B)
        # about ten seconds of oracle work: the long sequence's first 16 chunks
        nc = args.cpu_chunks or (min(nchunks, 16) if planted else nchunks)
        qs, vs, gs = (x[:ns].cpu() for x in (q, v, g))
        threads = oracle.num_threads()
        t1 = time.perf_counter()
        oracle.forward_seq(cfg, qs, vs, gs, *pristine, passes=1, chunk_limit=nc)
        dt = time.perf_counter() - t1
        tok = ns * min(T, nc * cfg.chunk)
        # the same oracle on one thread, over one sequence's first chunk
        oracle.set_threads(1)
        t1 = time.perf_counter()
        oracle.forward_seq(cfg, qs[:1], vs[:1], gs[:1], *(x[:1] for x in pristine), passes=1, chunk_limit=1)
        dt1 = time.perf_counter() - t1
        oracle.set_threads(threads)
        tok1 = min(T, cfg.chunk)
        result["cpu_baseline"] = {"value": tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                                  "sample": f"{ns} sequence(s) x first {nc} chunk(s) of pass 1 "
                                            f"({tok} tokens, {dt:.1f} s, fp64 C oracle, OpenMP)",
                                  "value_1thread": tok1 / dt1,
                                  "sample_1thread": f"1 sequence x first chunk ({tok1} tokens, {dt1:.1f} s)"}
        log(f"cpu oracle: {tok / dt:.4g} tokens/s on {threads} threads ({dt:.1f} s); "
            f"{tok1 / dt1:.4g} tokens/s on 1 thread ({dt1:.1f} s)")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
