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


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the FwPKM layer benchmark runs on one GPU; --gpus must be 1",
                          "requested_gpus": args.gpus}))
        sys.exit(2)

    import torch
    from sparse_weight_memory_sub_amd import fwpkm
    from sparse_weight_memory_sub_amd.workloads import WORKLOADS, make_state, make_tokens

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
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
    q, v, g, _ = make_tokens(cfg, B, T, wl.seed, wl.kind)
    K1, K2, V = make_state(cfg, B, wl.seed, device=dev)
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
        ns = args.cpu_seqs or 5
        pristine = [x[:ns].cpu() for x in (K1, K2, V)]

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
    result["kernels"] = kernels
    result["unique_rows_per_chunk_seq"] = U
    result["reads_per_chunk_seq"] = n_tgt * cfg.heads * cfg.k
    rl = result["roofline"]
    log(f"dominant kernel {dom}: {rl['achieved']:.1f} {rl['unit']} ({100 * rl['frac']:.1f}% of peak); U={U:.0f}")

    # --- CPU oracle on a bounded sample of the same workload ---
    if want_cpu:
        import oracle
        ns = args.cpu_seqs or 5
        nc = args.cpu_chunks or nchunks
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
