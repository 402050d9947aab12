#!/usr/bin/env python3
"""Benchmark of the hybrid sparse attention forward hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic inputs that
are already resident in HBM: block compression of K/V for CSA (m=4) and HCA
(m=128), lightning-indexer scoring + exact top-k, and the gated window + HCA
+ CSA attention.  Default workload: the CSA-only long prefill (B1 T131072
H32 Hkv4 d128 bf16, CSA m4 k512 with 4 indexer heads, W128, gates [0,1,0]),
the largest configuration that fits one GPU; every timed step starts from
flushed caches.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "hybrid sparse attn fwd queries/s + % HBM/MFMA roofline at 1 MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense, published
KERNEL_SOURCES = {
    "compress_csa": "compress.hip", "compress_hca": "compress.hip", "compress_dual": "compress.hip",
    "index_topk": "indexer.hip", "attention": "attention.hip", "backward": "backward.hip",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workload
def build_inputs(name, seed=0, gates=None, d_idx=None):
    from sparse_hybrid_attention_amd import synth
    over = {} if gates is None else {"gates": gates}
    if d_idx is not None:
        over["d_idx"] = d_idx
    return synth.make_inputs(name, seed=seed, **over)


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda:0")


def make_pipeline(inp, q4=False, rope=None, overlap=False):
    from sparse_hybrid_attention_amd import binding
    from sparse_hybrid_attention_amd.binding import HybridPipeline
    cfg = inp["cfg"]
    if cfg["kind"] == "decode":
        caches = {n: to_dev(inp[n]) for n in ("k_csa", "v_csa", "k_hca", "v_hca")}
        extra = {}
        if q4:
            # 4-bit storage of the compressed caches, made once by the library's
            # own encoder (outside the timed steps); the attention decodes them
            for br in ("hca", "csa"):
                pair = []
                for n in ("k_" + br, "v_" + br):
                    x = caches[n]
                    codes, params = binding.cache_quant4(x)
                    caches[n] = codes.view(*x.shape[:-1], x.shape[-1] // 2)
                    pair.append(params)
                extra["q4_" + br] = tuple(pair)
        return HybridPipeline(q=to_dev(inp["q"]), gates=to_dev(inp["gates"]), W=cfg["W"],
                              k_raw=to_dev(inp["k_win"]), v_raw=to_dev(inp["v_win"]),
                              q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"],
                              qI=to_dev(inp["qI"]), kI=to_dev(inp["kI"]), w=to_dev(inp["w"]),
                              k=cfg["k"], m_csa=cfg["m_csa"], m_hca=cfg["m_hca"], overlap=overlap, **caches,
                              **extra)
    if q4:
        raise SystemExit("--q4 applies to the decode workload (caches given up front)")
    kw = {}
    if cfg.get("m_csa"):
        kw.update(zk_csa=to_dev(inp["zk_csa"]), zv_csa=to_dev(inp["zv_csa"]), m_csa=cfg["m_csa"],
                  qI=to_dev(inp["qI"]), kI=to_dev(inp["kI"]), w=to_dev(inp["w"]), k=cfg["k"])
    if cfg.get("m_hca"):
        kw.update(zk_hca=to_dev(inp["zk_hca"]), zv_hca=to_dev(inp["zv_hca"]), m_hca=cfg["m_hca"])
    if rope is not None:
        # RoPE of the query on its last half (the Tiny-R2 split of a rope part
        # beside a non-rope part), base 10000
        d = cfg["d"]
        kw.update(rope_q=(d // 2, d // 2, 10000.0), rope_fused=rope == "fused")
    return HybridPipeline(q=to_dev(inp["q"]), gates=to_dev(inp["gates"]), W=cfg["W"],
                          k_raw=to_dev(inp["k"]), v_raw=to_dev(inp["v"]), **kw)


def n_visible(t, W, m, N):
    s = t - W + 1
    return 0 if s <= 0 else min(N, s // m)


def algorithmic(inp, pipe):
    """Algorithmic (compulsory) HBM bytes and MFMA flops per launch of each kernel."""
    import torch
    cfg = inp["cfg"]
    esz = 2 if cfg["dtype"] == 0 else 4
    B, H, Hkv, d, W = cfg["B"], cfg["H"], cfg["Hkv"], cfg["d"], cfg["W"]
    g = inp["gates"]
    out = {}
    if cfg["kind"] == "decode":
        Tq, Tr = 1, W
        q_pos0, raw_pos0 = inp["q_pos0"], inp["raw_pos0"]
        Nc, Nh = cfg["N_csa"], cfg["N_hca"]
    else:
        Tq = Tr = cfg["T"]
        q_pos0 = raw_pos0 = 0
        Nc = Tr // cfg["m_csa"] if cfg.get("m_csa") else 0
        Nh = Tr // cfg["m_hca"] if cfg.get("m_hca") else 0
    t = np.arange(Tq, dtype=np.int64) + q_pos0
    win = np.minimum(t + 1, W).astype(np.float64)                 # window keys per query
    for name, m in (("compress_csa", cfg.get("m_csa")), ("compress_hca", cfg.get("m_hca"))):
        if name in pipe.names():
            N = Tr // m
            out[name] = dict(bytes=2 * B * N * m * Hkv * d * esz + 2 * B * N * Hkv * d * esz
                             + 2 * m * Hkv * d * 4, flops=0.0, units=B * N, unit="entries")
    if "compress_dual" in pipe.names():
        m1, m2 = cfg["m_csa"], cfg["m_hca"]
        N1, N2 = Tr // m1, Tr // m2
        out["compress_dual"] = dict(bytes=2 * B * Tr * Hkv * d * esz + 2 * B * (N1 + N2) * Hkv * d * esz
                                    + 2 * (m1 + m2) * Hkv * d * 4, flops=0.0, units=B * (N1 + N2),
                                    unit="entries")
    if "rope_q" in pipe.names():
        # the rotated half of every query row read and written, one position per row
        out["rope_q"] = dict(bytes=2 * B * Tq * H * (d // 2) * esz + B * Tq * 8, flops=0.0, units=B * Tq,
                             unit="query rows")
    if "index_topk" in pipe.names():
        Hi, di, k = cfg["Hi"], cfg["d_idx"], cfg["k"]
        vis = np.array([n_visible(x, W, cfg["m_csa"], Nc) for x in t], dtype=np.float64)
        pairs = B * vis.sum()
        out["index_topk"] = dict(bytes=B * Tq * Hi * di * esz + B * Nc * di * esz + B * Tq * Hi * 4
                                 + B * Tq * k * 4, flops=2.0 * di * Hi * pairs, units=pairs,
                                 unit="scored pairs")
    # attention: each tensor once; the CSA cache counts the entries selected by anyone
    use_hca = pipe.k_hca is not None and (g[:, 0] != 0).any()
    use_csa = pipe.idx is not None and (g[:, 1] != 0).any()
    # bytes of one compressed-cache row: dtype values, or d / 2 bytes of 4-bit codes
    row_h = d // 2 if getattr(pipe, "q4_hca", False) else d * esz
    row_c = d // 2 if getattr(pipe, "q4_csa", False) else d * esz
    keys = win.copy()
    byt = 2 * B * Tq * H * d * esz + 2 * B * Tr * Hkv * d * esz + H * 3 * 4
    if use_hca:
        vis_h = np.array([n_visible(x, W, cfg["m_hca"], Nh) for x in t], dtype=np.float64)
        keys += vis_h
        byt += 2 * B * int(vis_h.max()) * Hkv * row_h
    if use_csa:
        idx = pipe.idx
        sel = (idx >= 0).sum(dim=-1).to(torch.float64).mean(dim=0).cpu().numpy()
        keys += sel
        used = 0
        for b in range(B):
            used += int(torch.unique(idx[b]).numel()) - int((idx[b] < 0).any().item())
        byt += 2 * used * Hkv * row_c + B * Tq * cfg["k"] * 4
    pairs = B * H * keys.sum()
    out["attention"] = dict(bytes=float(byt), flops=4.0 * d * pairs, units=B * keys.sum(),
                            unit="attended (query, key) pairs")
    if use_csa:
        # K and V rows of every selected entry, as the kernel reads them (once
        # per query and KV head): served mostly from L2 / MALL, not HBM
        out["attention"]["gathered_bytes"] = float(B * sel.sum() * Hkv * 2 * row_c)
    return out


PROBE_LIB = os.path.join(ROOT, "sparse_hybrid_attention_amd", "libshattn_probe.so")


def load_probes():
    """The device measurement probes (libshattn_probe.so, built beside the
    library; not part of it)."""
    lib = ctypes.CDLL(PROBE_LIB)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.shattn_probe_mfma.argtypes = [i32, i32, i32, vp, vp]
    lib.shattn_probe_mfma.restype = i32
    lib.shattn_probe_gather.argtypes = [vp, i64, i32, i64, i32, i64, i32, i32, vp, vp]
    lib.shattn_probe_gather.restype = i32
    lib.shattn_probe_stream.argtypes = [vp, i64, i32, i32, i32, vp, vp]
    lib.shattn_probe_stream.restype = i32
    return lib


def stream_read_rate(torch, nbytes, buf=None, flush=False):
    """Best streaming-read rate (GB/s) of `shattn_probe_stream` over `nbytes`
    bytes (rounded down to whole 2 KB tiles): 8192 workgroups, 1 KB of
    consecutive bytes per wave load, every W-th tile or one run of tiles per
    wave, 4 or 8 tiles in flight per lane; best of 3 launches each.  With
    `flush`, each launch follows the same 512 MiB overwrite that starts every
    cold timed step (outside the timed span, as the kernel events of a cold
    step exclude it)."""
    import ctypes
    nbytes = max(2048, (int(nbytes) // 2048) * 2048)
    a = buf if buf is not None else torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    probes = load_probes()
    sink = torch.empty(8192 * 256, dtype=torch.int32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    scratch = flush_buffer(torch) if flush else None
    best = None
    for mode in (0, 2):
        for depth in (4, 8):
            for r in range(3):
                if flush:
                    scratch.fill_(r & 255)
                e0.record()
                rc = probes.shattn_probe_stream(ctypes.c_void_p(a.data_ptr()), nbytes, mode, depth, 8192,
                                                ctypes.c_void_p(sink.data_ptr()), stream)
                e1.record()
                torch.cuda.synchronize()
                if rc != 0:
                    raise RuntimeError(f"probe launch failed ({rc})")
                ms = e0.elapsed_time(e1)
                best = ms if best is None else min(best, ms)
    return round(nbytes / (best * 1e-3) / 1e9, 1)


def measure_peaks(torch):
    """Measured device ceilings to read the roofline fractions against: a
    1 GiB device-to-device copy (bytes read + written per second), a 1 GiB
    streaming read (the probe library's stream kernel), the bf16
    MFMA issue rate of a loop of independent MFMAs, and the rate of random
    256-byte row gathers from a table that fits the last-level cache (64 MiB,
    the size of the 128K prefill's CSA cache) and from one that does not
    (4 GiB)."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_of(fn, reps=4):
        best = None
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best
    copy_gbs = 2.0 * n / (best_of(lambda: b.copy_(a)) * 1e-3) / 1e9
    del b
    # a streaming read of the same 1 GiB, the ceiling of read-bound passes
    read_gbs = stream_read_rate(torch, n, a)
    probes = load_probes()
    wgs, iters = 2048, 2048
    sink = torch.empty(16384 * 256, dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def chk(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed ({rc})")
    rates = {}
    for shape, name in ((0, "16x16x32"), (1, "32x32x16")):
        ms = best_of(lambda: chk(probes.shattn_probe_mfma(wgs, iters, shape, ctypes.c_void_p(sink.data_ptr()),
                                                          stream)))
        rates[name] = round(wgs * 4 * iters * 131072 / (ms * 1e-3) / 1e12, 1)
    gather = {}
    reads = 1 << 26                       # 16 GiB of 256-byte rows per launch
    for name, tbytes, slices, depth in (("llc_64MiB", 64 << 20, 1, 8), ("llc_64MiB_4slices", 64 << 20, 4, 8),
                                        ("llc_64MiB_4slices_depth16", 64 << 20, 4, 16),
                                        ("hbm_1GiB", 1 << 30, 1, 8)):
        nrows = tbytes // 256
        ms = best_of(lambda: chk(probes.shattn_probe_gather(ctypes.c_void_p(a.data_ptr()), nrows, 256, 256, slices,
                                                            reads, depth, 8192, ctypes.c_void_p(sink.data_ptr()),
                                                            stream)), 3)
        gather[name] = round(reads * 256 / (ms * 1e-3) / 1e9, 1)
    del a
    return {"copy_GBps": round(copy_gbs, 1), "read_GBps": round(read_gbs, 1),
            "mfma_bf16_TFLOPs": max(rates.values()),
            "mfma_bf16_TFLOPs_by_shape": rates,
            "gather_256B_rows_GBps": gather,
            "method": "best of 4 (gathers: 3): 1 GiB device copy (read + write bytes); 1 GiB streaming read "
                      "(shattn_probe_stream: 8192 workgroups, 16-byte loads, 1 KB per wave load, 4 or 8 tiles of "
                      "2 KB in flight per lane, best of 12); 2048 workgroups x 2048 "
                      "rounds of independent bf16 MFMAs per wave (8 x 16x16x32 or 4 x 32x32x16); 2^26 reads of "
                      "random 256-byte rows from a 64 MiB or 1 GiB table (4slices: each XCD reads one quarter, "
                      "as one KV head per pair of XCDs does in the attention), 8192 workgroups, 8 (or 16) reads "
                      "in flight per lane"}


def flush_buffer(torch, nbytes=512 << 20):
    return torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")


def source_hash(fname):
    p = os.path.join(ROOT, "sparse_hybrid_attention_amd", "csrc", fname)
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
        e = data.get(workload, {}).get(kernel)
        if not e or e.get("source_sha") != source_hash(KERNEL_SOURCES[kernel]):
            return None
        return float(e["hbm_bytes_per_launch"])
    except Exception:
        return None


# ------------------------------------------------------------------ CPU baseline
def host_info():
    """CPU model and the BLAS library NumPy is built with (for cpu_baseline)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]["name"]
    except Exception:
        pass
    return model, blas


def host_workers():
    """Worker processes for the oracle: the host cores this process may use,
    at most 16 (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


_CPU = {}   # inputs shared with forked workers (copy on write)


def _oracle_block(job):
    """Oracle work of one block of consecutive query rows [i0, i1) of sequence
    b (prefill) or of one sequence (decode): indexer + top-k, attention."""
    import oracle as O
    from threadpoolctl import threadpool_limits
    inp, cfg, comp = _CPU["inp"], _CPU["cfg"], _CPU["comp"]
    dt = cfg["dtype"]
    b, i0, i1 = job
    with threadpool_limits(limits=1):
        if cfg["kind"] == "decode":
            sl = slice(b, b + 1)
            q_pos0, raw_pos0 = inp["q_pos0"], inp["raw_pos0"]
            csa = None
            if cfg.get("m_csa"):
                sel = O.index_topk(inp["qI"][sl], inp["kI"][sl], inp["w"][sl], q_pos0, cfg["m_csa"], cfg["W"],
                                   cfg["k"], dt)
                csa = (inp["k_csa"][sl], inp["v_csa"][sl], sel)
            hca = (inp["k_hca"][sl], inp["v_hca"][sl], cfg["m_hca"]) if cfg.get("m_hca") else None
            O.hybrid_attn_fwd(inp["q"][sl], inp["k_win"][sl], inp["v_win"][sl], inp["gates"], W=cfg["W"], dtype=dt,
                              q_pos0=q_pos0, raw_pos0=raw_pos0, hca=hca, csa=csa)
            return 1
        W = cfg["W"]
        r0 = max(0, i0 - W + 1)
        sl = slice(b, b + 1)
        csa = None
        if cfg.get("m_csa"):
            sel = O.index_topk(inp["qI"][sl, i0:i1], inp["kI"][sl], inp["w"][sl, i0:i1], i0, cfg["m_csa"], W,
                               cfg["k"], dt)
            csa = (comp["kc"][sl], comp["vc"][sl], sel)
        hca = (comp["kh"][sl], comp["vh"][sl], cfg["m_hca"]) if cfg.get("m_hca") else None
        O.hybrid_attn_fwd(inp["q"][sl, i0:i1], inp["k"][sl, r0:i1], inp["v"][sl, r0:i1], inp["gates"], W=W,
                          dtype=dt, q_pos0=i0, raw_pos0=r0, hca=hca, csa=csa)
        return i1 - i0


def _oracle_worker(args):
    """Run blocks from this worker's list until its time budget is spent."""
    jobs, budget = args
    t0 = time.perf_counter()
    rows = 0
    for job in jobs:
        rows += _oracle_block(job)
        if time.perf_counter() - t0 >= budget:
            break
    return rows, time.perf_counter() - t0


def cpu_baseline(inp, budget_s=12.0, block=32):
    """The oracle, as it stands (float64 NumPy), on a bounded sample of the
    same workload, spread over the host cores: one worker process per core
    (at most 16), each single-threaded, each taking blocks of `block`
    consecutive query rows at random offsets until `budget_s` seconds are
    spent.  The block compression the sample needs is done once (one thread)
    and charged per query of the whole workload.  Runs before the GPU is
    initialised (the workers are forked)."""
    import multiprocessing as mp

    import oracle as O
    from threadpoolctl import threadpool_limits
    cfg = inp["cfg"]
    dt = cfg["dtype"]
    B = cfg["B"]
    comp = {}
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        if cfg["kind"] != "decode":
            if cfg.get("m_csa"):
                comp["kc"], comp["vc"] = O.compress_kv(inp["k"], inp["v"], inp["zk_csa"], inp["zv_csa"], cfg["m_csa"],
                                                       dt)
            if cfg.get("m_hca"):
                comp["kh"], comp["vh"] = O.compress_kv(inp["k"], inp["v"], inp["zk_hca"], inp["zv_hca"], cfg["m_hca"],
                                                       dt)
    t_comp = time.perf_counter() - t0
    nw = host_workers()
    rng = np.random.default_rng(1)
    if cfg["kind"] == "decode":
        total_q = B
        order = [(b, 0, 1) for b in rng.permutation(B)]
        lists = [order[w::nw] for w in range(nw)]
    else:
        T = cfg["T"]
        total_q = B * T
        lists = []
        for w in range(nw):
            lst = []
            for _ in range(4096):
                b = int(rng.integers(0, B))
                i0 = int(rng.integers(0, max(1, T - block + 1)))
                lst.append((b, i0, min(T, i0 + block)))
            lists.append(lst)
    _CPU.update(inp=inp, cfg=cfg, comp=comp)
    ctx = mp.get_context("fork")
    t1 = time.perf_counter()
    with ctx.Pool(nw) as pool:
        res = pool.map(_oracle_worker, [(l, budget_s) for l in lists])
    wall = time.perf_counter() - t1
    _CPU.clear()
    rows = sum(r for r, _ in res)
    per_query = t_comp / total_q + wall / rows
    model, blas = host_info()
    unit = "queries/s"
    return {"value": round(1.0 / per_query, 2), "unit": unit, "cores": nw, "kind": "oracle",
            "sample": (f"{rows} query rows (all heads, all branches: indexer + top-k + attention) in blocks of "
                       f"{block if cfg['kind'] != 'decode' else 1} consecutive rows at random offsets, {nw} worker "
                       f"processes x 1 thread for {wall:.1f} s wall; plus the block compression of the whole "
                       f"batch ({t_comp:.1f} s, one thread, charged per query); float64 NumPy (the oracle's only "
                       f"precision: the timed code is the code the parity tests check)"),
            "cpu_model": model, "blas": blas, "threads_per_worker": 1}


# ------------------------------------------------------------------ main
APPEND = dict(B=16, Hkv=1, d=128, W=128, m_csa=4, m_hca=128, d_idx=64, pos0=1048576)


def append_alg_bytes(c, steps):
    """Algorithmic HBM bytes of `steps` consecutive appends (positions pos0 ..):
    per token and sequence the new K, V, kI rows read and written to the ring;
    per completed block its m - 1 earlier ring rows read and the entry written;
    each launch reads the logits of the ratios it compresses once."""
    esz = 2
    row = (2 * c["Hkv"] * c["d"] + c["d_idx"]) * esz          # K + V + kI of one token
    kv = 2 * c["Hkv"] * c["d"] * esz
    total = 0
    for s in range(steps):
        t = c["pos0"] + s
        b = 2 * row                                             # new rows in, ring row out
        lg = 0
        if (t + 1) % c["m_csa"] == 0:
            b += (c["m_csa"] - 1) * row + row                   # earlier rows + entry (K, V, kI)
            lg += c["m_csa"] * (2 * c["Hkv"] * c["d"] + c["d_idx"]) * 4
        if (t + 1) % c["m_hca"] == 0:
            b += (c["m_hca"] - 1) * kv + kv
            lg += c["m_hca"] * 2 * c["Hkv"] * c["d"] * 4
        total += c["B"] * b + lg
    return total


def bench_append(args, torch, binding):
    """Decode cache maintenance at the 1M-context decode shape: one token per
    sequence per step, positions advancing from pos0 (a steady-state mix of
    plain appends, CSA completions every 4 tokens, HCA every 128)."""
    from sparse_hybrid_attention_amd import synth
    c = APPEND
    B, Hkv, d, W, d_idx = c["B"], c["Hkv"], c["d"], c["W"], c["d_idx"]
    steps, warm = max(args.steps, 256), args.warmup
    nsteps = warm + steps
    cap_csa = (c["pos0"] + nsteps) // c["m_csa"] + 1
    cap_hca = (c["pos0"] + nsteps) // c["m_hca"] + 1
    small = synth.make_append(B=B, Hkv=Hkv, d=d, W=W, m_csa=c["m_csa"], m_hca=c["m_hca"], d_idx=d_idx,
                              cap_csa=1, cap_hca=1, steps=nsteps, seed=0)
    dev = "cuda:0"
    bf = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    k_ring, v_ring, kI_ring = bf(small["k_ring"]), bf(small["v_ring"]), bf(small["kI_ring"])
    z = {k: torch.from_numpy(small[k]).to(dev) for k in ("zk_csa", "zv_csa", "zk_hca", "zv_hca", "zI")}
    k_csa = torch.zeros((B, cap_csa, Hkv, d), dtype=torch.bfloat16, device=dev)
    v_csa = torch.zeros_like(k_csa)
    k_hca = torch.zeros((B, cap_hca, Hkv, d), dtype=torch.bfloat16, device=dev)
    v_hca = torch.zeros_like(k_hca)
    kI_csa = torch.zeros((B, cap_csa, d_idx), dtype=torch.bfloat16, device=dev)
    k_new, v_new, kI_new = bf(small["k_new"]), bf(small["v_new"]), bf(small["kI_new"])
    pos = (torch.arange(nsteps, dtype=torch.int64, device=dev)[:, None] + c["pos0"]).expand(nsteps, B).contiguous()
    dropped = torch.zeros(1, dtype=torch.int32, device=dev)
    lib = binding.load_library()
    argv = []
    for s in range(nsteps):
        a, keep = binding.make_append_args(pos[s], k_new[s], v_new[s], k_ring, v_ring,
                                           csa=(c["m_csa"], z["zk_csa"], z["zv_csa"], k_csa, v_csa),
                                           hca=(c["m_hca"], z["zk_hca"], z["zv_hca"], k_hca, v_hca),
                                           indexer=(kI_new[s], kI_ring, z["zI"], kI_csa), dropped=dropped)
        argv.append((a, keep))
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    for s in range(warm):
        binding._check(lib.hybrid_cache_append(ctypes.byref(argv[s][0]), sp))
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        binding._check(lib.hybrid_cache_append(ctypes.byref(argv[warm + i][0]), sp))
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if int(dropped.item()) != 0:
        raise RuntimeError("cache append benchmark dropped entries (capacity too small)")
    kms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps
    alg = append_alg_bytes(dict(c, pos0=c["pos0"] + warm), steps) / steps
    ach = alg / (kms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        from threadpoolctl import threadpool_limits
        n_cpu = 512
        st = synth.make_append(B=B, Hkv=Hkv, d=d, W=W, m_csa=c["m_csa"], m_hca=c["m_hca"], d_idx=d_idx,
                               cap_csa=n_cpu // c["m_csa"] + 1, cap_hca=n_cpu // c["m_hca"] + 1, steps=n_cpu,
                               seed=1)
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            for s_ in range(n_cpu):
                O.cache_append([s_] * B, st["k_new"][s_], st["v_new"][s_], st["k_ring"], st["v_ring"], W=W,
                               dtype=0, branches=((c["m_csa"], st["zk_csa"], st["zv_csa"], st["k_csa"], st["v_csa"]),
                                                  (c["m_hca"], st["zk_hca"], st["zv_hca"], st["k_hca"], st["v_hca"])),
                               kI_new=st["kI_new"][s_], kI_ring=st["kI_ring"], kI_branch=(c["m_csa"], st["zI"], st["kI_csa"]))
            dt_cpu = time.perf_counter() - t1
        cpu = {"value": round(B * n_cpu / dt_cpu, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{n_cpu} consecutive appends of the {B} sequences from position 0 (same mix of block "
                         f"completions; the oracle's cost does not depend on the position); float64 NumPy, one "
                         f"thread; {dt_cpu:.1f} s"}
    line = {
        "metric": "decode cache append tokens/s (ring write + block compression)",
        "value": round(B * steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(wall * 1e3 / steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) draws, resident in HBM)",
        "config": {"workload": f"decode cache append, B{B} sequences x 1 token per step at positions from "
                               f"{c['pos0']}, Hkv{Hkv} d{d} bf16, W{W}, CSA m{c['m_csa']} (+ indexer keys "
                               f"d_idx {d_idx}), HCA m{c['m_hca']}", "name": "decode_append",
                   "gpu_ms_per_launch_events": round(kms, 5)},
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 6), "kernel": "cache_append", "traffic": None,
                     "alg_bytes_per_launch": round(alg, 1)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


ROPE = dict(B=8, T=2048, H=12, d=128, rope_off=64, rope_dim=64, base=10000.0)


def bench_rope(args, torch, binding):
    """RoPE in place on the Tiny-R2 query tensor (B8 T2048 H12 d128, the last
    64 channels of each head rotated), one launch per step."""
    from sparse_hybrid_attention_amd import synth
    c = ROPE
    B, T, H, d, off, rd = c["B"], c["T"], c["H"], c["d"], c["rope_off"], c["rope_dim"]
    rows = B * T
    inp = synth.make_rope(rows=rows, heads=H, d=d, max_pos=T, seed=0)
    dev = "cuda:0"
    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    pos = torch.arange(T, dtype=torch.int64, device=dev).repeat(B)   # each sequence from position 0
    lib = binding.load_library()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    call = lambda: binding._check(lib.rope_apply(x.data_ptr(), pos.data_ptr(), rows, H, d, off, rd, c["base"],
                                                 binding.DTYPE_BF16, sp))
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        call()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    alg = rows * H * rd * 2 * 2 + rows * 8     # rotated channels read and written once, one position per row
    ach = alg / (kms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        from threadpoolctl import threadpool_limits
        n_cpu = 4096
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            O.rope(inp["x"][:n_cpu], inp["pos"][:n_cpu], rope_off=off, rope_dim=rd, dtype=binding.DTYPE_BF16,
                   base=c["base"])
            dt_cpu = time.perf_counter() - t1
        cpu = {"value": round(n_cpu / dt_cpu, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"the first {n_cpu} of the {rows} query rows (all {H} heads); float64 NumPy, one thread; "
                         f"{dt_cpu:.1f} s"}
    line = {
        "metric": "RoPE tokens/s (query tensor, in place)",
        "value": round(rows * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) draws, resident in HBM)",
        "config": {"workload": f"RoPE on the Tiny-R2 query tensor, B{B} T{T} H{H} d{d} bf16, channels "
                               f"[{off}, {off + rd}) rotated, base {c['base']:g}", "name": "rope_q",
                   "gpu_ms_per_launch_events": round(kms, 5)},
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 6), "kernel": "rope", "traffic": None,
                     "alg_bytes_per_launch": alg},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


QUANT4 = dict(B=16, N=8192, Hkv=1, d=128)   # the HCA K cache of the 1M-context decode shape


def bench_quant4(args, torch, binding):
    """4-bit storage of the decode HCA K cache (16 x 8192 x 1 x 128 bf16): one
    encode (min/max pass + code pass) and one decode per step."""
    from sparse_hybrid_attention_amd import synth
    c = QUANT4
    n = c["B"] * c["N"] * c["Hkv"] * c["d"]
    xh = synth.make_quant(n=n, seed=0)
    dev = "cuda:0"
    x = torch.from_numpy(xh.view(np.int16)).to(dev).view(torch.bfloat16)
    codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=dev)
    params = torch.empty(2, dtype=torch.float32, device=dev)
    out = torch.empty_like(x)
    lib = binding.load_library()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step():
        binding._check(lib.cache_quant4(x.data_ptr(), n, binding.DTYPE_BF16, codes.data_ptr(), params.data_ptr(), sp))
        binding._check(lib.cache_dequant4(codes.data_ptr(), params.data_ptr(), n, binding.DTYPE_BF16,
                                          out.data_ptr(), sp))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        step()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    alg = 2 * n * 2 + (n + 1) // 2 + (n + 1) // 2 + n * 2   # encode reads x twice, writes codes; decode reads codes, writes x
    ach = alg / (kms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            pk, mn, st = O.quant4(xh, binding.DTYPE_BF16)
            O.dequant4(pk, mn, st, n, binding.DTYPE_BF16)
            dt_cpu = time.perf_counter() - t1
        cpu = {"value": round(n / dt_cpu, 1), "unit": "elements/s", "cores": 1, "kind": "oracle",
               "sample": f"one encode and decode of the whole {n}-element tensor; NumPy, one thread; {dt_cpu:.1f} s"}
    line = {
        "metric": "4-bit cache storage elements/s (encode + decode)",
        "value": round(n * args.steps / wall, 1),
        "unit": "elements/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) draws, resident in HBM)",
        "config": {"workload": f"4-bit storage of the decode HCA K cache, B{c['B']} x {c['N']} entries x "
                               f"Hkv{c['Hkv']} x d{c['d']} bf16", "name": "quant4_hca",
                   "gpu_ms_per_step_events": round(kms, 5)},
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 6), "kernel": "quant4 (all launches of a step)",
                     "traffic": None, "alg_bytes_per_step": alg},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def bench_backward(args, torch, binding):
    """Backward of the Tiny-R2 training-shape prefill (B8 T2048 H=Hkv=12 d128
    bf16; HCA m128, CSA m4 k64, W128, per-head gates U(0,1)): one
    hybrid_sparse_attn_bwd call per step (all its launches), with the
    compressed caches and the CSA selection made beforehand by the forward
    path's own kernels (untimed)."""
    import oracle as O
    from sparse_hybrid_attention_amd import synth
    inp = synth.make_backward("tinyr2_bf16", seed=0)
    cfg = inp["cfg"]
    B, T, H, Hkv, d, W, k = cfg["B"], cfg["T"], cfg["H"], cfg["Hkv"], cfg["d"], cfg["W"], cfg["k"]
    mh, mc = cfg["m_hca"], cfg["m_csa"]
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's float64 backward on the last rows of one sequence (every
        # branch present there), one process
        rows = 96
        q0 = T - rows
        t1 = time.perf_counter()
        kh, vh = O.compress_kv(inp["k"][:1], inp["v"][:1], inp["zk_hca"], inp["zv_hca"], mh, cfg["dtype"])
        kc, vc = O.compress_kv(inp["k"][:1], inp["v"][:1], inp["zk_csa"], inp["zv_csa"], mc, cfg["dtype"])
        idx0 = O.index_topk(inp["qI"][:1, q0:], inp["kI"][:1], inp["w"][:1, q0:], q0, mc, W, k, cfg["dtype"])
        dout = inp["dout"][:1, q0:]
        O.hybrid_attn_bwd(inp["q"][:1, q0:], inp["k"][:1], inp["v"][:1], inp["gates"],
                          (dout.astype(np.uint32) << 16).view(np.float32).astype(np.float64), W=W,
                          dtype=cfg["dtype"], q_pos0=q0, hca=(kh, vh, mh), csa=(kc, vc, idx0))
        dt_cpu = time.perf_counter() - t1
        cpu = {"value": round(rows / dt_cpu, 2), "unit": "query rows/s", "cores": 1, "kind": "oracle",
               "sample": f"the last {rows} query rows of one sequence (all {H} heads, every branch), with that "
                         f"sequence's compression and selection; float64 NumPy, one process; {dt_cpu:.1f} s"}
    dev = "cuda:0"
    D = lambda a: to_dev(a)
    q, kr, vr, dout = D(inp["q"]), D(inp["k"]), D(inp["v"]), D(inp["dout"])
    gates = D(inp["gates"])
    zk_h, zv_h, zk_c, zv_c = D(inp["zk_hca"]), D(inp["zv_hca"]), D(inp["zk_csa"]), D(inp["zv_csa"])
    (k_c, v_c), (k_h, v_h) = binding.hca_compress_kv_dual(kr, vr, zk_c, zv_c, mc, zk_h, zv_h, mh)
    qI, kI, w = D(inp["qI"]), D(inp["kI"]), D(inp["w"])
    idx = binding.csa_index_topk(qI, kI, w, 0, mc, W, k)
    torch.cuda.synchronize()
    lib = binding.load_library()
    a, grads, keep = binding.make_bwd_args(q, kr, vr, gates, dout, W, hca=(zk_h, zv_h, k_h, v_h, mh),
                                           csa=(zk_c, zv_c, k_c, v_c, mc, idx))
    nbytes = int(lib.hybrid_sparse_attn_bwd_workspace_size(ctypes.byref(a)))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    call = lambda: binding._check(lib.hybrid_sparse_attn_bwd(ctypes.byref(a), ctypes.c_void_p(ws.data_ptr()),
                                                             nbytes, sp))
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    scratch = flush_buffer(torch)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        scratch.fill_(i & 255)
        evs[i][0].record(stream)
        call()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    kms = sum(step_ms) / args.steps
    # algorithmic work: every (query row, head, key of its branch sets) pair
    # costs 10 d flops (scores, dout.v, dq, dk, dv); compulsory bytes: Q, dout,
    # K, V, the caches, idx and gates read once, dq, dk, dv and the small
    # logit / gate gradients written once
    pairs = 0
    for t in range(T):
        nw = min(W, t + 1)
        pairs += nw + n_visible(t, W, mh, T // mh) + min(k, n_visible(t, W, mc, T // mc))
    pairs *= B * H
    flops = 10 * d * pairs
    el = 2
    nbytes_alg = (2 * B * T * H * d + 2 * B * T * Hkv * d) * el + 2 * B * (T // mh + T // mc) * Hkv * d * el \
        + B * T * k * 4 + H * 3 * 4 + (B * T * H * d + 2 * B * T * Hkv * d) * 4 + 2 * (mh + mc) * Hkv * d * 4 * 2
    t_hbm = nbytes_alg / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_TFLOPS["bf16"] * 1e12)
    if t_mfma > t_hbm:
        ach = flops / (kms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 3), "peak": MFMA_PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                "frac": round(ach / MFMA_PEAK_TFLOPS["bf16"], 6)}
    else:
        ach = nbytes_alg / (kms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 6)}
    roof.update(kernel="hybrid_sparse_attn_bwd (all launches of a step)", kernel_ms=round(kms, 5),
                alg_bytes_per_launch=nbytes_alg, alg_flops_per_launch=flops,
                traffic=traffic_for("backward", "tinyr2_bwd"),
                TFLOPs_achieved=round(flops / (kms * 1e-3) / 1e12, 3))
    line = {
        "metric": "hybrid sparse attn backward query rows/s",
        "value": round(B * T * args.steps / wall, 1),
        "unit": "query rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) / U(0,1) draws, resident in HBM)",
        "config": {"workload": f"backward of the Tiny-R2 training-shape prefill, B{B} T{T} H=Hkv={H} d{d} bf16, "
                               f"HCA m{mh}, CSA m{mc} k{k} (selection by the indexer), W{W}, gates U(0,1); "
                               f"gradients float32", "name": "tinyr2_bwd",
                   "timing": "each timed step starts from flushed L2 / MALL (cold)",
                   "gpu_ms_per_step_median": round(step_ms[len(step_ms) // 2], 5),
                   "key_pairs_per_step": pairs},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


WORKLOADS = {
    "tinyr2_bf16": "Tiny-R2 training-shape forward, B8 T2048 H=Hkv=12 d128 bf16, CSA m4 k64 "
                   "(indexer 4 heads d_idx 64), HCA m128, W128, gates U(0,1) (all branches)",
    "tiny_fp32": "tiny fp32 forward, B1 T256 H=Hkv=4 d64, CSA m4 k8 (indexer 2 heads), HCA m32, W32",
    "hca_prefill_32k": "HCA-only prefill, B1 T32768 H16 Hkv2 d128 bf16, m128, W128, gates [1,0,0]",
    "csa_prefill_128k": "CSA-only long prefill, B1 T131072 H32 Hkv4 d128 bf16, m4 (32768 entries), k512 "
                        "(4 indexer heads, d_idx 64, fp32 scores), W128, gates [0,1,0]",
    "decode_1m": "decode, B16 x 1 query at 1,048,576 context, H32 Hkv1 d128 bf16, CSA 262144 entries "
                 "k1024 (4 indexer heads, d_idx 64), HCA 8192 entries, W128, gates U(0,1)",
}


def timed_steps(torch, pipe, names, steps, flush):
    """`steps` steps between two synchronisations; with `flush`, every step
    starts with L2 and MALL flushed (a 512 MiB buffer overwritten on the
    pipeline's stream just before it: the flush is inside the timed wall, so
    it only makes the figure conservative).  Per-kernel HIP events are
    recorded on the pipeline's stream around each launch."""
    scratch = flush_buffer(torch) if flush else None
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        if flush:
            with torch.cuda.stream(pipe.stream):
                scratch.fill_(s & 255)
        pipe.run(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del scratch
    ktime = {n: 0.0 for n in names}
    for s in range(steps):
        for j, n in enumerate(names):
            ktime[n] += evs[s][j].elapsed_time(evs[s][j + 1])
    ktime = {n: v / steps for n, v in ktime.items()}   # ms per launch (mean)
    step_ms = sorted(evs[s][0].elapsed_time(evs[s][-1]) for s in range(steps))
    return wall, ktime, step_ms


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="csa_prefill_128k",
                    help="csa_prefill_128k (default: the largest single-GPU configuration), tinyr2_bf16, "
                         "tiny_fp32, hca_prefill_32k, decode_1m, decode_append (cache maintenance), rope_q (RoPE "
                         "on the query tensor), quant4_hca (4-bit cache storage), tinyr2_bwd (backward of the "
                         "Tiny-R2 training-shape prefill)")
    ap.add_argument("--gates", default=None, choices=["mix", "hca", "csa", "swa"],
                    help="override the workload's gate setting (one-hot modes or the U(0,1) mix)")
    ap.add_argument("--d-idx", type=int, default=None, choices=[64, 128],
                    help="override the indexer key width of a workload with an indexer (CSA prefill, "
                         "Tiny-R2, decode)")
    ap.add_argument("--q4", action="store_true",
                    help="decode workload: the HCA and CSA caches in 4-bit storage, decoded by the attention")
    ap.add_argument("--rope", default=None, choices=["fused", "separate"],
                    help="prefill workloads: RoPE of the query (last d/2 channels), inside the attention's Q load "
                         "or as a rope_apply launch before it")
    ap.add_argument("--overlap", action="store_true",
                    help="decode: run the attention's window and HCA items on a second stream beside the indexer "
                         "(measured slower at decode_1m: the indexer already fills the chip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the warm (back-to-back) timing and the measured-peak probes")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall seconds of oracle work per host worker in the CPU baseline")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter scaling for rocprofv3)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the path has no multi-GPU implementation (prefill would "
              "shard by query tile or KV head, decode by sequence-sharded caches with an all-gather of "
              "top-k candidates). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    pipeline_workload = args.workload in WORKLOADS
    inp = cpu = None
    if pipeline_workload and not args.copy_probe:
        log(f"[bench] building inputs for {args.workload}")
        inp = build_inputs(args.workload, gates=args.gates, d_idx=args.d_idx)
        if not args.no_cpu_baseline:
            # before the GPU is touched: the oracle's worker processes are forked
            log("[bench] timing the CPU oracle on a bounded sample")
            cpu = cpu_baseline(inp, budget_s=args.cpu_seconds)
            log(f"[bench] cpu baseline {cpu['value']:.2f} queries/s on {cpu['cores']} workers")

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.copy_probe:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": n, "launches": 3}))
        return

    from sparse_hybrid_attention_amd import binding
    binding.load_library()
    if args.workload == "decode_append":
        bench_append(args, torch, binding)
        return
    if args.workload == "rope_q":
        bench_rope(args, torch, binding)
        return
    if args.workload == "quant4_hca":
        bench_quant4(args, torch, binding)
        return
    if args.workload == "tinyr2_bwd":
        bench_backward(args, torch, binding)
        return
    if not pipeline_workload:
        raise SystemExit(f"unknown workload {args.workload}")
    cfg = inp["cfg"]
    pipe = make_pipeline(inp, q4=args.q4, rope=args.rope, overlap=args.overlap)
    names = pipe.names()
    log(f"[bench] kernels per step: {names}; warmup {args.warmup}")
    for _ in range(args.warmup):
        pipe.run()
    torch.cuda.synchronize()
    alg = algorithmic(inp, pipe)

    # timed region: exactly K steps, each from flushed caches (headline)
    wall, ktime, step_ms = timed_steps(torch, pipe, names, args.steps, flush=True)
    log(f"[bench] timed {args.steps} cold steps in {wall * 1e3:.2f} ms")
    warm = None
    if not args.no_extras:
        w_wall, w_ktime, w_step = timed_steps(torch, pipe, names, args.steps, flush=False)
        warm = {"ms_per_step": round(w_wall * 1e3 / args.steps, 5),
                "gpu_ms_per_step_median": round(w_step[len(w_step) // 2], 5),
                "kernels_ms": {n: round(v, 5) for n, v in w_ktime.items()},
                "note": "the same steps back to back, caches warm from the previous step"}
    ms_per_step = wall * 1e3 / args.steps
    queries = cfg["B"] if cfg["kind"] == "decode" else cfg["B"] * cfg["T"]
    value = queries * args.steps / wall
    dtype = "bf16" if cfg["dtype"] == 0 else "f32"

    kernels = {}
    for n in names:
        a = alg.get(n)
        ms = ktime[n]
        e = {"ms": round(ms, 5)}
        if a:
            e["GB/s"] = round(a["bytes"] / (ms * 1e-3) / 1e9, 1)
            e["TFLOP/s"] = round(a["flops"] / (ms * 1e-3) / 1e12, 2)
            e[a["unit"] + "/s"] = a["units"] / (ms * 1e-3)
            e["alg_bytes"] = a["bytes"]
            e["alg_flops"] = a["flops"]
            if "gathered_bytes" in a:
                e["gathered_bytes"] = a["gathered_bytes"]
                e["gathered GB/s"] = round(a["gathered_bytes"] / (ms * 1e-3) / 1e9, 1)
        kernels[n] = e
    dom = max(names, key=lambda n: ktime[n])
    a = alg[dom]
    t_hbm = a["bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = a["flops"] / (MFMA_PEAK_TFLOPS[dtype] * 1e12)
    ms = ktime[dom]
    if t_mfma > t_hbm:
        ach = a["flops"] / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_PEAK_TFLOPS[dtype],
                "unit": "TFLOP/s", "frac": round(ach / MFMA_PEAK_TFLOPS[dtype], 4)}
    else:
        ach = a["bytes"] / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof["kernel"] = dom
    roof["kernel_ms"] = round(ms, 5)
    roof["alg_per_launch"] = a["flops"] if roof["unit"] == "TFLOP/s" else a["bytes"]
    roof["traffic"] = traffic_for(dom, args.workload)

    peaks = measure_peaks(torch) if not args.no_extras else None
    if peaks is not None and (roof["unit"] == "GB/s" or dtype == "bf16"):
        roof["measured_peak"] = peaks["copy_GBps"] if roof["unit"] == "GB/s" else peaks["mfma_bf16_TFLOPs"]
        roof["frac_of_measured"] = round(roof["achieved"] / roof["measured_peak"], 4)
        if roof["unit"] == "GB/s":
            # read-dominated passes (the decode indexer streams its keys) against
            # the measured streaming-read rate
            roof["measured_read_peak"] = peaks["read_GBps"]
            roof["frac_of_measured_read"] = round(roof["achieved"] / peaks["read_GBps"], 4)
            # the same streaming read over the kernel's own byte count: a
            # pass of a few hundred MB pays its launch, ramp and tail on fewer
            # bytes than the 1 GiB figure does
            # (cold: after the same flush as the timed steps; warm: back to back)
            nb = min(roof["alg_per_launch"], 1 << 30)
            rs = stream_read_rate(torch, nb, flush=True)
            roof["measured_read_peak_same_bytes"] = rs
            roof["frac_of_measured_read_same_bytes"] = round(roof["achieved"] / rs, 4)
            roof["measured_read_peak_same_bytes_warm"] = stream_read_rate(torch, nb)
    if "gathered_bytes" in a:
        # the gathered CSA rows: bytes the kernel reads from L2 / MALL per launch
        # against the measured random-row gather rate of a cache-resident table
        g = a["gathered_bytes"] / (ms * 1e-3) / 1e9
        roof["gather"] = {"bytes_per_launch": a["gathered_bytes"], "achieved_GBps": round(g, 1)}
        if peaks is not None:
            ceil = max(peaks["gather_256B_rows_GBps"].values())
            roof["gather"].update(ceiling_GBps=ceil, frac=round(g / ceil, 4),
                                  ceiling="best measured rate of random 256-byte row gathers (measured_peaks)")
            if roof.get("traffic"):
                # the part of the gather L2 does not serve: the measured bytes
                # past L2 per launch against the probe's rate on a 64 MiB
                # table read by every XCD (whose reads almost never hit L2)
                t = roof["traffic"] / (ms * 1e-3) / 1e9
                c64 = peaks["gather_256B_rows_GBps"]["llc_64MiB"]
                roof["gather"].update(past_l2_GBps=round(t, 1), past_l2_ceiling_GBps=c64,
                                      frac_past_l2=round(t / c64, 4))

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) / U(0,1) draws, resident in HBM)",
        "config": {"workload": WORKLOADS[args.workload] + ("" if args.gates is None else f" [gates: {args.gates}]")
                   + (" [HCA and CSA caches in 4-bit storage]" if args.q4 else "")
                   + (f" [indexer d_idx {args.d_idx}]" if args.d_idx else "")
                   + (f" [RoPE of q, {args.rope}]" if args.rope else "")
                   + (" [window / HCA attention items beside the indexer]" if args.overlap else ""),
                   "name": args.workload, "gates": cfg.get("gates"), "batch": cfg["B"],
                   "query_rows": queries, "timing": "each timed step starts from flushed L2 / MALL (cold)",
                   "gpu_ms_per_step_median": round(step_ms[len(step_ms) // 2], 5)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "warm": warm,
        "measured_peaks": peaks,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
