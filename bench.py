#!/usr/bin/env python3
"""Benchmark of the hybrid sparse attention forward hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic inputs that
are already resident in HBM: block compression of K/V for CSA (m=4) and HCA
(m=128), lightning-indexer scoring + exact top-k, and the gated window + HCA
+ CSA attention.  Default workload: the Tiny-R2 training shape (B8 T2048
H=Hkv=12 d128 bf16, CSA k64 with 4 indexer heads, HCA m128, W128, all three
branches mixed with U(0,1) gates).  Prints one JSON line.

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
    "index_topk": "indexer.hip", "attention": "attention.hip",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ workload
def build_inputs(name, seed=0, gates=None):
    from sparse_hybrid_attention_amd import synth
    over = {} if gates is None else {"gates": gates}
    return synth.make_inputs(name, seed=seed, **over)


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda:0")


def make_pipeline(inp):
    from sparse_hybrid_attention_amd.binding import HybridPipeline
    cfg = inp["cfg"]
    if cfg["kind"] == "decode":
        return HybridPipeline(q=to_dev(inp["q"]), gates=to_dev(inp["gates"]), W=cfg["W"],
                              k_raw=to_dev(inp["k_win"]), v_raw=to_dev(inp["v_win"]),
                              q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"],
                              qI=to_dev(inp["qI"]), kI=to_dev(inp["kI"]), w=to_dev(inp["w"]),
                              k=cfg["k"], m_csa=cfg["m_csa"], m_hca=cfg["m_hca"],
                              k_csa=to_dev(inp["k_csa"]), v_csa=to_dev(inp["v_csa"]),
                              k_hca=to_dev(inp["k_hca"]), v_hca=to_dev(inp["v_hca"]))
    kw = {}
    if cfg.get("m_csa"):
        kw.update(zk_csa=to_dev(inp["zk_csa"]), zv_csa=to_dev(inp["zv_csa"]), m_csa=cfg["m_csa"],
                  qI=to_dev(inp["qI"]), kI=to_dev(inp["kI"]), w=to_dev(inp["w"]), k=cfg["k"])
    if cfg.get("m_hca"):
        kw.update(zk_hca=to_dev(inp["zk_hca"]), zv_hca=to_dev(inp["zv_hca"]), m_hca=cfg["m_hca"])
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
    keys = win.copy()
    byt = 2 * B * Tq * H * d * esz + 2 * B * Tr * Hkv * d * esz + H * 3 * 4
    if use_hca:
        vis_h = np.array([n_visible(x, W, cfg["m_hca"], Nh) for x in t], dtype=np.float64)
        keys += vis_h
        byt += 2 * B * int(vis_h.max()) * Hkv * d * esz
    if use_csa:
        idx = pipe.idx
        sel = (idx >= 0).sum(dim=-1).to(torch.float64).mean(dim=0).cpu().numpy()
        keys += sel
        used = 0
        for b in range(B):
            used += int(torch.unique(idx[b]).numel()) - int((idx[b] < 0).any().item())
        byt += 2 * used * Hkv * d * esz + B * Tq * cfg["k"] * 4
    pairs = B * H * keys.sum()
    out["attention"] = dict(bytes=float(byt), flops=4.0 * d * pairs, units=B * keys.sum(),
                            unit="attended (query, key) pairs")
    if use_csa:
        # K and V rows of every selected entry, as the kernel reads them (once
        # per query and KV head): served mostly from L2 / MALL, not HBM
        out["attention"]["gathered_bytes"] = float(B * sel.sum() * Hkv * 2 * d * esz)
    return out


def measure_peaks(torch, binding):
    """Measured device peaks to read the roofline fractions against: a 1 GiB
    device-to-device copy (bytes read + written per second) and the bf16 MFMA
    issue rate of a loop of independent MFMAs (shattn_mfma_peak_probe)."""
    import ctypes
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(4):
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    copy_gbs = 2.0 * n / (best * 1e-3) / 1e9
    del a, b
    lib = binding.load_library()
    wgs, iters = 2048, 2048
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rates = {}
    for shape, name in ((0, "16x16x32"), (1, "32x32x16")):
        best = None
        for _ in range(4):
            e0.record()
            rc = lib.shattn_mfma_peak_probe(wgs, iters, shape, ctypes.c_void_p(sink.data_ptr()), stream)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(lib.shattn_last_error().decode())
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        rates[name] = round(wgs * 4 * iters * 131072 / (best * 1e-3) / 1e12, 1)
    return {"copy_GBps": round(copy_gbs, 1), "mfma_bf16_TFLOPs": max(rates.values()),
            "mfma_bf16_TFLOPs_by_shape": rates,
            "method": "best of 4: 1 GiB device copy (read + write bytes); 2048 workgroups x 2048 rounds of "
                      "independent bf16 MFMAs per wave (8 x 16x16x32 or 4 x 32x32x16)"}


def cold_steps(torch, pipe, reps=20, flush_bytes=512 << 20):
    """Median step time with L2 / MALL flushed before every step (a 512 MiB
    buffer is overwritten between steps; the flush is outside the timed span)."""
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda:0")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for r in range(reps):
        scratch.fill_(r & 255)
        e0.record(pipe.stream)
        pipe.run()
        e1.record(pipe.stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del scratch
    times.sort()
    return {"ms_per_step_median": round(times[len(times) // 2], 5), "reps": reps,
            "flush_MiB": flush_bytes >> 20}


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
def cpu_baseline(inp, budget_rows):
    """The oracle, as it stands, on a bounded sample of the same workload."""
    import oracle as O
    cfg = inp["cfg"]
    dt = cfg["dtype"]
    t0 = time.perf_counter()
    B = cfg["B"]
    if cfg["kind"] == "decode":
        Tq = 1
        q_pos0, raw_pos0 = inp["q_pos0"], inp["raw_pos0"]
        rows = [(b, 0) for b in range(min(B, 2))]
        t_comp = 0.0
        hca = (inp["k_hca"], inp["v_hca"], cfg["m_hca"])
        kc, vc = inp["k_csa"], inp["v_csa"]
        kr, vr = inp["k_win"], inp["v_win"]
        total_q = B
    else:
        Tq = cfg["T"]
        q_pos0 = raw_pos0 = 0
        rng = np.random.default_rng(1)
        rows = sorted({(int(rng.integers(0, B)), int(rng.integers(0, Tq))) for _ in range(budget_rows)})
        hca = None
        kc = vc = None
        if cfg.get("m_hca"):
            kh, vh = O.compress_kv(inp["k"], inp["v"], inp["zk_hca"], inp["zv_hca"], cfg["m_hca"], dt)
            hca = (kh, vh, cfg["m_hca"])
        if cfg.get("m_csa"):
            kc, vc = O.compress_kv(inp["k"], inp["v"], inp["zk_csa"], inp["zv_csa"], cfg["m_csa"], dt)
        t_comp = time.perf_counter() - t0
        kr, vr = inp["k"], inp["v"]
        total_q = B * Tq
    t1 = time.perf_counter()
    csa = None
    if cfg.get("m_csa"):
        sel = O.index_topk(inp["qI"], inp["kI"], inp["w"], q_pos0, cfg["m_csa"], cfg["W"], cfg["k"], dt,
                           rows=rows)
        idx = np.full((B, Tq, cfg["k"]), -1, dtype=np.int32)
        for r, (b, i) in enumerate(rows):
            idx[b, i] = sel[r]
        csa = (kc, vc, idx)
    O.hybrid_attn_fwd(inp["q"], kr, vr, inp["gates"], W=cfg["W"], dtype=dt, q_pos0=q_pos0,
                      raw_pos0=raw_pos0, hca=hca, csa=csa, rows=rows)
    t_rows = time.perf_counter() - t1
    per_query = t_comp / total_q + t_rows / len(rows)
    return {"value": 1.0 / per_query, "unit": "queries/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(rows)} query rows (all heads, all branches, indexer + attention) "
                      f"plus the full K/V compression of the batch ({t_comp:.1f} s, charged "
                      f"per query); float64 NumPy, single thread; {t_comp + t_rows:.1f} s total"}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="tinyr2_bf16",
                    help="tinyr2_bf16 (default), tiny_fp32, hca_prefill_32k, csa_prefill_128k, decode_1m, "
                         "decode_append (cache maintenance), rope_q (RoPE on the query tensor), "
                         "quant4_hca (4-bit cache storage)")
    ap.add_argument("--gates", default=None, choices=["mix", "hca", "csa", "swa"],
                    help="override the workload's gate setting (one-hot modes or the U(0,1) mix)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the cache-flushed step timing and the measured-peak probes")
    ap.add_argument("--cpu-rows", type=int, default=10000,
                    help="query rows of the CPU-baseline sample (about 10-15 s of oracle work at the default workload)")
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
    log(f"[bench] building inputs for {args.workload}")
    inp = build_inputs(args.workload, gates=args.gates)
    cfg = inp["cfg"]
    pipe = make_pipeline(inp)
    names = pipe.names()
    stream = pipe.stream
    log(f"[bench] kernels per step: {names}; warmup {args.warmup}")
    for _ in range(args.warmup):
        pipe.run()
    torch.cuda.synchronize()
    alg = algorithmic(inp, pipe)

    # timed region: K steps, per-kernel HIP events on the pipeline's stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        pipe.run(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {wall * 1e3:.2f} ms")
    ktime = {n: 0.0 for n in names}
    for s in range(args.steps):
        for j, n in enumerate(names):
            ktime[n] += evs[s][j].elapsed_time(evs[s][j + 1])
    ktime = {n: v / args.steps for n, v in ktime.items()}   # ms per launch
    gpu_ms = sum(evs[s][0].elapsed_time(evs[s][-1]) for s in range(args.steps)) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    if cfg["kind"] == "decode":
        queries = cfg["B"]
    else:
        queries = cfg["B"] * cfg["T"]
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
    roof["traffic"] = traffic_for(dom, args.workload)

    # after the timed region: the same step with caches flushed, and the
    # measured device peaks (extra fields beside the headline)
    cold = cold_steps(torch, pipe) if not args.no_extras else None
    peaks = measure_peaks(torch, binding) if not args.no_extras else None
    if peaks is not None and (roof["unit"] == "GB/s" or dtype == "bf16"):
        roof["measured_peak"] = peaks["copy_GBps"] if roof["unit"] == "GB/s" else peaks["mfma_bf16_TFLOPs"]
        roof["frac_of_measured"] = round(roof["achieved"] / roof["measured_peak"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):   # the oracle runs on exactly one host thread
            cpu = cpu_baseline(inp, args.cpu_rows)
        log(f"[bench] cpu baseline {cpu['value']:.1f} queries/s")

    desc = {
        "tinyr2_bf16": "Tiny-R2 training-shape forward, B8 T2048 H=Hkv=12 d128 bf16, CSA m4 k64 "
                       "(indexer 4 heads d_idx 64), HCA m128, W128, gates U(0,1) (all branches)",
        "tiny_fp32": "tiny fp32 forward, B1 T256 H=Hkv=4 d64, CSA m4 k8 (indexer 2 heads), HCA m32, W32",
        "hca_prefill_32k": "HCA-only prefill, B1 T32768 H16 Hkv2 d128 bf16, m128, W128, gates [1,0,0]",
        "csa_prefill_128k": "CSA-only prefill, B1 T131072 H32 Hkv4 d128 bf16, m4, k512 (4 indexer heads), "
                            "W128, gates [0,1,0]",
        "decode_1m": "decode, B16 x 1 query at 1,048,576 context, H32 Hkv1 d128 bf16, CSA 262144 entries "
                     "k1024, HCA 8192 entries, W128, gates U(0,1)",
    }[args.workload]
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
        "config": {"workload": desc + ("" if args.gates is None else f" [gates: {args.gates}]"),
                   "name": args.workload, "gates": cfg.get("gates"), "batch": cfg["B"],
                   "query_rows": queries, "gpu_ms_per_step_events": round(gpu_ms, 5)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "cold": cold,
        "measured_peaks": peaks,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
