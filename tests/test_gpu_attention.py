"""GPU parity of hybrid_sparse_attn_fwd against the oracle's gated attention.

Compressed caches and CSA selections fed to the kernel come from the oracle
(never from the HIP path), so this isolates the attention kernel."""
import numpy as np
import pytest

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import assert_close, dev, host, lib

pytestmark = pytest.mark.gpu


def prefill_case(name, seed=0, gates=None, branches=("hca", "csa"), **over):
    inp = synth.make_inputs(name, seed=seed, **over)
    cfg = inp["cfg"]
    dt = cfg["dtype"]
    if gates is not None:
        inp["gates"] = np.tile(np.asarray(gates, np.float32), (cfg["H"], 1))
    hca = csa = None
    if "hca" in branches and cfg.get("m_hca"):
        kh, vh = O.compress_kv(inp["k"], inp["v"], inp["zk_hca"], inp["zv_hca"], cfg["m_hca"], dt)
        hca = (kh, vh, cfg["m_hca"])
    if "csa" in branches and cfg.get("m_csa"):
        kc, vc = O.compress_kv(inp["k"], inp["v"], inp["zk_csa"], inp["zv_csa"], cfg["m_csa"], dt)
        idx = O.index_topk(inp["qI"], inp["kI"], inp["w"], 0, cfg["m_csa"], cfg["W"], cfg["k"], dt)
        csa = (kc, vc, idx)
    return inp, hca, csa


def gpu_attn(inp, hca, csa, q_pos0=0, raw_pos0=0, k_raw="k", v_raw="v", gate_mode=0):
    cfg = inp["cfg"]
    hca_d = None if hca is None else (dev(hca[0]), dev(hca[1]), hca[2])
    csa_d = None if csa is None else (dev(csa[0]), dev(csa[1]), dev(csa[2]))
    out = binding.hybrid_sparse_attn_fwd(dev(inp["q"]), dev(inp[k_raw]), dev(inp[v_raw]),
                                         dev(inp["gates"]), cfg["W"], q_pos0=q_pos0,
                                         raw_pos0=raw_pos0, hca=hca_d, csa=csa_d,
                                         gate_logits=gate_mode == 2)
    return host(out)


def sample_rows(B, T, W, n=96, seed=0):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, W - 2, W - 1, W, W + 1, 2 * W - 1, 2 * W, 63, 64, 65, T - 1, T - 2}
    rows = set()
    for b in range(B):
        for t in fixed:
            if 0 <= t < T:
                rows.add((b, t))
    while len(rows) < min(n + len(fixed) * B, B * T):
        rows.add((int(rng.integers(0, B)), int(rng.integers(0, T))))
    return sorted(rows)


def check(inp, hca, csa, got, rows=None, q_pos0=0, raw_pos0=0, k_raw="k", v_raw="v", what="",
          gate_mode=0):
    cfg = inp["cfg"]
    want = O.hybrid_attn_fwd(inp["q"], inp[k_raw], inp[v_raw], inp["gates"], W=cfg["W"],
                             dtype=cfg["dtype"], q_pos0=q_pos0, raw_pos0=raw_pos0, hca=hca,
                             csa=csa, rows=rows, gate_mode=gate_mode)
    if rows is not None:
        got = np.stack([got[b, i] for b, i in rows])
    return assert_close(got, want, what)


@pytest.mark.parametrize("gates", [[1, 0, 0], [0, 1, 0], [0, 0, 1], None])
def test_tiny_fp32_all_rows(gates):
    lib()
    inp, hca, csa = prefill_case("tiny_fp32", gates=gates)
    got = gpu_attn(inp, hca, csa)
    check(inp, hca, csa, got, what=f"tiny gates={gates}")


@pytest.mark.parametrize("gates", [[1, 0, 0], [0, 1, 0], [0, 0, 1], None])
def test_tinyr2_reduced(gates):
    lib()
    inp, hca, csa = prefill_case("tinyr2_bf16", gates=gates, seed=1, B=2, T=640)
    got = gpu_attn(inp, hca, csa)
    check(inp, hca, csa, got, rows=sample_rows(2, 640, 128), what=f"tinyr2 gates={gates}")


@pytest.mark.parametrize("mode,kind", [(1, "weights"), (2, "logits")])
def test_per_token_gates_tiny_fp32_all_rows(mode, kind):
    lib()
    inp, hca, csa = prefill_case("tiny_fp32", seed=3)
    cfg = inp["cfg"]
    inp["gates"] = synth.token_gates(cfg["B"], cfg["T"], cfg["H"], kind, seed=50 + mode)
    got = gpu_attn(inp, hca, csa, gate_mode=mode)
    check(inp, hca, csa, got, what=f"tiny per-token gates mode {mode}", gate_mode=mode)


@pytest.mark.parametrize("mode,kind", [(1, "weights"), (2, "logits")])
def test_per_token_gates_tinyr2_reduced(mode, kind):
    lib()
    inp, hca, csa = prefill_case("tinyr2_bf16", seed=4, B=2, T=640)
    inp["gates"] = synth.token_gates(2, 640, inp["cfg"]["H"], kind, seed=60 + mode)
    got = gpu_attn(inp, hca, csa, gate_mode=mode)
    check(inp, hca, csa, got, rows=sample_rows(2, 640, 128, seed=5), what=f"tinyr2 per-token gates mode {mode}",
          gate_mode=mode)


def test_per_token_gate_logits_gqa_ragged():
    # several query heads per KV head: the gate of column (query, head) uses
    # the query head, not the KV head
    lib()
    inp, hca, csa = prefill_case("tinyr2_bf16", seed=6, B=2, T=333, H=16, Hkv=2)
    inp["gates"] = synth.token_gates(2, 333, 16, "logits", seed=80)
    got = gpu_attn(inp, hca, csa, gate_mode=2)
    check(inp, hca, csa, got, rows=sample_rows(2, 333, 128, seed=7), what="GQA per-token gate logits",
          gate_mode=2)


def test_gqa_hca_prefill_reduced():
    lib()
    inp, hca, csa = prefill_case("hca_prefill_32k", seed=2, T=2048)
    got = gpu_attn(inp, hca, csa)
    check(inp, hca, csa, got, rows=sample_rows(1, 2048, 128, n=64), what="hca gqa")


def test_gqa_csa_gather_reduced():
    lib()
    inp, hca, csa = prefill_case("csa_prefill_128k", seed=3, T=4096, k=96)
    got = gpu_attn(inp, hca, csa)
    check(inp, hca, csa, got, rows=sample_rows(1, 4096, 128, n=64), what="csa gqa gather")


def test_all_branches_gqa_ragged():
    # G = 3 (non power of two), T not a multiple of any tile, small window
    lib()
    inp, hca, csa = prefill_case("tinyr2_bf16", seed=4, B=1, T=333, H=6, Hkv=2, d=64, W=16,
                                 m_hca=8, k=12)
    got = gpu_attn(inp, hca, csa)
    check(inp, hca, csa, got, what="ragged G=3")


def test_short_sequence_and_window_one():
    lib()
    inp, hca, csa = prefill_case("tinyr2_bf16", seed=5, B=2, T=40, W=1, m_hca=4, k=3)
    got = gpu_attn(inp, hca, csa)
    check(inp, hca, csa, got, what="W=1")
    inp, hca, csa = prefill_case("tinyr2_bf16", seed=6, B=1, T=100, W=128)   # T < W
    got = gpu_attn(inp, hca, csa)
    check(inp, hca, csa, got, what="T<W")


def test_csa_gather_many_heads_per_group():
    # G = 16: one query per wave in the gather path
    lib()
    inp, hca, csa = prefill_case("csa_prefill_128k", seed=7, T=1024, H=32, Hkv=2, k=40)
    got = gpu_attn(inp, hca, csa)
    check(inp, hca, csa, got, rows=sample_rows(1, 1024, 128, n=48), what="G=16 gather")


@pytest.mark.parametrize("H,Hkv,T,k", [(16, 4, 2048, 37), (8, 4, 2048, 30), (4, 4, 1024, 13)])
def test_csa_gather_several_queries_per_wave(H, Hkv, T, k):
    # G = 4, 2, 1: a wave's 16 columns hold 4, 8 or 16 queries, and it walks
    # each query's selection in turn (k not a multiple of 4 takes the gather
    # instead of the dense-masked stream; ragged last chunks)
    lib()
    inp, hca, csa = prefill_case("csa_prefill_128k", seed=18, T=T, H=H, Hkv=Hkv, k=k)
    got = gpu_attn(inp, hca, csa)
    check(inp, hca, csa, got, rows=sample_rows(1, T, 128, n=48), what=f"gather G={H // Hkv}")


def test_csa_gather_d64():
    # the direct-to-LDS gather tiles at d = 64 (8 rows per wave load)
    lib()
    inp, hca, csa = prefill_case("csa_prefill_128k", seed=11, T=2048, d=64, k=64)
    got = gpu_attn(inp, hca, csa)
    check(inp, hca, csa, got, rows=sample_rows(1, 2048, 128, n=64), what="csa gather d=64")


def test_gather_with_no_cache_entries():
    # T < m: the CSA branch is present (G = 8: gather mode) but its cache holds
    # no entry; the branch is its window-only attention
    lib()
    inp, hca, csa = prefill_case("csa_prefill_128k", seed=13, T=3, W=2, k=8)
    assert csa[0].shape[1] == 0
    got = gpu_attn(inp, hca, csa)
    check(inp, hca, csa, got, what="empty CSA cache")


def with_holes(idx, N, seed):
    """The selection with entries knocked out mid-row: -1 (padding), other
    negative values and values >= N, all of which the kernel ignores (the
    attention's contract: only entries with 0 <= idx < N_csa are attended).
    Returns (what the kernel gets, what the oracle gets: the same rows with
    every ignored entry as -1)."""
    rng = np.random.default_rng(seed)
    bad = idx.copy()
    u = rng.random(idx.shape)
    bad[u < 0.2] = -1
    bad[(u >= 0.2) & (u < 0.25)] = -7
    bad[(u >= 0.25) & (u < 0.3)] = N + 3
    bad[(u >= 0.3) & (u < 0.32)] = np.iinfo(np.int32).max
    clean = bad.copy()
    clean[(clean < 0) | (clean >= N)] = -1
    return bad, clean


@pytest.mark.parametrize("case", ["gather", "dense_masked", "gather_d64"])
def test_csa_entries_outside_the_cache_are_ignored(case):
    # prefill: the per-wave gather (G = 8) and the selection bitmap of the
    # dense-masked stream (G = 1, small cache)
    lib()
    if case == "gather":
        inp, hca, csa = prefill_case("csa_prefill_128k", seed=14, T=1536, k=72)
    elif case == "gather_d64":
        inp, hca, csa = prefill_case("csa_prefill_128k", seed=16, T=1024, d=64, k=40)
    else:
        inp, hca, csa = prefill_case("tinyr2_bf16", seed=15, B=1, T=700, k=24)
    kc, vc, idx = csa
    bad, clean = with_holes(idx, kc.shape[1], seed=20)
    got = gpu_attn(inp, hca, (kc, vc, bad))
    rows = sample_rows(1, inp["cfg"]["T"], inp["cfg"]["W"], n=48) if case != "dense_masked" else None
    check(inp, hca, (kc, vc, clean), got, rows=rows, what=f"holes {case}")


def test_decode_split_entries_outside_the_cache_are_ignored():
    lib()
    inp, hca, csa = decode_case(seed=17, B=3, N_csa=4096, N_hca=512, k=200)
    kc, vc, idx = csa
    bad, clean = with_holes(idx, kc.shape[1], seed=21)
    got = gpu_attn(inp, hca, (kc, vc, bad), q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"],
                   k_raw="k_win", v_raw="v_win")
    check(inp, hca, (kc, vc, clean), got, q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"], k_raw="k_win",
          v_raw="v_win", what="decode split holes")


def decode_case(seed=0, **over):
    inp = synth.make_inputs("decode_1m", seed=seed, **over)
    cfg = inp["cfg"]
    # selections from the oracle indexer over the whole cache
    idx = O.index_topk(inp["qI"], inp["kI"], inp["w"], inp["q_pos0"], cfg["m_csa"], cfg["W"],
                       cfg["k"], cfg["dtype"])
    hca = (inp["k_hca"], inp["v_hca"], cfg["m_hca"])
    csa = (inp["k_csa"], inp["v_csa"], idx)
    return inp, hca, csa


def test_decode_split_reduced():
    lib()
    inp, hca, csa = decode_case(seed=8, B=3, N_csa=4096, N_hca=2048, k=300)
    got = gpu_attn(inp, hca, csa, q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"],
                   k_raw="k_win", v_raw="v_win")
    check(inp, hca, csa, got, q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"], k_raw="k_win",
          v_raw="v_win", what="decode split")


def test_decode_split_d64():
    lib()
    inp, hca, csa = decode_case(seed=12, B=2, N_csa=2048, N_hca=512, k=128, d=64)
    got = gpu_attn(inp, hca, csa, q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"],
                   k_raw="k_win", v_raw="v_win")
    check(inp, hca, csa, got, q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"], k_raw="k_win",
          v_raw="v_win", what="decode split d=64")


def test_decode_split_per_token_gate_logits():
    lib()
    inp, hca, csa = decode_case(seed=13, B=3, N_csa=4096, N_hca=2048, k=300)
    cfg = inp["cfg"]
    inp["gates"] = synth.token_gates(cfg["B"], 1, cfg["H"], "logits", seed=70)
    got = gpu_attn(inp, hca, csa, q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"], k_raw="k_win",
                   v_raw="v_win", gate_mode=2)
    check(inp, hca, csa, got, q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"], k_raw="k_win",
          v_raw="v_win", what="decode split, per-token gate logits", gate_mode=2)


def test_decode_full_size():
    lib()
    inp, hca, csa = decode_case(seed=0)
    got = gpu_attn(inp, hca, csa, q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"],
                   k_raw="k_win", v_raw="v_win")
    check(inp, hca, csa, got, q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"], k_raw="k_win",
          v_raw="v_win", what="decode 1M")


def test_attention_deterministic_and_constant_values():
    lib()
    inp, hca, csa = prefill_case("tinyr2_bf16", seed=9, B=1, T=512)
    a = gpu_attn(inp, hca, csa)
    b = gpu_attn(inp, hca, csa)
    assert np.array_equal(a, b)
    # V = constant row everywhere => out = (sum of gates) * row
    row = synth.f32_to_bf16_bits(np.linspace(-1, 1, 128).astype(np.float32))
    inp["v"] = np.ascontiguousarray(np.broadcast_to(row, inp["v"].shape))
    cfg = inp["cfg"]
    kh, vh = O.compress_kv(inp["k"], inp["v"], inp["zk_hca"], inp["zv_hca"], cfg["m_hca"], cfg["dtype"])
    kc, vc = O.compress_kv(inp["k"], inp["v"], inp["zk_csa"], inp["zv_csa"], cfg["m_csa"], cfg["dtype"])
    got = gpu_attn(inp, (kh, vh, cfg["m_hca"]), (kc, vc, csa[2]))
    vrow = O.bf16_bits_to_f64(row)
    g = inp["gates"].astype(np.float64)
    for b_, i in [(0, 0), (0, 200), (0, 511)]:
        t = i
        # every branch is present (HCA and CSA gates nonzero); a branch with
        # no visible entries still attends its window, so each contributes
        # gate * row whatever the position
        gsum = g[:, 0] + g[:, 1] + g[:, 2]
        want = gsum[:, None] * vrow[None, :]
        # compressed constant rows round to the same bf16 value, so every branch averages `row`
        np.testing.assert_allclose(O.bf16_bits_to_f64(got[b_, i]), want, rtol=2e-2, atol=2e-2)
