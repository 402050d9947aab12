"""GPU parity of csa_index_topk against the oracle's float64 indexer + top-k.

The bar is bit-exact index rows: the kernel re-scores every candidate inside
the float32 error band of the k-th score in float64, so its selection must be
the one the float64 oracle makes (equal-score ties broken by lower index)."""
import numpy as np
import pytest

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import dev, host, lib

pytestmark = pytest.mark.gpu


def gpu_topk(qI, kI, w, q_pos0, m, W, k):
    return host(binding.csa_index_topk(dev(qI), dev(kI), dev(w), q_pos0, m, W, k))


def oracle_rows(qI, kI, w, q_pos0, m, W, k, dt, rows):
    return O.index_topk(qI, kI, w, q_pos0, m, W, k, dt, rows=rows)


def assert_rows_equal(got, want, rows, what):
    bad = [r for r, (g, w_) in enumerate(zip(got, want)) if not np.array_equal(g, w_)]
    assert not bad, f"{what}: {len(bad)} of {len(rows)} rows differ; first row {rows[bad[0]]}: " \
                    f"gpu {got[bad[0]][:12]} oracle {want[bad[0]][:12]}"


def run_case(inp, q_pos0=0, rows=None, what=""):
    cfg = inp["cfg"]
    m, W, k, dt = cfg["m_csa"], cfg["W"], cfg["k"], cfg["dtype"]
    got = gpu_topk(inp["qI"], inp["kI"], inp["w"], q_pos0, m, W, k)
    B, Tq = got.shape[:2]
    if rows is None:
        rows = [(b, i) for b in range(B) for i in range(Tq)]
    want = oracle_rows(inp["qI"], inp["kI"], inp["w"], q_pos0, m, W, k, dt, rows)
    assert_rows_equal([got[b, i] for b, i in rows], want, rows, what)
    return got


def test_tiny_fp32_all_rows():
    lib()
    run_case(synth.make_inputs("tiny_fp32", seed=0), what="tiny fp32")


def test_tinyr2_full_all_rows():
    lib()
    run_case(synth.make_inputs("tinyr2_bf16", seed=0), what="tinyr2 full")


# Hi=16, d_idx=128 on the dense (N <= 2048) kernel: one build of that kernel
# took a GPU memory fault on this case; the cause is not identified, the
# kernel is back to its earlier form, and the case stays skipped until the
# cause is shown.  The dense kernel is no longer built for Hi = 16: such
# inputs take the list pipeline, which test_hi16_short_candidate_sets covers
# at N <= 2048 for d_idx 64 and 128.
DENSE_16_128_FAULT = "dense kernel Hi=16 d_idx=128: memory fault with one build, cause not identified"


@pytest.mark.parametrize("Hi,d_idx", [(1, 64), (2, 128), (8, 64),
                                      pytest.param(16, 128, marks=pytest.mark.skip(reason=DENSE_16_128_FAULT))])
def test_head_counts(Hi, d_idx):
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=10 + Hi, B=2, T=700, Hi=Hi, d_idx=d_idx, k=40)
    run_case(inp, what=f"Hi={Hi} d_idx={d_idx}")


@pytest.mark.parametrize("d_idx", [64, 128])
def test_hi16_short_candidate_sets(d_idx):
    # Hi = 16 with N <= 2048 takes the long pipeline (sampling at four row
    # tiles per wave, filter, list selection), never the dense kernel
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=40 + d_idx, B=2, T=650, Hi=16, d_idx=d_idx, k=33)
    run_case(inp, what=f"Hi=16 d_idx={d_idx} N<=2048")


@pytest.mark.parametrize("Hi", [4, 16])
def test_no_candidates(Hi):
    # N = 0: every row is -1
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=50 + Hi, B=2, T=64, Hi=Hi, d_idx=64, k=12)
    got = gpu_topk(inp["qI"], inp["kI"][:, :0], inp["w"], 0, 4, 128, 12)
    assert got.shape == (2, 64, 12) and (got == -1).all()


def test_dense_two_row_tiles_per_wave():
    # 32768 query rows: the dense plan gives each wave 8 queries (two row
    # tiles of 4 queries x 4 heads), the per-wave scoring path; smaller row
    # counts give one row tile per wave and the workgroup-cooperative path
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=21, B=16)
    B, T = inp["qI"].shape[:2]
    rows = [(b, i) for b in range(B) for i in range(b % 7, T, 37)] + [(b, T - 1) for b in range(B)]
    run_case(inp, rows=rows, what="two row tiles per wave")


def test_fp32_small_ragged():
    lib()
    inp = synth.make_inputs("tiny_fp32", seed=11, T=203, k=5, W=9, m_hca=8)
    run_case(inp, what="fp32 ragged")


def test_all_zero_scores_tie_break():
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=12, B=1, T=600, k=16)
    # qI <= 0 and kI >= 0 elementwise: every dot <= 0, every score exactly 0
    q = O.bf16_bits_to_f64(inp["qI"])
    kk = O.bf16_bits_to_f64(inp["kI"])
    inp["qI"] = O.f64_to_bf16_bits(-np.abs(q))
    inp["kI"] = O.f64_to_bf16_bits(np.abs(kk))
    got = run_case(inp, what="all-zero ties")
    for i in range(600):
        nv = O.visible_count(i, 128, 4, 150)
        kk_ = min(16, nv)
        assert got[0, i, :kk_].tolist() == list(range(kk_))


def test_duplicate_keys_tie_break():
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=13, B=1, T=1200, k=20)
    kI = inp["kI"].copy()
    kI[:, 1::3] = kI[:, 0:-1:3][:, : kI[:, 1::3].shape[1]]   # entries 3j+1 duplicate 3j
    inp["kI"] = kI
    run_case(inp, what="duplicate keys")


def test_identical_keys_band_overflow():
    lib()
    # every candidate has the same score: the whole buffer sits in the error
    # band; ties go to the lowest indices
    inp = synth.make_inputs("tinyr2_bf16", seed=14, B=1, T=4000, k=30)
    inp["kI"] = np.ascontiguousarray(np.broadcast_to(inp["kI"][:, :1], inp["kI"].shape))
    run_case(inp, what="identical keys")


def test_k_at_least_visible():
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=15, B=1, T=900, k=300)
    run_case(inp, what="k >= visible")


def sampled_rows(B, T, n, seed):
    rng = np.random.default_rng(seed)
    rows = {(b, t) for b in range(B) for t in (0, 127, 128, 131, T // 2, T - 1)}
    while len(rows) < n:
        rows.add((int(rng.integers(0, B)), int(rng.integers(0, T))))
    return sorted(rows)


# Above 2048 entries prefill takes the long pipeline: a threshold from every
# S-th entry, per-query lists of the entries above it, the exact selection over
# each list, and the streaming kernel (bounded per-query buffers with
# compactions) for the queries whose list cannot decide.  The cases below
# repeat the small-N checks on that path (N = T / 4 > 2048).
@pytest.mark.parametrize("Hi,d_idx", [(1, 64), (2, 128), (4, 64), (4, 128), (8, 64), (8, 128), (16, 128)])
def test_streaming_head_counts(Hi, d_idx):
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=30 + Hi, B=2, T=8500, Hi=Hi, d_idx=d_idx, k=64)
    run_case(inp, rows=sampled_rows(2, 8500, 200, Hi), what=f"streaming Hi={Hi} d_idx={d_idx}")


def test_streaming_fp32_ragged():
    lib()
    inp = synth.make_inputs("tiny_fp32", seed=34, T=8403, k=37, W=9, m_hca=8)
    run_case(inp, rows=sampled_rows(1, 8403, 200, 34), what="streaming fp32 ragged")


def test_streaming_duplicate_and_identical_keys():
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=35, B=1, T=9000, k=20)
    kI = inp["kI"].copy()
    kI[:, 1::3] = kI[:, 0:-1:3][:, : kI[:, 1::3].shape[1]]
    inp["kI"] = kI
    run_case(inp, rows=sampled_rows(1, 9000, 150, 35), what="streaming duplicate keys")
    inp["kI"] = np.ascontiguousarray(np.broadcast_to(inp["kI"][:, :1], inp["kI"].shape))
    got = run_case(inp, rows=sampled_rows(1, 9000, 150, 36), what="streaming identical keys")
    assert got[0, 8999, :20].tolist() == list(range(20))


def test_long_prefill_periodic_structure_falls_back():
    """Keys at every 16th entry scaled by 8 dominate the scores.  The sampling
    stride divides 16, so the sampled threshold ranks only those entries and
    too few entries (about the threshold rank, below k) reach it: every query
    with more visible entries than its list holds is redone by the streaming
    kernel.  The rows must still be the oracle's."""
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=37, B=1, T=9000, k=64)
    kI = inp["kI"].copy()
    f = (kI[:, ::16].astype(np.uint32) << np.uint32(16)).view(np.float32) * np.float32(8.0)
    kI[:, ::16] = synth.f32_to_bf16_bits(f)
    inp["kI"] = kI
    run_case(inp, rows=sampled_rows(1, 9000, 200, 37), what="periodic structure")


def test_csa_prefill_reduced_all_rows():
    lib()
    inp = synth.make_inputs("csa_prefill_128k", seed=16, T=8192)
    run_case(inp, what="csa prefill 8k")


def test_csa_prefill_full_sampled():
    lib()
    inp = synth.make_inputs("csa_prefill_128k", seed=0)
    rng = np.random.default_rng(0)
    T = inp["qI"].shape[1]
    rows = sorted({(0, int(t)) for t in rng.integers(0, T, 40)} | {(0, T - 1), (0, 127 + 4 * 600), (0, 130)})
    run_case(inp, rows=rows, what="csa prefill 128k sampled")


def test_decode_full():
    lib()
    inp = synth.make_inputs("decode_1m", seed=0)
    cfg = inp["cfg"]
    got = gpu_topk(inp["qI"], inp["kI"], inp["w"], inp["q_pos0"], cfg["m_csa"], cfg["W"], cfg["k"])
    rows = [(b, 0) for b in range(cfg["B"])]
    want = oracle_rows(inp["qI"], inp["kI"], inp["w"], inp["q_pos0"], cfg["m_csa"], cfg["W"], cfg["k"],
                       cfg["dtype"], rows)
    assert_rows_equal([got[b, 0] for b, _ in rows], want, rows, "decode 1M")


def test_decode_ragged_chunks():
    lib()
    inp = synth.make_inputs("decode_1m", seed=17, B=3, N_csa=10000, N_hca=64, k=100)
    cfg = inp["cfg"]
    got = gpu_topk(inp["qI"], inp["kI"], inp["w"], inp["q_pos0"], cfg["m_csa"], cfg["W"], cfg["k"])
    rows = [(b, 0) for b in range(3)]
    want = oracle_rows(inp["qI"], inp["kI"], inp["w"], inp["q_pos0"], cfg["m_csa"], cfg["W"], cfg["k"],
                       cfg["dtype"], rows)
    assert_rows_equal([got[b, 0] for b, _ in rows], want, rows, "decode ragged")


def test_decode_identical_keys_list_overflow():
    # every score of a row ties: every chunk's candidate list overflows, the
    # final pass streams whole chunks and the lowest indices win
    lib()
    inp = synth.make_inputs("decode_1m", seed=19, B=2, N_csa=10000, N_hca=64, k=100)
    inp["kI"] = np.ascontiguousarray(np.broadcast_to(inp["kI"][:, :1], inp["kI"].shape))
    cfg = inp["cfg"]
    got = gpu_topk(inp["qI"], inp["kI"], inp["w"], inp["q_pos0"], cfg["m_csa"], cfg["W"], cfg["k"])
    rows = [(b, 0) for b in range(2)]
    want = oracle_rows(inp["qI"], inp["kI"], inp["w"], inp["q_pos0"], cfg["m_csa"], cfg["W"], cfg["k"],
                       cfg["dtype"], rows)
    assert_rows_equal([got[b, 0] for b, _ in rows], want, rows, "decode identical keys")
    assert got[0, 0].tolist() == list(range(100))


def test_indexer_deterministic():
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=18, B=2, T=1024)
    a = gpu_topk(inp["qI"], inp["kI"], inp["w"], 0, 4, 128, 64)
    b = gpu_topk(inp["qI"], inp["kI"], inp["w"], 0, 4, 128, 64)
    assert np.array_equal(a, b)
