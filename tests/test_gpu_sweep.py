"""Seeded sweep of small random configurations through the whole GPU path
(compression, indexer, attention, as the pipeline launches them) against
the oracle on every row: head dims, head grouping, windows, block ratios
(fused and separate compression), k, indexer heads, both storage dtypes,
ragged lengths and sequences shorter than a block; and seeded decode
configurations through the split indexer and split attention."""
import numpy as np
import pytest

from sparse_hybrid_attention_amd import binding, synth
from gpu_util import assert_close, host, lib
from test_gpu_pipeline import oracle_pipeline, pipeline

pytestmark = pytest.mark.gpu


def random_config(i):
    rng = np.random.default_rng(1000 + i)
    pick = lambda xs: xs[int(rng.integers(0, len(xs)))]
    dtype = pick([binding.DTYPE_BF16, binding.DTYPE_F32])
    Hkv = pick([1, 2, 3])
    G = pick([1, 2, 4, 8])
    return dict(dtype=dtype, B=int(rng.integers(1, 3)), T=int(rng.integers(1, 260)), H=Hkv * G, Hkv=Hkv,
                d=pick([64, 128]), W=pick([1, 3, 16, 40, 128]), m_csa=pick([1, 2, 3, 4, 8]),
                k=pick([1, 5, 16, 33]), Hi=pick([1, 2, 4, 8]), d_idx=pick([64, 128]),
                m_hca=pick([4, 5, 8, 32, 128]), gates="mix")


# short prefills of few heads take two-wave attention workgroups (at most 32
# query-head columns per KV head); these pin that variant with the dense CSA
FIXED = {
    16: dict(dtype=binding.DTYPE_BF16, B=2, T=20, H=2, Hkv=2, d=128, W=8, m_csa=2, k=4, Hi=4, d_idx=64,
             m_hca=4, gates="mix"),
    17: dict(dtype=binding.DTYPE_BF16, B=3, T=7, H=8, Hkv=2, d=64, W=3, m_csa=1, k=3, Hi=2, d_idx=64,
             m_hca=2, gates="mix"),
}


@pytest.mark.parametrize("i", list(range(48)) + sorted(FIXED))
def test_random_config_matches_oracle(i):
    lib()
    over = FIXED[i] if i in FIXED else random_config(i)
    base = "tinyr2_bf16" if over["dtype"] == binding.DTYPE_BF16 else "tiny_fp32"
    inp = synth.make_inputs(base, seed=2000 + i, **over)
    pipe = pipeline(inp)
    out = host(pipe.run())
    B, T = over["B"], over["T"]
    rows = [(b, t) for b in range(B) for t in range(T)]
    want, sel = oracle_pipeline(inp, rows)
    got = np.stack([out[b, t] for b, t in rows])
    assert_close(got, want, f"config {i}: {over}")
    if sel is not None:
        idx = host(pipe.idx)
        bad = [r for r, (b, t) in enumerate(rows) if not np.array_equal(idx[b, t], sel[r])]
        assert not bad, f"config {i}: {len(bad)} index rows differ, first {rows[bad[0]]}"


def random_decode(i):
    rng = np.random.default_rng(3000 + i)
    pick = lambda xs: xs[int(rng.integers(0, len(xs)))]
    Hkv = pick([1, 2])
    G = pick([1, 4, 8, 32])
    return dict(B=int(rng.integers(1, 5)), H=Hkv * G, Hkv=Hkv, d=pick([64, 128]),
                N_csa=int(rng.integers(8192, 20000)), N_hca=int(rng.integers(0, 3000)),
                k=pick([64, 300, 1024]), Hi=pick([1, 4]), d_idx=pick([64, 128]))


@pytest.mark.parametrize("i", range(8))
def test_random_decode_matches_oracle(i):
    # decode shapes: the split indexer (scores per chunk, candidate lists, exact
    # final select) and the split attention with its combine kernel, two-wave
    # workgroups when a KV head serves at most 32 query heads
    import oracle as O
    from gpu_util import dev
    lib()
    over = random_decode(i)
    inp = synth.make_inputs("decode_1m", seed=4000 + i, **over)
    cfg = inp["cfg"]
    q_pos0, raw_pos0 = inp["q_pos0"], inp["raw_pos0"]
    want_idx = O.index_topk(inp["qI"], inp["kI"], inp["w"], q_pos0, cfg["m_csa"], cfg["W"], cfg["k"], cfg["dtype"])
    got_idx = host(binding.csa_index_topk(dev(inp["qI"]), dev(inp["kI"]), dev(inp["w"]), q_pos0, cfg["m_csa"],
                                          cfg["W"], cfg["k"]))
    assert np.array_equal(got_idx, want_idx), f"decode config {i}: {over}: index rows differ"
    hca = (inp["k_hca"], inp["v_hca"], cfg["m_hca"])
    csa = (inp["k_csa"], inp["v_csa"], want_idx)
    out = binding.hybrid_sparse_attn_fwd(dev(inp["q"]), dev(inp["k_win"]), dev(inp["v_win"]), dev(inp["gates"]),
                                         cfg["W"], q_pos0=q_pos0, raw_pos0=raw_pos0,
                                         hca=(dev(hca[0]), dev(hca[1]), hca[2]),
                                         csa=(dev(csa[0]), dev(csa[1]), dev(csa[2])))
    want = O.hybrid_attn_fwd(inp["q"], inp["k_win"], inp["v_win"], inp["gates"], W=cfg["W"], dtype=cfg["dtype"],
                             q_pos0=q_pos0, raw_pos0=raw_pos0, hca=hca, csa=csa)
    assert_close(host(out), want, f"decode config {i}: {over}")
