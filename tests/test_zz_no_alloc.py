"""hybrid_sparse_attn_fwd_noalloc (the library's own per-GPU scratch array
instead of a caller workspace) against hybrid_sparse_attn_fwd on the same
arguments: two calls in a row, the second with a smaller problem, both on
decode shapes whose launch splits the key list (and so needs scratch), and
one prefill shape that needs none.  Results must be bitwise equal (same
kernels, same arithmetic)."""
import numpy as np
import pytest

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import dev, host, lib

pytestmark = pytest.mark.gpu


def decode_args(seed, **over):
    inp = synth.make_inputs("decode_1m", seed=seed, **over)
    cfg = inp["cfg"]
    # selections from the oracle indexer (inputs of the attention only)
    idx = O.index_topk(inp["qI"], inp["kI"], inp["w"], inp["q_pos0"], cfg["m_csa"], cfg["W"], cfg["k"],
                       cfg["dtype"])
    kw = dict(q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"],
              hca=(dev(inp["k_hca"]), dev(inp["v_hca"]), cfg["m_hca"]),
              csa=(dev(inp["k_csa"]), dev(inp["v_csa"]), dev(idx)))
    return (dev(inp["q"]), dev(inp["k_win"]), dev(inp["v_win"]), dev(inp["gates"]), cfg["W"]), kw


def both(args, kw):
    a = host(binding.hybrid_sparse_attn_fwd(*args, **kw))
    b = host(binding.hybrid_sparse_attn_fwd_noalloc(*args, **kw))
    return a, b


def test_noalloc_matches_workspace_entry_point_twice():
    lib()
    big = decode_args(70, B=4, N_csa=16384, N_hca=512, k=1024)
    small = decode_args(71, B=2, N_csa=8192, N_hca=256, k=768)
    q, kr, vr, g, W = big[0]
    a_big = binding.make_fwd_args(q, kr, vr, g, W, **big[1])[0]
    a_small = binding.make_fwd_args(*small[0], **small[1])[0]
    n_big = binding.hybrid_sparse_attn_fwd_workspace_size(a_big)
    n_small = binding.hybrid_sparse_attn_fwd_workspace_size(a_small)
    assert n_big > n_small > 0, (n_big, n_small)       # both take the split (scratch) path
    for args, kw in (big, small):
        a, b = both(args, kw)
        assert np.array_equal(a, b)


def test_noalloc_without_scratch_and_too_large():
    lib()
    # a prefill shape needs no scratch at all
    inp = synth.make_inputs("tinyr2_bf16", seed=72, B=1, T=384)
    cfg = inp["cfg"]
    kh, vh = O.compress_kv(inp["k"], inp["v"], inp["zk_hca"], inp["zv_hca"], cfg["m_hca"], cfg["dtype"])
    args = (dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["gates"]), cfg["W"])
    kw = dict(hca=(dev(kh), dev(vh), cfg["m_hca"]))
    assert binding.hybrid_sparse_attn_fwd_workspace_size(binding.make_fwd_args(*args, **kw)[0]) == 0
    a, b = both(args, kw)
    assert np.array_equal(a, b)
    # more partial states than the scratch array holds (32 sequences x 32768
    # HCA entries split into 130 items): a clear error, nothing launched
    import torch
    B, H, d, W, N = 32, 32, 128, 128, 32768
    z = lambda *shape: torch.zeros(shape, dtype=torch.bfloat16, device="cuda:0")
    args = (z(B, 1, H, d), z(B, W, 1, d), z(B, W, 1, d), torch.ones((H, 3), dtype=torch.float32, device="cuda:0"), W)
    kw = dict(q_pos0=N * 128 + W - 1, raw_pos0=N * 128, hca=(z(B, N, 1, d), z(B, N, 1, d), 128))
    assert binding.hybrid_sparse_attn_fwd_workspace_size(binding.make_fwd_args(*args, **kw)[0]) > 32 << 20
    with pytest.raises(binding.ShattnError) as e:
        binding.hybrid_sparse_attn_fwd_noalloc(*args, **kw)
    assert e.value.code == binding.SHATTN_EUNSUPPORTED and "scratch" in str(e.value)
