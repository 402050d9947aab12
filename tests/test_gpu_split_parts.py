"""The attention in two calls on one workspace (split_part): 1 = the window
and HCA items, 2 = the CSA items and the merge.  The same kernels run the
same items, so the result must equal the single call bit for bit: on split
decode shapes (with and without CSA entries), for a prefill (no split: call
1 writes nothing, call 2 does it all), and through the pipeline with the
first call on a second stream beside the indexer."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import dev, host, lib

pytestmark = pytest.mark.gpu


def two_calls(args, kw):
    L = lib()
    a0, out0, k0 = binding.make_fwd_args(*args, **kw)
    nbytes = binding.hybrid_sparse_attn_fwd_workspace_size(a0)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda:0")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    wsp = ctypes.c_void_p(ws.data_ptr()) if nbytes else None
    binding._check(L.hybrid_sparse_attn_fwd(ctypes.byref(a0), wsp, nbytes, s))
    full = host(out0)
    out = torch.full_like(out0, 7.0)
    a1, _, k1 = binding.make_fwd_args(*args, out=out, split_part=1, **kw)
    a2, _, k2 = binding.make_fwd_args(*args, out=out, split_part=2, **kw)
    binding._check(L.hybrid_sparse_attn_fwd(ctypes.byref(a1), wsp, nbytes, s))
    after1 = host(out)
    binding._check(L.hybrid_sparse_attn_fwd(ctypes.byref(a2), wsp, nbytes, s))
    return nbytes, full, after1, host(out), host(torch.full_like(out0, 7.0))


def decode_args(seed, csa=True, **over):
    inp = synth.make_inputs("decode_1m", seed=seed, **over)
    cfg = inp["cfg"]
    kw = dict(q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"],
              hca=(dev(inp["k_hca"]), dev(inp["v_hca"]), cfg["m_hca"]))
    if csa:
        idx = O.index_topk(inp["qI"], inp["kI"], inp["w"], inp["q_pos0"], cfg["m_csa"], cfg["W"], cfg["k"],
                           cfg["dtype"])
        kw["csa"] = (dev(inp["k_csa"]), dev(inp["v_csa"]), dev(idx))
    return (dev(inp["q"]), dev(inp["k_win"]), dev(inp["v_win"]), dev(inp["gates"]), cfg["W"]), kw


@pytest.mark.parametrize("csa", [True, False])
def test_two_calls_equal_one_on_split_decode(csa):
    # without CSA the query sits later (N_csa sets its position), so that all
    # 1024 HCA entries are visible and the key count calls for the split
    args, kw = decode_args(60, csa=csa, B=3, N_csa=16384 if csa else 65536, N_hca=1024, k=512)
    nbytes, full, after1, got, sentinel = two_calls(args, kw)
    assert nbytes > 0                                   # the split launch
    assert np.array_equal(after1, sentinel)            # call 1 only writes partial states
    assert np.array_equal(got, full)


def test_two_calls_without_split():
    inp = synth.make_inputs("tiny_fp32", seed=61, dtype=binding.DTYPE_BF16, T=200)
    cfg = inp["cfg"]
    kh, vh = O.compress_kv(inp["k"], inp["v"], inp["zk_hca"], inp["zv_hca"], cfg["m_hca"], cfg["dtype"])
    args = (dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["gates"]), cfg["W"])
    nbytes, full, after1, got, sentinel = two_calls(args, dict(hca=(dev(kh), dev(vh), cfg["m_hca"])))
    assert nbytes == 0
    assert np.array_equal(after1, sentinel)            # call 1 does nothing
    assert np.array_equal(got, full)                   # call 2 does it all


def test_pipeline_overlap_equals_serial():
    lib()
    inp = synth.make_inputs("decode_1m", seed=62, B=4, N_csa=32768, N_hca=1024, k=1024)
    cfg = inp["cfg"]
    outs = []
    for overlap in (False, True):
        pipe = binding.HybridPipeline(q=dev(inp["q"]), gates=dev(inp["gates"]), W=cfg["W"], k_raw=dev(inp["k_win"]),
                                      v_raw=dev(inp["v_win"]), q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"],
                                      qI=dev(inp["qI"]), kI=dev(inp["kI"]), w=dev(inp["w"]), k=cfg["k"],
                                      m_csa=cfg["m_csa"], m_hca=cfg["m_hca"], k_csa=dev(inp["k_csa"]),
                                      v_csa=dev(inp["v_csa"]), k_hca=dev(inp["k_hca"]), v_hca=dev(inp["v_hca"]),
                                      overlap=overlap)
        assert (pipe.part1 is not None) == overlap
        for _ in range(3):
            out = pipe.run()
        torch.cuda.synchronize()
        outs.append(host(out))
    assert np.array_equal(outs[0], outs[1])
