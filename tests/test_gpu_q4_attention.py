"""Attention over 4-bit compressed caches (cache_q4): the HCA and/or CSA K/V
caches are given as the codes and (min, step) the oracle's quant4 makes of
them, and decoded inside the attention's loads.

Two checks per case:
  * against the oracle: quant4 -> dequant4 of each cache, then the oracle's
    attention over those values (the 4-bit storage of [V4-code] section 1
    followed by the path), within the bf16 bar;
  * bit for bit against the same GPU attention fed the decoded caches in
    bf16 (the oracle's dequant4 values): the decode tables give exactly
    those values and everything after the loads is the same code.
Cases cover the split decode path (HCA stream items and CSA gathers), the
HCA prefill stream, the CSA dense-masked stream and the CSA prefill gather,
d 64 and 128, and one coded branch beside a bf16 one."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import assert_close, dev, host, lib

pytestmark = pytest.mark.gpu
BF16 = binding.DTYPE_BF16


def coded(cache):
    """(codes [B, N, Hkv, d/2] uint8, params float32 [2], decoded storage array)."""
    B, N, Hkv, d = cache.shape
    packed, mn, st = O.quant4(cache.reshape(-1), BF16)
    dec = O.dequant4(packed, mn, st, cache.size, BF16).reshape(cache.shape)
    return packed.reshape(B, N, Hkv, d // 2), np.array([mn, st], np.float32), dec


def run_case(q, kr, vr, gates, W, *, q_pos0, raw_pos0, hca, csa, q4_hca, q4_csa):
    """hca = (k, v, m) storage arrays, csa = (k, v, idx); returns (q4 output,
    bf16-decoded output, oracle output)."""
    kw_q4, kw_bf, o_hca, o_csa = {}, {}, None, None
    if hca is not None:
        kh, vh, m = hca
        if q4_hca:
            (ck, pk, dk), (cv, pv, dv) = coded(kh), coded(vh)
            kw_q4["hca"] = (dev(ck), dev(cv), m, (dev(pk), dev(pv)))
            kh, vh = dk, dv
        else:
            kw_q4["hca"] = (dev(kh), dev(vh), m)
        kw_bf["hca"] = (dev(kh), dev(vh), m)
        o_hca = (kh, vh, m)
    if csa is not None:
        kc, vc, idx = csa
        if q4_csa:
            (ck, pk, dk), (cv, pv, dv) = coded(kc), coded(vc)
            kw_q4["csa"] = (dev(ck), dev(cv), dev(idx), (dev(pk), dev(pv)))
            kc, vc = dk, dv
        else:
            kw_q4["csa"] = (dev(kc), dev(vc), dev(idx))
        kw_bf["csa"] = (dev(kc), dev(vc), dev(idx))
        o_csa = (kc, vc, idx)
    args = (dev(q), dev(kr), dev(vr), dev(gates), W)
    got = host(binding.hybrid_sparse_attn_fwd(*args, q_pos0=q_pos0, raw_pos0=raw_pos0, **kw_q4))
    ref = host(binding.hybrid_sparse_attn_fwd(*args, q_pos0=q_pos0, raw_pos0=raw_pos0, **kw_bf))
    want = O.hybrid_attn_fwd(q, kr, vr, gates, W=W, dtype=BF16, q_pos0=q_pos0, raw_pos0=raw_pos0, hca=o_hca,
                             csa=o_csa)
    return got, ref, want


@pytest.mark.parametrize("q4_hca,q4_csa", [(True, True), (True, False), (False, True)])
def test_q4_decode_split(q4_hca, q4_csa):
    lib()
    inp = synth.make_inputs("decode_1m", seed=80, B=3, N_csa=16384, N_hca=512, k=448)
    cfg = inp["cfg"]
    idx = O.index_topk(inp["qI"], inp["kI"], inp["w"], inp["q_pos0"], cfg["m_csa"], cfg["W"], cfg["k"], BF16)
    args = binding.make_fwd_args(dev(inp["q"]), dev(inp["k_win"]), dev(inp["v_win"]), dev(inp["gates"]), cfg["W"],
                                 q_pos0=inp["q_pos0"], raw_pos0=inp["raw_pos0"],
                                 hca=(dev(inp["k_hca"]), dev(inp["v_hca"]), cfg["m_hca"]),
                                 csa=(dev(inp["k_csa"]), dev(inp["v_csa"]), dev(idx)))[0]
    assert binding.hybrid_sparse_attn_fwd_workspace_size(args) > 0          # the split decode launch
    got, ref, want = run_case(inp["q"], inp["k_win"], inp["v_win"], inp["gates"], cfg["W"], q_pos0=inp["q_pos0"],
                              raw_pos0=inp["raw_pos0"], hca=(inp["k_hca"], inp["v_hca"], cfg["m_hca"]),
                              csa=(inp["k_csa"], inp["v_csa"], idx), q4_hca=q4_hca, q4_csa=q4_csa)
    assert np.array_equal(got, ref)
    assert_close(got, want, f"q4 decode hca={q4_hca} csa={q4_csa}")


@pytest.mark.parametrize("d,G", [(128, 8), (64, 2)])
def test_q4_prefill_hca_stream(d, G):
    lib()
    inp = synth.make_inputs("hca_prefill_32k", seed=81, T=1152, H=2 * G, Hkv=2, d=d, gates="mix")
    cfg = inp["cfg"]
    kh, vh = O.compress_kv(inp["k"], inp["v"], inp["zk_hca"], inp["zv_hca"], cfg["m_hca"], BF16)
    got, ref, want = run_case(inp["q"], inp["k"], inp["v"], inp["gates"], cfg["W"], q_pos0=0, raw_pos0=0,
                              hca=(kh, vh, cfg["m_hca"]), csa=None, q4_hca=True, q4_csa=False)
    assert np.array_equal(got, ref)
    assert_close(got, want, f"q4 HCA prefill d={d} G={G}")


@pytest.mark.parametrize("H,Hkv,d", [(4, 4, 64), (16, 2, 128)])
def test_q4_prefill_csa(H, Hkv, d):
    # (4, 4, 64): G = 1, the dense-masked CSA stream; (16, 2, 128): G = 8, the gather
    lib()
    inp = synth.make_inputs("tiny_fp32", seed=82, dtype=BF16, T=320, H=H, Hkv=Hkv, d=d, k=12)
    cfg = inp["cfg"]
    m = cfg["m_csa"]
    kc, vc = O.compress_kv(inp["k"], inp["v"], inp["zk_csa"], inp["zv_csa"], m, BF16)
    kh, vh = O.compress_kv(inp["k"], inp["v"], inp["zk_hca"], inp["zv_hca"], cfg["m_hca"], BF16)
    idx = O.index_topk(inp["qI"], inp["kI"], inp["w"], 0, m, cfg["W"], cfg["k"], BF16)
    got, ref, want = run_case(inp["q"], inp["k"], inp["v"], inp["gates"], cfg["W"], q_pos0=0, raw_pos0=0,
                              hca=(kh, vh, cfg["m_hca"]), csa=(kc, vc, idx), q4_hca=True, q4_csa=True)
    assert np.array_equal(got, ref)
    assert_close(got, want, f"q4 CSA prefill H={H} Hkv={Hkv} d={d}")


def test_q4_rejected_outside_bf16():
    lib()
    z = lambda *s, dt=torch.float32: torch.zeros(s, dtype=dt, device="cuda:0")
    p = z(2)
    with pytest.raises(binding.ShattnError) as e:
        binding.hybrid_sparse_attn_fwd(z(1, 4, 2, 64), z(1, 4, 1, 64), z(1, 4, 1, 64), z(2, 3), 4,
                                       hca=(z(1, 2, 1, 32, dt=torch.uint8), z(1, 2, 1, 32, dt=torch.uint8), 1,
                                            (p, p)))
    assert e.value.code == binding.SHATTN_EUNSUPPORTED
