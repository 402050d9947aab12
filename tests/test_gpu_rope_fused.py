"""RoPE of the query fused into the attention's Q load (rope_q) against
  * the oracle: RoPE of q at each row's position (reading R10), then the
    oracle's attention, within the dtype's bar;
  * bit for bit, the GPU path in two launches: rope_apply on q, then the
    attention without rope_q (the fused rotation rounds exactly as
    rope_apply stores).
Prefill in bf16 (the Tiny-R2 split: the last 64 of 128 channels rotated)
and fp32 (the whole head), a rope range that starts mid-head, and decode at
per-sequence positions read from rings."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import assert_close, dev, host, lib

pytestmark = pytest.mark.gpu


def check(inp, rope, *, q_pos0=0, raw_pos0=0, hca=None, csa=None, q_pos=None, raw_ring=False, pos_rows=None,
          k_raw=None, v_raw=None):
    cfg = inp["cfg"]
    dt = cfg["dtype"]
    q = inp["q"]
    B, Tq, H, d = q.shape
    k_raw = inp["k"] if k_raw is None else k_raw
    v_raw = inp["v"] if v_raw is None else v_raw
    kw = dict(q_pos0=q_pos0, raw_pos0=raw_pos0, q_pos=None if q_pos is None else dev(q_pos), raw_ring=raw_ring,
              hca=None if hca is None else (dev(hca[0]), dev(hca[1]), hca[2]),
              csa=None if csa is None else (dev(csa[0]), dev(csa[1]), dev(csa[2])))
    args = (dev(k_raw), dev(v_raw), dev(inp["gates"]), cfg["W"])
    fused = host(binding.hybrid_sparse_attn_fwd(dev(q), *args, rope_q=rope, **kw))
    # two launches: rope_apply in place on a copy of q, then the plain attention
    qd = dev(q)
    pos = torch.from_numpy(np.ascontiguousarray(pos_rows)).to("cuda:0")
    binding.rope_apply(qd.view(B * Tq, H, d), pos, rope_off=rope[0], rope_dim=rope[1], base=rope[2])
    two = host(binding.hybrid_sparse_attn_fwd(qd, *args, **kw))
    assert np.array_equal(fused, two)
    qr = O.rope(q.reshape(B * Tq, H, d), pos_rows, rope_off=rope[0], rope_dim=rope[1], dtype=dt,
                base=rope[2]).reshape(q.shape)
    return fused, qr


def rows_pos(B, Tq, first):
    return (np.asarray(first, np.int64).reshape(B, 1) + np.arange(Tq, dtype=np.int64)[None, :]).reshape(-1)


@pytest.mark.parametrize("name,over,rope", [
    ("tinyr2_bf16", dict(B=2, T=320), (64, 64, 10000.0)),
    ("tiny_fp32", dict(), (0, 64, 10000.0)),
    ("tinyr2_bf16", dict(B=1, T=200, H=8, Hkv=2), (10, 36, 500.0)),
])
def test_rope_q_prefill(name, over, rope):
    lib()
    inp = synth.make_inputs(name, seed=90, **over)
    cfg = inp["cfg"]
    dt = cfg["dtype"]
    B, T = cfg["B"], cfg["T"]
    kh, vh = O.compress_kv(inp["k"], inp["v"], inp["zk_hca"], inp["zv_hca"], cfg["m_hca"], dt)
    kc, vc = O.compress_kv(inp["k"], inp["v"], inp["zk_csa"], inp["zv_csa"], cfg["m_csa"], dt)
    idx = O.index_topk(inp["qI"], inp["kI"], inp["w"], 0, cfg["m_csa"], cfg["W"], cfg["k"], dt)
    got, qr = check(inp, rope, hca=(kh, vh, cfg["m_hca"]), csa=(kc, vc, idx), pos_rows=rows_pos(B, T, [0] * B))
    want = O.hybrid_attn_fwd(qr, inp["k"], inp["v"], inp["gates"], W=cfg["W"], dtype=dt, hca=(kh, vh, cfg["m_hca"]),
                             csa=(kc, vc, idx))
    assert_close(got, want, f"fused RoPE {name} {rope}")


def test_rope_q_decode_per_sequence_positions():
    # three sequences at different positions, one query each; the raw window
    # is a ring (position t in row t % Tr)
    lib()
    inp = synth.make_inputs("decode_1m", seed=91, B=3, N_csa=2048, N_hca=64, k=64)
    cfg = inp["cfg"]
    B, W = cfg["B"], cfg["W"]
    pos = np.array([8191, 3000, 5321], np.int64)
    # ring rows: the window of each sequence, written at row t % W
    k_ring = np.empty_like(inp["k_win"])
    v_ring = np.empty_like(inp["v_win"])
    for b in range(B):
        for j in range(W):
            t = pos[b] - W + 1 + j
            k_ring[b, t % W] = inp["k_win"][b, j]
            v_ring[b, t % W] = inp["v_win"][b, j]
    idx = np.concatenate([O.index_topk(inp["qI"][b:b + 1], inp["kI"][b:b + 1], inp["w"][b:b + 1], int(pos[b]),
                                       cfg["m_csa"], W, cfg["k"], cfg["dtype"]) for b in range(B)])
    rope = (64, 64, 10000.0)
    got, qr = check(inp, rope, q_pos=pos, raw_ring=True, hca=(inp["k_hca"], inp["v_hca"], cfg["m_hca"]),
                    csa=(inp["k_csa"], inp["v_csa"], idx), pos_rows=pos, k_raw=k_ring, v_raw=v_ring)
    for b in range(B):
        want = O.hybrid_attn_fwd(qr[b:b + 1], inp["k_win"][b:b + 1], inp["v_win"][b:b + 1], inp["gates"], W=W,
                                 dtype=cfg["dtype"], q_pos0=int(pos[b]), raw_pos0=int(pos[b]) - W + 1,
                                 hca=(inp["k_hca"][b:b + 1], inp["v_hca"][b:b + 1], cfg["m_hca"]),
                                 csa=(inp["k_csa"][b:b + 1], inp["v_csa"][b:b + 1], idx[b:b + 1]))
        assert_close(got[b:b + 1], want, f"fused RoPE decode sequence {b}")
