"""End-to-end multi-step decode on the GPU: every step appends one token per
sequence (hybrid_cache_append), selects CSA entries for the new query at each
sequence's own position (csa_index_topk_varlen) and attends over the window
ring and the compressed caches (hybrid_sparse_attn_fwd with per-sequence
positions and ring addressing).  Each step is compared with the oracle doing
the same three things on its own state (cache_append, index_topk,
hybrid_attn_fwd on the window read back from its ring).

Sequences start at different positions (their history is compressed into
the initial caches by the oracle and given to both sides); one batch slot
stays inactive (position -1) and must be left untouched."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import DEV, assert_close, dev, host, lib

pytestmark = pytest.mark.gpu


def initial_state(inp, W, m_csa, m_hca, cap_csa, cap_hca):
    """Rings holding the last W tokens before each sequence's start and the
    caches holding every block completed by then (oracle compression)."""
    B, Hkv, d, di, dt = inp["B"], inp["Hkv"], inp["d"], inp["d_idx"], inp["dtype"]
    zero = (lambda shape: np.zeros(shape, np.uint16)) if dt == binding.DTYPE_BF16 else \
        (lambda shape: np.zeros(shape, np.float32))
    st = {"k_ring": zero((B, W, Hkv, d)), "v_ring": zero((B, W, Hkv, d)), "kI_ring": zero((B, W, di)),
          "k_csa": zero((B, cap_csa, Hkv, d)), "v_csa": zero((B, cap_csa, Hkv, d)), "kI_csa": zero((B, cap_csa, di)),
          "k_hca": zero((B, cap_hca, Hkv, d)), "v_hca": zero((B, cap_hca, Hkv, d))}
    for b in range(B):
        p0 = inp["lengths"][b]
        ks, vs, kis = inp["k_seq"][b], inp["v_seq"][b], inp["kI_seq"][b]
        for p in range(max(0, p0 - W), p0):
            st["k_ring"][b, p % W] = ks[p]
            st["v_ring"][b, p % W] = vs[p]
            st["kI_ring"][b, p % W] = kis[p]
        for m, zk, zv, kc, vc in ((m_csa, "zk_csa", "zv_csa", "k_csa", "v_csa"),
                                  (m_hca, "zk_hca", "zv_hca", "k_hca", "v_hca")):
            nb = p0 // m
            if nb:
                a, c = O.compress_kv(ks[None, :nb * m], vs[None, :nb * m], inp[zk][:m], inp[zv][:m], m, dt)
                st[kc][b, :nb], st[vc][b, :nb] = a[0], c[0]
        nb = p0 // m_csa
        if nb:
            kI = O.to_f64(kis[None, :nb * m_csa, None, :], dt)
            st["kI_csa"][b, :nb] = O.to_storage(O.compress(kI, inp["zI"][:m_csa, None, :], m_csa)[0, :, 0], dt)
    return st


def near_tie(inp, s, b, t, kIc, W, m, k, got, want):
    """True when every entry in the symmetric difference of two selections
    scores (float64, oracle) within the float32 cache-rounding band of the
    k-th score: the two sides compress indexer keys in float32 and float64,
    so their keys may differ by a few float32 units in the last place."""
    dt = inp["dtype"]
    q = O.to_f64(inp["qI"][s, b], dt)
    w = inp["w"][s, b].astype(np.float64)
    keys = O.to_f64(kIc[b], dt)[:O.visible_count(t, W, m, kIc.shape[1])]
    sc = O.indexer_scores(q, w, keys)
    kth = np.sort(sc)[::-1][min(k, sc.size) - 1]
    diff = set(got[got >= 0].tolist()) ^ set(want[want >= 0].tolist())
    qn = float(np.sum(np.abs(w) * np.linalg.norm(q, axis=1)))
    for e in diff:
        band = 16 * 2.0 ** -24 * 2 * qn * float(np.linalg.norm(keys[e]))
        if abs(sc[e] - kth) > band:
            return False
    return True


def run_stream(dtype, m_csa, m_hca, cap_csa, cap_hca, lengths, steps, seed, exact_idx):
    lib()
    W, k = 64, 32
    inp = synth.make_decode_stream(B=len(lengths), H=8, Hkv=2, d=128, d_idx=64, Hi=4, lengths=lengths,
                                   steps=steps, dtype=dtype, seed=seed)
    B, H, d, dt = inp["B"], inp["H"], inp["d"], dtype
    active = [L > 0 for L in lengths]          # a zero-length slot stays inactive throughout
    st = initial_state(inp, W, m_csa, m_hca, cap_csa, cap_hca)
    ost = {n: a.copy() for n, a in st.items()}                 # the oracle's own state
    gst = {n: dev(a) for n, a in st.items()}                   # the GPU's
    z = {n: dev(np.ascontiguousarray(inp[n][:m])) for n, m in
         (("zk_csa", m_csa), ("zv_csa", m_csa), ("zI", m_csa), ("zk_hca", m_hca), ("zv_hca", m_hca))}
    gates = dev(inp["gates"])
    sentinel = np.full((B, 1, H, d), 0x3F80 if dt == binding.DTYPE_BF16 else 1.0,
                       np.uint16 if dt == binding.DTYPE_BF16 else np.float32)
    out = dev(sentinel)
    exempt = checked = 0
    for s in range(steps):
        pos = [lengths[b] + s if active[b] else -1 for b in range(B)]
        new = {n: np.stack([inp[src][b][pos[b]] if active[b] else inp[src][b][0] for b in range(B)])
               for n, src in (("k", "k_seq"), ("v", "v_seq"), ("kI", "kI_seq"))}
        pos_t = torch.tensor(pos, dtype=torch.int64, device=DEV)
        # ---- GPU: append, select, attend
        binding.cache_append(pos_t, dev(new["k"]), dev(new["v"]), gst["k_ring"], gst["v_ring"],
                             csa=(m_csa, z["zk_csa"], z["zv_csa"], gst["k_csa"], gst["v_csa"]),
                             hca=(m_hca, z["zk_hca"], z["zv_hca"], gst["k_hca"], gst["v_hca"]),
                             indexer=(dev(new["kI"]), gst["kI_ring"], z["zI"], gst["kI_csa"]))
        idx = binding.csa_index_topk(dev(inp["qI"][s][:, None]), gst["kI_csa"], dev(inp["w"][s][:, None]), pos_t,
                                     m_csa, W, k)
        binding.hybrid_sparse_attn_fwd(dev(inp["q"][s][:, None]), gst["k_ring"], gst["v_ring"], gates, W,
                                       q_pos=pos_t, raw_ring=True, hca=(gst["k_hca"], gst["v_hca"], m_hca),
                                       csa=(gst["k_csa"], gst["v_csa"], idx), out=out)
        g_idx, g_out = host(idx), host(out)
        # ---- oracle: the same on its own state
        O.cache_append(pos, new["k"], new["v"], ost["k_ring"], ost["v_ring"], W=W, dtype=dt,
                       branches=((m_csa, inp["zk_csa"][:m_csa], inp["zv_csa"][:m_csa], ost["k_csa"], ost["v_csa"]),
                                 (m_hca, inp["zk_hca"][:m_hca], inp["zv_hca"][:m_hca], ost["k_hca"], ost["v_hca"])),
                       kI_new=new["kI"], kI_ring=ost["kI_ring"], kI_branch=(m_csa, inp["zI"][:m_csa], ost["kI_csa"]))
        for b in range(B):
            if not active[b]:
                assert (g_idx[b] == -1).all(), f"step {s}: inactive slot {b} got indices"
                assert np.array_equal(g_out[b], sentinel[b]), f"step {s}: inactive slot {b} output written"
                continue
            t = pos[b]
            want_idx = O.index_topk(inp["qI"][s][b][None, None], ost["kI_csa"][b][None], inp["w"][s][b][None, None],
                                    t, m_csa, W, k, dt)[0, 0]
            checked += 1
            if not np.array_equal(g_idx[b, 0], want_idx):
                assert not exact_idx, f"step {s} seq {b} (t={t}): index row differs: gpu {g_idx[b, 0][:10]} " \
                                      f"oracle {want_idx[:10]}"
                assert near_tie(inp, s, b, t, ost["kI_csa"], W, m_csa, k, g_idx[b, 0], want_idx), \
                    f"step {s} seq {b} (t={t}): index row differs beyond the cache-rounding band"
                exempt += 1
                continue
            lo = max(0, t - W + 1)
            slots = [p % W for p in range(lo, t + 1)]
            want = O.hybrid_attn_fwd(inp["q"][s][b][None, None], ost["k_ring"][b][slots][None],
                                     ost["v_ring"][b][slots][None], inp["gates"], W=W, dtype=dt, q_pos0=t,
                                     raw_pos0=lo, hca=(ost["k_hca"][b][None], ost["v_hca"][b][None], m_hca),
                                     csa=(ost["k_csa"][b][None], ost["v_csa"][b][None], want_idx[None, None]))
            assert_close(g_out[b], want[0], f"step {s} seq {b} (t={t}) attention")
    assert exempt <= 0.02 * checked, f"{exempt} of {checked} index rows differ (near ties)"
    return checked


def test_decode_stream_bf16_split_paths():
    # bf16, CSA ratio 1 (compressed keys equal the tokens on both sides, so
    # every index row must match exactly); a CSA capacity of 8192 entries
    # takes the split (decode) indexer and the split attention; one slot
    # inactive; 200 steps
    n = run_stream(binding.DTYPE_BF16, m_csa=1, m_hca=8, cap_csa=8192, cap_hca=1024,
                   lengths=[700, 1500, 2300, 0], steps=200, seed=60, exact_idx=True)
    assert n == 600


def test_decode_stream_fp32_ratio4():
    # fp32, CSA ratio 4 and HCA ratio 16 with short caches (the dense indexer
    # and unsplit attention); sequences start inside their first window and
    # well past it; near ties within the cache-rounding band may differ
    run_stream(binding.DTYPE_F32, m_csa=4, m_hca=16, cap_csa=1024, cap_hca=256,
               lengths=[10, 900, 2500], steps=200, seed=61, exact_idx=False)
