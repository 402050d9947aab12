"""GPU parity of hybrid_cache_append (decode cache maintenance) against the
oracle's cache_append: ring rows bit-exact, compressed entries within the
storage-dtype tolerance, untouched entries unchanged, the dropped count exact.
A token-by-token stream must also end with the caches that compressing each
whole sequence at once gives (the oracle's and hca_compress_kv's)."""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import DEV, assert_close, dev, host, lib

pytestmark = pytest.mark.gpu

STATE = ("k_ring", "v_ring", "kI_ring", "k_csa", "v_csa", "k_hca", "v_hca", "kI_csa")


def gpu_run(inp, positions, hca=True, indexer=True):
    """positions: [steps][B] ints.  Returns the final state (host) and drops."""
    s = {k: dev(inp[k]) for k in STATE}
    z = {k: dev(inp[k]) for k in ("zk_csa", "zv_csa", "zk_hca", "zv_hca", "zI")}
    dropped = torch.zeros(1, dtype=torch.int32, device=DEV)
    for step, pos in enumerate(positions):
        p = torch.tensor(pos, dtype=torch.int64, device=DEV)
        binding.cache_append(p, dev(inp["k_new"][step]), dev(inp["v_new"][step]), s["k_ring"], s["v_ring"],
                             csa=(inp["m_csa"], z["zk_csa"], z["zv_csa"], s["k_csa"], s["v_csa"]),
                             hca=(inp["m_hca"], z["zk_hca"], z["zv_hca"], s["k_hca"], s["v_hca"]) if hca else None,
                             indexer=(dev(inp["kI_new"][step]), s["kI_ring"], z["zI"], s["kI_csa"])
                             if indexer else None,
                             dropped=dropped)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in s.items()}, int(dropped.item())


def oracle_run(inp, positions, hca=True, indexer=True):
    s = {k: inp[k].copy() for k in STATE}
    dropped = 0
    for step, pos in enumerate(positions):
        branches = [(inp["m_csa"], inp["zk_csa"], inp["zv_csa"], s["k_csa"], s["v_csa"])]
        if hca:
            branches.append((inp["m_hca"], inp["zk_hca"], inp["zv_hca"], s["k_hca"], s["v_hca"]))
        dropped += O.cache_append(
            pos, inp["k_new"][step], inp["v_new"][step], s["k_ring"], s["v_ring"], W=inp["W"], dtype=inp["dtype"],
            branches=branches,
            kI_new=inp["kI_new"][step] if indexer else None, kI_ring=s["kI_ring"] if indexer else None,
            kI_branch=(inp["m_csa"], inp["zI"], s["kI_csa"]) if indexer else None)
    return s, dropped


def check(inp, positions, what, hca=True, indexer=True):
    lib()
    got, gd = gpu_run(inp, positions, hca=hca, indexer=indexer)
    want, wd = oracle_run(inp, positions, hca=hca, indexer=indexer)
    assert gd == wd, f"{what}: dropped {gd} != {wd}"
    for k in ("k_ring", "v_ring", "kI_ring"):
        assert np.array_equal(got[k], want[k]), f"{what}: {k}"
    for k in ("k_csa", "v_csa", "k_hca", "v_hca", "kI_csa"):
        same = want[k] == inp[k]
        assert np.array_equal(got[k][same], inp[k][same]), f"{what}: {k} entry written that should not be"
        assert_close(got[k], want[k], f"{what}: {k}")
    return got, want


def test_append_one_step_all_cases():
    # per sequence: both blocks complete (t=255), CSA only (259), neither (257),
    # HCA stored but CSA past capacity (383), both past capacity (511), inactive
    inp = synth.make_append(B=6, Hkv=2, d=128, W=128, m_csa=4, m_hca=128, d_idx=64, cap_csa=80, cap_hca=3,
                            steps=1, seed=30)
    got, want = check(inp, [[255, 259, 257, 383, 511, -1]], "one step")
    _, wd = oracle_run(inp, [[255, 259, 257, 383, 511, -1]])
    assert wd == 2 + 3       # (CSA K/V + indexer keys) of t=383; those and the HCA pair of t=511


@pytest.mark.parametrize("dtype", [binding.DTYPE_BF16, binding.DTYPE_F32])
def test_append_stream_matches_whole_sequence_compression(dtype):
    # three sequences, the third joining 40 steps late (inactive before)
    W, m_csa, m_hca, T = 32, 4, 32, 200
    inp = synth.make_append(B=3, Hkv=2, d=64, W=W, m_csa=m_csa, m_hca=m_hca, d_idx=64, cap_csa=T // m_csa,
                            cap_hca=T // m_hca, steps=T, dtype=dtype, zero_state=True, seed=31)
    positions = [[s, s, s - 40] for s in range(T)]
    got, _ = check(inp, positions, f"stream dtype={dtype}")
    lens = [T, T, T - 40]
    for b in range(3):
        n = lens[b]
        start = T - n
        kseq = inp["k_new"][start:, b][None]       # [1, n, Hkv, d]
        vseq = inp["v_new"][start:, b][None]
        for m, zk, zv, kc, vc in ((m_csa, "zk_csa", "zv_csa", "k_csa", "v_csa"),
                                  (m_hca, "zk_hca", "zv_hca", "k_hca", "v_hca")):
            ok_, ov_ = O.compress_kv(kseq, vseq, inp[zk], inp[zv], m, dtype)
            nb = n // m
            assert_close(got[kc][b:b + 1, :nb], ok_, f"{kc} seq {b} vs whole-sequence oracle")
            assert_close(got[vc][b:b + 1, :nb], ov_, f"{vc} seq {b} vs whole-sequence oracle")
            gk, gv = binding.hca_compress_kv(dev(kseq), dev(vseq), dev(inp[zk]), dev(inp[zv]), m)
            assert_close(got[kc][b:b + 1, :nb], host(gk), f"{kc} seq {b} vs hca_compress_kv")
            assert_close(got[vc][b:b + 1, :nb], host(gv), f"{vc} seq {b} vs hca_compress_kv")
        kIseq = inp["kI_new"][start:, b][None, :, None, :]
        want_I = O.to_storage(O.compress(O.to_f64(kIseq, dtype), inp["zI"][:, None, :], m_csa)[:, :, 0], dtype)
        assert_close(got["kI_csa"][b:b + 1, :n // m_csa], want_I, f"kI seq {b} vs whole-sequence oracle")


def test_append_fp32_d64_csa_only_without_indexer_keys():
    # one ratio, no HCA caches, no indexer keys (their ring and cache must stay
    # untouched), a ring exactly one block long (W = m)
    inp = synth.make_append(B=4, Hkv=3, d=64, W=4, m_csa=4, m_hca=4, d_idx=64, cap_csa=12, cap_hca=1,
                            steps=40, dtype=binding.DTYPE_F32, seed=32)
    got, _ = check(inp, [[s, s + 3, s + 5, s - 7] for s in range(40)], "fp32 d64 CSA only", hca=False,
                   indexer=False)
    assert np.array_equal(got["kI_ring"], inp["kI_ring"]) and np.array_equal(got["kI_csa"], inp["kI_csa"])
    assert np.array_equal(got["k_hca"], inp["k_hca"])


def test_append_zero_capacity_drops_every_hca_entry():
    inp = synth.make_append(B=2, Hkv=1, d=128, W=8, m_csa=2, m_hca=8, d_idx=128, cap_csa=6, cap_hca=0,
                            steps=20, seed=33)
    lib()
    _, gd = gpu_run(inp, [[s, s] for s in range(20)])
    # HCA: 2 completed blocks per sequence, none stored; CSA K/V and indexer
    # keys: 10 blocks per sequence, 6 stored
    assert gd == 2 * 2 + 2 * (10 - 6) * 2
    check(inp, [[s, s] for s in range(20)], "zero-capacity HCA")

