"""GPU parity of hca_compress_kv against the oracle's block compression."""
import numpy as np
import pytest

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import assert_close, dev, host, lib

pytestmark = pytest.mark.gpu


def _run(inp, m, zk, zv):
    k, v = dev(inp["k"]), dev(inp["v"])
    kc, vc = binding.hca_compress_kv(k, v, dev(zk), dev(zv), m)
    return host(kc), host(vc)


@pytest.mark.parametrize("name,over,m", [
    ("tiny_fp32", {}, 4),
    ("tiny_fp32", {}, 32),
    ("tiny_fp32", {"T": 250}, 4),                    # ragged tail: 250 % 4 = 2
    ("tiny_fp32", {"T": 77, "Hkv": 3, "H": 3}, 1),   # identity ratio
    ("tinyr2_bf16", {"B": 2, "T": 520}, 4),
    ("tinyr2_bf16", {"B": 2, "T": 520}, 128),        # ragged: 520 % 128 = 8
    ("tinyr2_bf16", {"B": 1, "T": 700, "H": 2, "Hkv": 2, "d": 64}, 12),  # m not a power of two
    ("tinyr2_bf16", {"B": 1, "T": 1100, "H": 1, "Hkv": 1}, 256),
    ("hca_prefill_32k", {"T": 4096}, 128),
])
def test_compress_matches_oracle(name, over, m):
    lib()
    inp = synth.make_inputs(name, seed=3, **over)
    Hkv, d = inp["k"].shape[2], inp["k"].shape[3]
    rng = np.random.default_rng(4)
    zk = (rng.standard_normal((m, Hkv, d)) / 8).astype(np.float32)
    zv = (rng.standard_normal((m, Hkv, d)) / 8).astype(np.float32)
    kc, vc = _run(inp, m, zk, zv)
    dt = inp["cfg"]["dtype"]
    okc, ovc = O.compress_kv(inp["k"], inp["v"], zk, zv, m, dt)
    assert kc.shape == okc.shape
    assert_close(kc, okc, f"kc m={m}")
    assert_close(vc, ovc, f"vc m={m}")


@pytest.mark.parametrize("m", [4, 128])
def test_compress_full_tinyr2(m):
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=0)
    kc, vc = _run(inp, m, inp[f"zk_{'csa' if m == 4 else 'hca'}"], inp[f"zv_{'csa' if m == 4 else 'hca'}"])
    okc, ovc = O.compress_kv(inp["k"], inp["v"], inp[f"zk_{'csa' if m == 4 else 'hca'}"],
                             inp[f"zv_{'csa' if m == 4 else 'hca'}"], m, O.DTYPE_BF16)
    assert_close(kc, okc, "kc")
    assert_close(vc, ovc, "vc")


def test_compress_deterministic_and_empty():
    lib()
    inp = synth.make_inputs("tinyr2_bf16", seed=5, B=1, T=1024)
    a = _run(inp, 128, inp["zk_hca"], inp["zv_hca"])
    b = _run(inp, 128, inp["zk_hca"], inp["zv_hca"])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # T < m: no entries, nothing launched
    small = synth.make_inputs("tinyr2_bf16", seed=6, B=1, T=100)
    kc, vc = _run(small, 128, np.zeros((128, 12, 128), np.float32), np.zeros((128, 12, 128), np.float32))
    assert kc.shape == (1, 0, 12, 128)


@pytest.mark.parametrize("name,over,m1,m2", [
    ("tinyr2_bf16", {}, 4, 128),                                   # the Tiny-R2 shape, both ratios
    ("tinyr2_bf16", {"B": 2, "T": 700}, 4, 128),                   # ragged: 700 = 5*128 + 60
    ("tinyr2_bf16", {"B": 1, "T": 530, "H": 2, "Hkv": 2, "d": 64}, 8, 64),
    ("tinyr2_bf16", {"B": 1, "T": 300, "H": 3, "Hkv": 3}, 1, 8),
    ("tinyr2_bf16", {"B": 1, "T": 2100, "H": 1, "Hkv": 1}, 2, 256),
    ("tiny_fp32", {}, 4, 32),
    ("tiny_fp32", {"T": 250}, 4, 32),
    ("tinyr2_bf16", {"B": 1, "T": 100}, 4, 128),                   # no full m2-block
])
def test_dual_compress_matches_oracle(name, over, m1, m2):
    lib()
    inp = synth.make_inputs(name, seed=7, **over)
    Hkv, d = inp["k"].shape[2], inp["k"].shape[3]
    rng = np.random.default_rng(8)
    z = [(rng.standard_normal((m, Hkv, d)) / 8).astype(np.float32) for m in (m1, m1, m2, m2)]
    (kc1, vc1), (kc2, vc2) = binding.hca_compress_kv_dual(dev(inp["k"]), dev(inp["v"]), dev(z[0]), dev(z[1]), m1,
                                                          dev(z[2]), dev(z[3]), m2)
    dt = inp["cfg"]["dtype"]
    o1 = O.compress_kv(inp["k"], inp["v"], z[0], z[1], m1, dt)
    o2 = O.compress_kv(inp["k"], inp["v"], z[2], z[3], m2, dt)
    assert_close(host(kc1), o1[0], "kc1")
    assert_close(host(vc1), o1[1], "vc1")
    assert_close(host(kc2), o2[0], "kc2")
    assert_close(host(vc2), o2[1], "vc2")
