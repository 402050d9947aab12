"""Backward pass of the prefill path on the GPU (hybrid_sparse_attn_bwd)
against the oracle's float64 backward (reading R12: the derivative of the
forward value with the CSA selection fixed and the cache rounding taken as
the identity).

Small shapes span several 64-row tiles with a ragged tail and are compared
element by element on every output: dq, dk, dv, the compression-logit
gradients, the gate gradients and the compressed-cache gradients.  At the
Tiny-R2 training shape (B8 T2048 H=Hkv=12 d128 bf16, W128, HCA m128, CSA m4
k64 from the oracle indexer) the oracle computes the last 128 query rows of
two sequences exactly; those rows alone decide dq and the per-token gate
gradients of those rows, dk/dv of raw rows 1920.., the HCA entry 14 and the
CSA entries 448.. (no earlier row sees them).  The rest is checked through
properties that hold at any size: the v-gradients of each sequence sum to
the gated incoming gradient, the k-gradients sum to zero, and every
logit gradient sums to zero over the block positions.

The bar: |got - want| <= BWD_TOL * max|want| per tensor (with a floor for
outputs that cancel, see below).  Both sides read the
same exactly-representable inputs (the caches are the oracle's), so the
difference is the kernel's float32 arithmetic: dot products of length d,
exp2/log2, and sums of at most a few thousand terms per output (n u <= 2.5e-4
relative to the sum of magnitudes for n <= 4096, u = 2^-24); 1e-3 of the
tensor's largest magnitude bounds that with room for cancellation.
"""
import numpy as np
import pytest
import torch

import oracle as O
from sparse_hybrid_attention_amd import binding, synth
from gpu_util import as_f64, dev, host, lib

pytestmark = pytest.mark.gpu

BWD_TOL = 1e-3


def random_selection(B, T, W, m, N, k, seed):
    """Up to k distinct visible entries per row, ascending, -1 padded (the
    selection is an input of the backward, not the top-k of anything)."""
    rng = np.random.default_rng([seed, 2])
    idx = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        for t in range(T):
            n = O.visible_count(t, W, m, N)
            sel = np.sort(rng.permutation(n)[: min(k, n)])
            idx[b, t, : sel.size] = sel
    return idx


def setup_case(inp, gate_mode, idx=None, seed=0):
    cfg = inp["cfg"]
    dt, W = cfg["dtype"], cfg["W"]
    B, T = cfg["B"], cfg["T"]
    hca = csa = None
    gpu_hca = gpu_csa = None
    if cfg.get("m_hca"):
        m = cfg["m_hca"]
        kc, vc = O.compress_kv(inp["k"], inp["v"], inp["zk_hca"], inp["zv_hca"], m, dt)
        hca = (inp["zk_hca"], inp["zv_hca"], m)
        gpu_hca = (dev(inp["zk_hca"]), dev(inp["zv_hca"]), dev(kc), dev(vc), m)
    if cfg.get("m_csa"):
        m = cfg["m_csa"]
        kc, vc = O.compress_kv(inp["k"], inp["v"], inp["zk_csa"], inp["zv_csa"], m, dt)
        if idx is None:
            idx = random_selection(B, T, W, m, T // m, cfg["k"], seed)
        csa = (inp["zk_csa"], inp["zv_csa"], m)
        gpu_csa = (dev(inp["zk_csa"]), dev(inp["zv_csa"]), dev(kc), dev(vc), m, dev(idx))
    gpu = binding.hybrid_sparse_attn_bwd(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["gates"]),
                                         dev(inp["dout"]), W, hca=gpu_hca, csa=gpu_csa,
                                         gate_logits=gate_mode == 2, cache_grads=True)
    return gpu, hca, csa, idx


def check(got, want, what, scale=None):
    """|got - want| <= BWD_TOL * scale, scale = max|want| unless the output is
    a difference of larger terms (then the caller passes their magnitude)."""
    got = np.asarray(got, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite"
    if scale is None:
        scale = np.abs(want).max() if want.size else 0.0
    err = np.abs(got - want).max() if want.size else 0.0
    print(f"  {what}: max err {err:.3e} of max |want| {scale:.3e} ({err / max(scale, 1e-300):.2e})")
    assert err <= BWD_TOL * scale, f"{what}: max err {err} > {BWD_TOL} * {scale}"


CASES = {
    # name: (config overrides, gate_mode)
    "all_bf16_d128": (dict(dtype=0, B=2, T=136, H=4, Hkv=2, d=128, W=24, m_hca=16, m_csa=4, k=6), 0),
    "all_f32_d64_token": (dict(dtype=1, B=2, T=136, H=4, Hkv=2, d=64, W=24, m_hca=16, m_csa=4, k=6), 1),
    "all_bf16_d64_logits": (dict(dtype=0, B=1, T=200, H=2, Hkv=2, d=64, W=32, m_hca=32, m_csa=4, k=8), 2),
    "hca_only_gqa4": (dict(dtype=0, B=1, T=160, H=8, Hkv=2, d=128, W=16, m_hca=8, m_csa=None), 0),
    "csa_only_mqa": (dict(dtype=1, B=2, T=100, H=4, Hkv=1, d=128, W=16, m_hca=None, m_csa=4, k=5), 0),
    "swa_only": (dict(dtype=0, B=2, T=90, H=2, Hkv=1, d=64, W=20, m_hca=None, m_csa=None), 1),
    "csa_ratio1_k70": (dict(dtype=1, B=1, T=136, H=2, Hkv=2, d=64, W=24, m_hca=None, m_csa=1, k=70), 0),
    "window_covers_all": (dict(dtype=0, B=1, T=70, H=2, Hkv=2, d=64, W=100, m_hca=16, m_csa=4, k=4), 2),
    "hca_longer_than_T": (dict(dtype=0, B=2, T=50, H=2, Hkv=2, d=128, W=8, m_hca=64, m_csa=4, k=3), 0),
    "one_row": (dict(dtype=1, B=3, T=1, H=2, Hkv=1, d=64, W=4, m_hca=4, m_csa=2, k=2), 1),
}


@pytest.mark.parametrize("case", list(CASES))
def test_backward_matches_oracle(case):
    lib()
    over, gate_mode = CASES[case]
    inp = synth.make_backward("tiny_fp32", seed=100 + list(CASES).index(case), gate_mode=gate_mode,
                              gates="mix", Hi=2, d_idx=64, **over)
    cfg = inp["cfg"]
    gpu, hca, csa, idx = setup_case(inp, gate_mode, seed=len(case))
    want = O.hybrid_path_bwd(inp["q"], inp["k"], inp["v"], inp["gates"], as_f64(inp["dout"]), W=cfg["W"],
                             dtype=cfg["dtype"], idx=idx, hca=hca, csa=csa, gate_mode=gate_mode)
    print(case)
    names = ["dq", "dk", "dv", "dgates"]
    for br in (("hca",) if hca else ()) + (("csa",) if csa else ()):
        names += ["dzk_" + br, "dzv_" + br, "dk_" + br, "dv_" + br]
    assert set(names) == set(gpu), (sorted(names), sorted(gpu))
    # outputs that cancel (exactly zero when a row's only key is itself or
    # when the branches see the same keys) are measured against a floor: 1e-3
    # of the largest v-gradient, a positive-weight sum of the incoming
    # gradient, so of its magnitude
    floor = 1e-3 * np.abs(want["dv"]).max()
    for n in names:
        scale = max(np.abs(want[n]).max() if want[n].size else 0.0, floor)
        if n == "dgates" and gate_mode == 2:
            # the logit gradient w_b (D_b - sum_l w_l D_l) cancels (to zero
            # when every branch sees the same keys): measure it against the
            # magnitude of D_b = dout . O_b, from the oracle's branch outputs
            scale = max(scale, branch_dots(inp, hca, csa, idx).max())
        check(host(gpu[n]), want[n], f"{case} {n}", scale)


def branch_dots(inp, hca, csa, idx):
    """|dout . O_b| of every (row, head, present branch) from the oracle forward."""
    cfg = inp["cfg"]
    dt = cfg["dtype"]
    hc = None if hca is None else (*O.compress_kv(inp["k"], inp["v"], hca[0], hca[1], hca[2], dt), hca[2])
    cc = None if csa is None else (*O.compress_kv(inp["k"], inp["v"], csa[0], csa[1], csa[2], dt), idx)
    _, br = O.hybrid_attn_fwd(inp["q"], inp["k"], inp["v"], inp["gates"], W=cfg["W"], dtype=dt, hca=hc, csa=cc,
                              gate_mode=2, branches=True)
    dout = as_f64(inp["dout"])
    return np.stack([np.abs((dout * o).sum(axis=-1)) for o in br.values()])


def test_backward_empty_batch_zeroes_the_shared_gradients():
    lib()
    inp = synth.make_backward("tiny_fp32", seed=5, B=1, T=64, H=2, Hkv=2, d=64, W=8, m_hca=8, m_csa=4, k=2)
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device="cuda:0")
    f = lambda a: dev(np.ascontiguousarray(a))
    gpu = binding.hybrid_sparse_attn_bwd(
        z(0, 64, 2, 64), z(0, 64, 2, 64), z(0, 64, 2, 64), f(inp["gates"]), z(0, 64, 2, 64), 8,
        hca=(f(inp["zk_hca"]), f(inp["zv_hca"]), z(0, 8, 2, 64), z(0, 8, 2, 64), 8),
        csa=(f(inp["zk_csa"]), f(inp["zv_csa"]), z(0, 16, 2, 64), z(0, 16, 2, 64), 4,
             torch.zeros((0, 64, 2), dtype=torch.int32, device="cuda:0")))
    for n in ("dgates", "dzk_hca", "dzv_hca", "dzk_csa", "dzv_csa"):
        assert not host(gpu[n]).any(), n


def test_backward_is_deterministic():
    lib()
    over, gate_mode = CASES["all_bf16_d128"]
    inp = synth.make_backward("tiny_fp32", seed=7, gate_mode=gate_mode, gates="mix", Hi=2, d_idx=64, **over)
    a, _, _, idx = setup_case(inp, gate_mode, seed=7)
    b, _, _, _ = setup_case(inp, gate_mode, idx=idx)
    for n in a:
        assert torch.equal(a[n], b[n]), n


def test_backward_tinyr2_tail_rows_and_sums():
    """Tiny-R2 training shape, all three branches, per-head gates."""
    lib()
    inp = synth.make_backward("tinyr2_bf16", seed=11)
    cfg = inp["cfg"]
    B, T, H, Hkv, d, W, dt = cfg["B"], cfg["T"], cfg["H"], cfg["Hkv"], cfg["d"], cfg["W"], cfg["dtype"]
    mh, mc = cfg["m_hca"], cfg["m_csa"]
    idx = O.index_topk(inp["qI"], inp["kI"], inp["w"], 0, mc, W, cfg["k"], dt)
    gpu, _, _, _ = setup_case(inp, 0, idx=idx)
    g = {n: host(t).astype(np.float64) for n, t in gpu.items()}
    t0 = T - 128
    for b in (0, B - 1):
        kh, vh = O.compress_kv(inp["k"][b:b + 1], inp["v"][b:b + 1], inp["zk_hca"], inp["zv_hca"], mh, dt)
        kc, vc = O.compress_kv(inp["k"][b:b + 1], inp["v"][b:b + 1], inp["zk_csa"], inp["zv_csa"], mc, dt)
        want = O.hybrid_attn_bwd(inp["q"][b:b + 1, t0:], inp["k"][b:b + 1], inp["v"][b:b + 1], inp["gates"],
                                 as_f64(inp["dout"][b:b + 1, t0:]), W=W, dtype=dt, q_pos0=t0,
                                 hca=(kh, vh, mh), csa=(kc, vc, idx[b:b + 1, t0:]))
        print(f"sequence {b}")
        check(g["dq"][b, t0:], want["dq"][0], f"b{b} dq rows {t0}..")
        check(g["dk"][b, t0:], want["dk_raw"][0, t0:], f"b{b} dk raw rows {t0}..")
        check(g["dv"][b, t0:], want["dv_raw"][0, t0:], f"b{b} dv raw rows {t0}..")
        c_h = (t0 - W + 1) // mh                 # first HCA entry only the tail rows see
        c_c = (t0 - W + 1) // mc
        check(g["dk_hca"][b, c_h:], want["dk_hca"][0, c_h:], f"b{b} dk_hca entries {c_h}..")
        check(g["dv_hca"][b, c_h:], want["dv_hca"][0, c_h:], f"b{b} dv_hca entries {c_h}..")
        check(g["dk_csa"][b, c_c:], want["dk_csa"][0, c_c:], f"b{b} dk_csa entries {c_c}..")
        check(g["dv_csa"][b, c_c:], want["dv_csa"][0, c_c:], f"b{b} dv_csa entries {c_c}..")
    # every key set's softmax sums to one and the block weights sum to one:
    # the v-gradients of a sequence and KV head sum to sum_t sum_h (sum of the
    # present branches' gate weights) dout, and the k-gradients sum to zero
    gw = inp["gates"].astype(np.float64).sum(axis=1)                           # [H]
    dout = as_f64(inp["dout"])
    G = H // Hkv
    want_v = (dout * gw[None, None, :, None]).sum(axis=1).reshape(B, Hkv, G, d).sum(axis=2)
    check(g["dv"].sum(axis=1), want_v, "sum over rows of dv")
    mag = np.abs(g["dk"]).sum(axis=1)
    assert (np.abs(g["dk"].sum(axis=1)) <= 1e-4 * mag.max()).all(), "k-gradients do not sum to zero"
    for n in ("dzk_hca", "dzv_hca", "dzk_csa", "dzv_csa"):
        s, mag = np.abs(g[n].sum(axis=0)), np.abs(g[n]).sum(axis=0)
        assert (s <= 1e-4 * mag.max()).all(), f"{n} does not sum to zero over block positions"
