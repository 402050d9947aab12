"""Pins of the oracle's backward pass (reading R12) against things other than
itself: torch's CPU autograd (a library routine) where the path reduces to a
textbook operation, and central finite differences of the oracle's own
forward value everywhere else (a check that the backward is the derivative of
the forward, which the forward pins tie to the pages).  Each case is chosen
so that a plausible slip (a dropped key set, a transposed operand, a missing
scale, the softmax Jacobian's centring term, a gate chain-rule factor, a
cache gradient not routed through the compression) fails it."""

import numpy as np
import pytest
import torch

import oracle as O

F64 = O.DTYPE_F64


def _rng(seed):
    return np.random.default_rng(seed)


# -------------------------------------------------------------- compression
def test_compress_backward_matches_autograd():
    rng = _rng(0)
    B, T, Hkv, d, m = 2, 14, 2, 3, 4            # T % m != 0: the trailing rows get no gradient
    x = rng.standard_normal((B, T, Hkv, d))
    z = rng.standard_normal((m, Hkv, d))
    dxc = rng.standard_normal((B, T // m, Hkv, d))
    dx, dz = O.compress_backward(x, z, m, dxc)
    xt = torch.tensor(x, requires_grad=True)
    zt = torch.tensor(z, requires_grad=True)
    n = T // m
    xc = (torch.softmax(zt, dim=0)[None, None] * xt[:, : n * m].reshape(B, n, m, Hkv, d)).sum(dim=2)
    (xc * torch.tensor(dxc)).sum().backward()
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dz, zt.grad.numpy(), rtol=0, atol=1e-12)
    assert not dx[:, n * m:].any()


def test_compress_backward_ratio_one_has_no_logit_gradient():
    rng = _rng(1)
    x = rng.standard_normal((1, 5, 1, 4))
    dx, dz = O.compress_backward(x, rng.standard_normal((1, 1, 4)), 1, rng.standard_normal((1, 5, 1, 4)))
    assert not dz.any()


# ------------------------------------------- reductions to dense attention
def _sdpa_grads(qf, kf, vf, dout):
    """torch autograd of causal softmax attention (float64, CPU) with GQA by
    repeating K/V over the group; returns (dq, dk, dv) in [B, T, H|Hkv, d]."""
    B, T, H, d = qf.shape
    Hkv = kf.shape[2]
    G = H // Hkv
    q = torch.tensor(qf, requires_grad=True)
    k = torch.tensor(kf, requires_grad=True)
    v = torch.tensor(vf, requires_grad=True)
    kk = k.repeat_interleave(G, dim=2).transpose(1, 2).contiguous()
    vv = v.repeat_interleave(G, dim=2).transpose(1, 2).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q.transpose(1, 2).contiguous(), kk, vv,
                                                         is_causal=True)
    (o.transpose(1, 2) * torch.tensor(dout)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def _all_visible_idx(B, T, W, k):
    idx = np.full((B, T, k), -1, np.int32)
    for t in range(T):
        n = O.visible_count(t, W, 1, T)
        idx[:, t, :n] = np.arange(n)
    return idx


@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 2)])
def test_backward_csa_ratio1_all_selected_is_dense_causal(H, Hkv):
    rng = _rng(2)
    B, T, d, W = 1, 19, 8, 5
    q, k, v = (rng.standard_normal(s) for s in ((B, T, H, d), (B, T, Hkv, d), (B, T, Hkv, d)))
    dout = rng.standard_normal((B, T, H, d))
    gates = np.tile(np.array([0.0, 1.0, 0.0], np.float32), (H, 1))
    zk, zv = rng.standard_normal((1, Hkv, d)), rng.standard_normal((1, Hkv, d))
    res = O.hybrid_path_bwd(q, k, v, gates, dout, W=W, dtype=F64, idx=_all_visible_idx(B, T, W, T),
                            csa=(zk, zv, 1))
    dq, dk, dv = _sdpa_grads(q, k, v, dout)
    np.testing.assert_allclose(res["dq"], dq, rtol=0, atol=1e-11)
    np.testing.assert_allclose(res["dk"], dk, rtol=0, atol=1e-11)
    np.testing.assert_allclose(res["dv"], dv, rtol=0, atol=1e-11)
    assert not res["dzk_csa"].any() and not res["dzv_csa"].any()


def test_backward_window_covering_the_sequence_is_dense_causal():
    rng = _rng(3)
    B, T, H, Hkv, d = 2, 11, 4, 1, 6
    q, k, v = (rng.standard_normal(s) for s in ((B, T, H, d), (B, T, Hkv, d), (B, T, Hkv, d)))
    dout = rng.standard_normal((B, T, H, d))
    gates = np.tile(np.array([0.0, 0.0, 1.0], np.float32), (H, 1))
    res = O.hybrid_path_bwd(q, k, v, gates, dout, W=T + 3, dtype=F64)
    dq, dk, dv = _sdpa_grads(q, k, v, dout)
    for name, want in (("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(res[name], want, rtol=0, atol=1e-11)


# ----------------------------------------------------- finite differences
def _forward_value(q, k, v, gates, dout, *, W, hca, csa, idx, gate_mode):
    out = O.hybrid_attn_fwd(q, k, v, gates, W=W, dtype=F64, gate_mode=gate_mode,
                            hca=None if hca is None else (*O.compress_kv(k, v, hca[0], hca[1], hca[2], F64), hca[2]),
                            csa=None if csa is None else (*O.compress_kv(k, v, csa[0], csa[1], csa[2], F64), idx))
    return float((out * dout).sum())


@pytest.mark.parametrize("gate_mode", [0, 1, 2])
def test_backward_matches_central_differences(gate_mode):
    rng = _rng(10 + gate_mode)
    B, T, H, Hkv, d, W = 1, 24, 4, 2, 4, 5
    m_h, m_c, kk = 4, 2, 3
    q, k, v = (rng.standard_normal(s) for s in ((B, T, H, d), (B, T, Hkv, d), (B, T, Hkv, d)))
    dout = rng.standard_normal((B, T, H, d))
    hca = (rng.standard_normal((m_h, Hkv, d)) / 2, rng.standard_normal((m_h, Hkv, d)) / 2, m_h)
    csa = (rng.standard_normal((m_c, Hkv, d)) / 2, rng.standard_normal((m_c, Hkv, d)) / 2, m_c)
    # a selection of up to kk visible entries per row (not the top-k of anything: the selection is an input)
    idx = np.full((B, T, kk), -1, np.int32)
    for t in range(T):
        n = O.visible_count(t, W, m_c, T // m_c)
        sel = np.sort(rng.permutation(n)[: min(kk, n)])
        idx[0, t, : sel.size] = sel
    if gate_mode == 0:
        gates = rng.random((H, 3)).astype(np.float32)
    else:
        gates = (rng.standard_normal((B, T, H, 3)) * (1.0 if gate_mode == 2 else 0.5)).astype(np.float32)
    kw = dict(W=W, hca=hca, csa=csa, idx=idx, gate_mode=gate_mode)
    res = O.hybrid_path_bwd(q, k, v, gates, dout, W=W, dtype=F64, idx=idx, hca=hca, csa=csa, gate_mode=gate_mode)
    eps = 1e-6

    def fd(arr, pos, rebuild, h=eps):
        a_p, a_m = arr.copy(), arr.copy()
        a_p[pos] += h
        a_m[pos] -= h
        return (rebuild(a_p) - rebuild(a_m)) / (2 * h)

    checks = []
    for _ in range(6):
        pos = tuple(int(rng.integers(0, s)) for s in q.shape)
        checks.append(("dq", pos, fd(q, pos, lambda a: _forward_value(a, k, v, gates, dout, **kw))))
        pos = tuple(int(rng.integers(0, s)) for s in k.shape)
        checks.append(("dk", pos, fd(k, pos, lambda a: _forward_value(q, a, v, gates, dout, **kw))))
        pos = tuple(int(rng.integers(0, s)) for s in v.shape)
        checks.append(("dv", pos, fd(v, pos, lambda a: _forward_value(q, k, a, gates, dout, **kw))))
    # raw rows late in the sequence reach every branch (window, HCA and CSA blocks)
    for pos in ((0, T - 9, 1, 2), (0, 3, 0, 1)):
        checks.append(("dk", pos, fd(k, pos, lambda a: _forward_value(q, a, v, gates, dout, **kw))))
        checks.append(("dv", pos, fd(v, pos, lambda a: _forward_value(q, k, a, gates, dout, **kw))))
    for name, br, slot in (("dzk_hca", "hca", 0), ("dzv_hca", "hca", 1), ("dzk_csa", "csa", 0),
                           ("dzv_csa", "csa", 1)):
        src = hca if br == "hca" else csa
        for _ in range(2):
            pos = tuple(int(rng.integers(0, s)) for s in src[slot].shape)

            def rebuild(a, br=br, slot=slot, src=src):
                new = list(src)
                new[slot] = a
                kw2 = dict(kw, **{br: tuple(new)})
                return _forward_value(q, k, v, gates, dout, **kw2)
            checks.append((name, pos, fd(src[slot], pos, rebuild)))
    # gates are float32 by the interface: a step of 2^-12 keeps g +- step exact
    for _ in range(4):
        pos = tuple(int(rng.integers(0, s)) for s in gates.shape)
        checks.append(("dgates", pos, fd(gates, pos, lambda a: _forward_value(q, k, v, a, dout, **kw), 2.0 ** -12)))
    for name, pos, want in checks:
        got = res[name][pos]
        tol = (1e-5 if name == "dgates" else 1e-6) * max(1.0, abs(want))
        assert abs(got - want) <= tol, (name, pos, got, want)


def test_backward_gate_gradient_is_branch_output():
    # per-head gates: dL/dg[h, b] = sum over rows of dout . O_b; check against
    # the forward's own per-branch outputs (a different code path)
    rng = _rng(20)
    B, T, H, Hkv, d, W = 1, 16, 2, 1, 4, 3
    q, k, v = (rng.standard_normal(s) for s in ((B, T, H, d), (B, T, Hkv, d), (B, T, Hkv, d)))
    dout = rng.standard_normal((B, T, H, d))
    gates = rng.random((H, 3)).astype(np.float32)
    hca = (rng.standard_normal((4, Hkv, d)), rng.standard_normal((4, Hkv, d)), 4)
    res = O.hybrid_path_bwd(q, k, v, gates, dout, W=W, dtype=F64, hca=hca)
    kh, vh = O.compress_kv(k, v, hca[0], hca[1], 4, F64)
    _, br = O.hybrid_attn_fwd(q, k, v, gates, W=W, dtype=F64, hca=(kh, vh, 4), branches=True)
    for col, name in ((0, "hca"), (2, "swa")):
        want = (dout * br[name]).sum(axis=(0, 1, 3))
        np.testing.assert_allclose(res["dgates"][:, col], want, rtol=0, atol=1e-12)
    assert not res["dgates"][:, 1].any()          # the CSA branch is absent
