"""Seeded synthetic inputs for the hybrid sparse attention forward pass.

This module only draws random numbers and packs them into the storage layout;
it holds none of the method's arithmetic.  Tests feed the same arrays to the
HIP library and to the CPU oracle, and the benchmark uses it for its inputs.

Every array is drawn from ``numpy.random.Generator(PCG64(seed))`` in a fixed
order, as float32, and bfloat16 tensors are produced from those draws by
round-to-nearest-even on the float32 bit pattern (ties to even; finite values
only).  Storage form: ``np.uint16`` bit patterns for bfloat16, ``np.float32``
otherwise.

Workloads (all sizes are the ones the method is quoted on):

``tiny_fp32``       B1 T256 H=Hkv=4 d64 fp32; CSA m4 (64 entries) k8, indexer
                    2 heads d_idx 64; HCA m32; W32; gates U(0,1).
``tinyr2_bf16``     B8 T2048 H=Hkv=12 d128 bf16 (Tiny-R2 training shape);
                    CSA m4 (512 entries) k64, indexer 4 heads d_idx 64;
                    HCA m128 (16 entries); W128; gates U(0,1) or a one-hot mode.
``hca_prefill_32k`` B1 T32768 H16 Hkv2 d128 bf16; Q ~ N(0,1)/sqrt(d); HCA m128
                    (256 entries); W128; gates [1,0,0].
``csa_prefill_128k`` B1 T131072 H32 Hkv4 d128 bf16; CSA m4 (32768 entries),
                    indexer 4 heads d_idx 64, k512; W128; gates [0,1,0].
``decode_1m``       B16 x 1 query at 1,048,576 tokens of context, H32 Hkv1 d128
                    bf16; caches N(0,1): CSA 262,144 entries with indexer keys,
                    k1024; HCA 8,192 entries; raw window 128; gates U(0,1).
"""
from __future__ import annotations

import math

import numpy as np

DTYPE_BF16 = 0
DTYPE_F32 = 1

MODES = {
    "hca": (1.0, 0.0, 0.0),
    "csa": (0.0, 1.0, 0.0),
    "swa": (0.0, 0.0, 1.0),
}

CONFIGS = {
    "tiny_fp32": dict(kind="prefill", dtype=DTYPE_F32, B=1, T=256, H=4, Hkv=4, d=64,
                      m_csa=4, k=8, Hi=2, d_idx=64, m_hca=32, W=32, gates="mix"),
    "tinyr2_bf16": dict(kind="prefill", dtype=DTYPE_BF16, B=8, T=2048, H=12, Hkv=12,
                        d=128, m_csa=4, k=64, Hi=4, d_idx=64, m_hca=128, W=128,
                        gates="mix"),
    "hca_prefill_32k": dict(kind="prefill", dtype=DTYPE_BF16, B=1, T=32768, H=16, Hkv=2,
                            d=128, m_csa=None, m_hca=128, W=128, gates="hca",
                            q_scale="rsqrt_d"),
    "csa_prefill_128k": dict(kind="prefill", dtype=DTYPE_BF16, B=1, T=131072, H=32,
                             Hkv=4, d=128, m_csa=4, k=512, Hi=4, d_idx=64, m_hca=None,
                             W=128, gates="csa"),
    "decode_1m": dict(kind="decode", dtype=DTYPE_BF16, B=16, H=32, Hkv=1, d=128,
                      N_csa=262144, m_csa=4, k=1024, Hi=4, d_idx=64, N_hca=8192,
                      m_hca=128, W=128, gates="mix"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normal(rng, shape, dtype, scale=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if dtype == DTYPE_BF16:
        return f32_to_bf16_bits(x)
    return x


def _gates(rng, H, spec):
    if spec == "mix":
        return rng.random(size=(H, 3), dtype=np.float32)
    if isinstance(spec, str):
        return np.tile(np.asarray(MODES[spec], dtype=np.float32), (H, 1))
    g = np.asarray(spec, dtype=np.float32)
    return np.tile(g, (H, 1)) if g.ndim == 1 else g


def config(name: str, **overrides) -> dict:
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    cfg["name"] = name
    return cfg


def make_prefill(cfg: dict, seed: int = 0) -> dict:
    """Prefill inputs.  Draw order: Q, K, V, Zk_csa, Zv_csa, Zk_hca, Zv_hca, qI,
    kI, w, gates (branches a workload lacks are skipped)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dt, B, T, H, Hkv, d = cfg["dtype"], cfg["B"], cfg["T"], cfg["H"], cfg["Hkv"], cfg["d"]
    q_scale = 1.0 / math.sqrt(d) if cfg.get("q_scale") == "rsqrt_d" else 1.0
    out = dict(cfg=cfg)
    out["q"] = _normal(rng, (B, T, H, d), dt, q_scale)
    out["k"] = _normal(rng, (B, T, Hkv, d), dt)
    out["v"] = _normal(rng, (B, T, Hkv, d), dt)
    if cfg.get("m_csa"):
        m = cfg["m_csa"]
        out["zk_csa"] = rng.standard_normal((m, Hkv, d), dtype=np.float32) / np.float32(8)
        out["zv_csa"] = rng.standard_normal((m, Hkv, d), dtype=np.float32) / np.float32(8)
    if cfg.get("m_hca"):
        m = cfg["m_hca"]
        out["zk_hca"] = rng.standard_normal((m, Hkv, d), dtype=np.float32) / np.float32(8)
        out["zv_hca"] = rng.standard_normal((m, Hkv, d), dtype=np.float32) / np.float32(8)
    if cfg.get("m_csa"):
        Hi, di = cfg["Hi"], cfg["d_idx"]
        n_csa = T // cfg["m_csa"]
        out["qI"] = _normal(rng, (B, T, Hi, di), dt)
        out["kI"] = _normal(rng, (B, n_csa, di), dt)
        w_h = rng.random(size=(Hi,), dtype=np.float32)
        out["w"] = np.ascontiguousarray(np.broadcast_to(w_h, (B, T, Hi)))
    out["gates"] = _gates(rng, H, cfg.get("gates", "mix"))
    return out


def make_decode(cfg: dict, seed: int = 0) -> dict:
    """Decode inputs.  Draw order: Q, window K, window V, Kc_csa, Vc_csa, kI,
    Kc_hca, Vc_hca, qI, w, gates.  The query sits at the last position of a raw
    window that follows N_csa * m_csa tokens of compressed history."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dt, B, H, Hkv, d, W = cfg["dtype"], cfg["B"], cfg["H"], cfg["Hkv"], cfg["d"], cfg["W"]
    Nc, Nh, Hi, di = cfg["N_csa"], cfg["N_hca"], cfg["Hi"], cfg["d_idx"]
    out = dict(cfg=cfg)
    out["q"] = _normal(rng, (B, 1, H, d), dt)
    out["k_win"] = _normal(rng, (B, W, Hkv, d), dt)
    out["v_win"] = _normal(rng, (B, W, Hkv, d), dt)
    out["k_csa"] = _normal(rng, (B, Nc, Hkv, d), dt)
    out["v_csa"] = _normal(rng, (B, Nc, Hkv, d), dt)
    out["kI"] = _normal(rng, (B, Nc, di), dt)
    out["k_hca"] = _normal(rng, (B, Nh, Hkv, d), dt)
    out["v_hca"] = _normal(rng, (B, Nh, Hkv, d), dt)
    out["qI"] = _normal(rng, (B, 1, Hi, di), dt)
    w_h = rng.random(size=(Hi,), dtype=np.float32)
    out["w"] = np.ascontiguousarray(np.broadcast_to(w_h, (B, 1, Hi)))
    out["gates"] = _gates(rng, H, cfg.get("gates", "mix"))
    out["raw_pos0"] = Nc * cfg["m_csa"]
    out["q_pos0"] = Nc * cfg["m_csa"] + W - 1
    return out


def token_gates(B, T, H, kind, seed: int = 0) -> np.ndarray:
    """Per-token gates [B, T, H, 3] float32: kind "weights" draws U(0,1) with
    exact zeros planted (head 0 never uses HCA, head 1 skips CSA on the first
    half of the tokens) so that branch skipping is exercised; kind "logits"
    draws N(0, 2^2) logits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "weights":
        g = rng.random(size=(B, T, H, 3), dtype=np.float32)
        g[:, :, 0, 0] = 0.0
        if H > 1:
            g[:, : T // 2, 1, 1] = 0.0
        return g
    if kind == "logits":
        return (rng.standard_normal(size=(B, T, H, 3), dtype=np.float32) * np.float32(2.0))
    raise ValueError(f"unknown gate kind {kind}")


def make_append(*, B, Hkv, d, W, m_csa, m_hca, d_idx, cap_csa, cap_hca, steps, dtype=DTYPE_BF16,
                zero_state=False, seed: int = 0) -> dict:
    """Decode cache-maintenance inputs.  Draw order: ring K, ring V, ring kI,
    Zk_csa, Zv_csa, Zk_hca, Zv_hca, Z_I, cache K/V (CSA, HCA), cache kI, new K,
    new V, new kI.  The state is random (so a stray write shows) unless
    zero_state; new rows are [steps, B, ...]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = dict(B=B, Hkv=Hkv, d=d, W=W, m_csa=m_csa, m_hca=m_hca, d_idx=d_idx, dtype=dtype)
    st = (lambda shape: np.zeros(shape, np.uint16 if dtype == DTYPE_BF16 else np.float32)) if zero_state \
        else (lambda shape: _normal(rng, shape, dtype))
    out["k_ring"] = st((B, W, Hkv, d))
    out["v_ring"] = st((B, W, Hkv, d))
    out["kI_ring"] = st((B, W, d_idx))
    out["zk_csa"] = rng.standard_normal(size=(m_csa, Hkv, d), dtype=np.float32)
    out["zv_csa"] = rng.standard_normal(size=(m_csa, Hkv, d), dtype=np.float32)
    out["zk_hca"] = rng.standard_normal(size=(m_hca, Hkv, d), dtype=np.float32)
    out["zv_hca"] = rng.standard_normal(size=(m_hca, Hkv, d), dtype=np.float32)
    out["zI"] = rng.standard_normal(size=(m_csa, d_idx), dtype=np.float32)
    out["k_csa"] = st((B, cap_csa, Hkv, d))
    out["v_csa"] = st((B, cap_csa, Hkv, d))
    out["k_hca"] = st((B, cap_hca, Hkv, d))
    out["v_hca"] = st((B, cap_hca, Hkv, d))
    out["kI_csa"] = st((B, cap_csa, d_idx))
    out["k_new"] = _normal(rng, (steps, B, Hkv, d), dtype)
    out["v_new"] = _normal(rng, (steps, B, Hkv, d), dtype)
    out["kI_new"] = _normal(rng, (steps, B, d_idx), dtype)
    return out


def make_decode_stream(*, B, H, Hkv, d, d_idx, Hi, lengths, steps, dtype=DTYPE_BF16, seed: int = 0) -> dict:
    """Token streams for a multi-step decode of B sequences whose histories
    have different lengths.  Draw order: per sequence b, raw K, V [L_b, Hkv, d]
    and indexer keys kI [L_b, d_idx] with L_b = lengths[b] + steps (positions
    0 .. L_b - 1; the last `steps` are the ones decoded); then per step and
    sequence the query q [steps, B, H, d], indexer query qI [steps, B, Hi,
    d_idx], indexer weights w [steps, B, Hi] ~ U(0,1); then per-head gates
    [H, 3] ~ U(0,1) and the compression logits (CSA K, V, indexer keys; HCA
    K, V) ~ N(0,1)/8, drawn at their largest block size (1024 rows) so that
    any ratio takes the leading rows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = dict(B=B, H=H, Hkv=Hkv, d=d, d_idx=d_idx, Hi=Hi, lengths=list(lengths), steps=steps, dtype=dtype)
    out["k_seq"], out["v_seq"], out["kI_seq"] = [], [], []
    for b in range(B):
        L = lengths[b] + steps
        out["k_seq"].append(_normal(rng, (L, Hkv, d), dtype))
        out["v_seq"].append(_normal(rng, (L, Hkv, d), dtype))
        out["kI_seq"].append(_normal(rng, (L, d_idx), dtype))
    out["q"] = _normal(rng, (steps, B, H, d), dtype)
    out["qI"] = _normal(rng, (steps, B, Hi, d_idx), dtype)
    out["w"] = rng.random(size=(steps, B, Hi), dtype=np.float32)
    out["gates"] = rng.random(size=(H, 3), dtype=np.float32)
    for name, ch in (("zk_csa", d), ("zv_csa", d), ("zI", d_idx), ("zk_hca", d), ("zv_hca", d)):
        shape = (1024, Hkv, ch) if name != "zI" else (1024, ch)
        out[name] = (rng.standard_normal(size=shape, dtype=np.float32) / np.float32(8.0)).astype(np.float32)
    return out


def make_inputs(name: str, seed: int = 0, **overrides) -> dict:
    cfg = config(name, **overrides)
    if cfg["kind"] == "decode":
        return make_decode(cfg, seed)
    return make_prefill(cfg, seed)


def make_backward(name: str, seed: int = 0, gate_mode: int = 0, **overrides) -> dict:
    """Inputs of the prefill backward: make_inputs(name, seed, **overrides),
    plus, from a second stream PCG64([seed, 1]) in this order, the incoming
    gradient dout ~ N(0, 1) [B, T, H, d] (storage dtype) and, for gate_mode 1
    or 2, per-token gates [B, T, H, 3]: U(0, 1) weights (1) or N(0, 1) logits
    (2), which replace the per-head gates."""
    out = make_inputs(name, seed, **overrides)
    cfg = out["cfg"]
    rng = np.random.Generator(np.random.PCG64([seed, 1]))
    B, T, H, d = cfg["B"], cfg["T"], cfg["H"], cfg["d"]
    out["dout"] = _normal(rng, (B, T, H, d), cfg["dtype"])
    if gate_mode == 1:
        out["gates"] = rng.random(size=(B, T, H, 3), dtype=np.float32)
    elif gate_mode == 2:
        out["gates"] = rng.standard_normal(size=(B, T, H, 3), dtype=np.float32)
    return out


def make_rope(*, rows, heads, d, dtype=DTYPE_BF16, max_pos=1 << 20, seed: int = 0) -> dict:
    """RoPE inputs.  Draw order: x [rows, heads, d] ~ N(0, 1), then positions
    U{0, .., max_pos - 1}; row 0 sits at position 0, row 1 is inactive (-1)
    and the last row at max_pos - 1 when there are rows enough."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal(rng, (rows, heads, d), dtype)
    pos = rng.integers(0, max_pos, size=(rows,), dtype=np.int64)
    if rows > 2:
        pos[0], pos[1], pos[-1] = 0, -1, max_pos - 1
    return dict(x=x, pos=pos)


def make_quant(*, n, dtype=DTYPE_BF16, constant=None, seed: int = 0) -> np.ndarray:
    """A flat cache-like tensor of n N(0, 1) draws in storage form (or n
    copies of `constant`)."""
    if constant is not None:
        x = np.full(n, constant, np.float32)
        return f32_to_bf16_bits(x) if dtype == DTYPE_BF16 else x
    rng = np.random.Generator(np.random.PCG64(seed))
    return _normal(rng, (n,), dtype)
