"""Thin ctypes binding of libhybridattn.so (the C interface in include/hybrid_attn.h).

Argument marshalling only: validate torch tensors, allocate outputs and
workspace with torch on the caller's device, pass raw device pointers and the
current HIP stream.  Every step of the computation runs in the HIP kernels;
there is no fallback.  Importing this module does not load the library; the
first call does, and raises if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

DTYPE_BF16 = 0
DTYPE_F32 = 1

SHATTN_OK = 0
SHATTN_EINVAL = -1
SHATTN_EUNSUPPORTED = -2
SHATTN_EWORKSPACE = -3
SHATTN_EHIP = -4

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhybridattn.so")

EXPORTED = (
    "hca_compress_kv",
    "hca_compress_kv_dual",
    "csa_index_topk_workspace_size",
    "csa_index_topk",
    "csa_index_topk_varlen",
    "hybrid_sparse_attn_fwd_workspace_size",
    "hybrid_sparse_attn_fwd",
    "hybrid_sparse_attn_fwd_noalloc",
    "hybrid_sparse_attn_bwd_workspace_size",
    "hybrid_sparse_attn_bwd",
    "hybrid_cache_append",
    "rope_apply",
    "cache_quant4",
    "cache_dequant4",
    "shattn_last_error",
)


class ShattnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class FwdArgs(ctypes.Structure):
    """Mirror of shattn_fwd_args (same field order; C alignment rules)."""
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Tq", ctypes.c_int32), ("H", ctypes.c_int32),
        ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("W", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("gate_mode", ctypes.c_int32),
        ("q_pos0", ctypes.c_int64),
        ("q", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("raw_pos0", ctypes.c_int64),
        ("Tr", ctypes.c_int32),
        ("m_hca", ctypes.c_int32),
        ("k_raw", ctypes.c_void_p),
        ("v_raw", ctypes.c_void_p),
        ("N_hca", ctypes.c_int32),
        ("N_csa", ctypes.c_int32),
        ("k_hca", ctypes.c_void_p),
        ("v_hca", ctypes.c_void_p),
        ("m_csa", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("k_csa", ctypes.c_void_p),
        ("v_csa", ctypes.c_void_p),
        ("idx", ctypes.c_void_p),
        ("gates", ctypes.c_void_p),
        ("q_pos", ctypes.c_void_p),
        ("raw_ring", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("cache_q4", ctypes.c_int32),
        ("reserved1", ctypes.c_int32),
        ("q4_k_hca", ctypes.c_void_p), ("q4_v_hca", ctypes.c_void_p),
        ("q4_k_csa", ctypes.c_void_p), ("q4_v_csa", ctypes.c_void_p),
        ("rope_q", ctypes.c_int32), ("rope_off", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
        ("reserved2", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("split_part", ctypes.c_int32),
        ("reserved3", ctypes.c_int32),
    ]


class AppendArgs(ctypes.Structure):
    """Mirror of shattn_append_args (same field order; C alignment rules)."""
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("W", ctypes.c_int32),
        ("m_csa", ctypes.c_int32), ("m_hca", ctypes.c_int32), ("d_idx", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("pos", ctypes.c_void_p),
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("k_ring", ctypes.c_void_p), ("v_ring", ctypes.c_void_p),
        ("zk_csa", ctypes.c_void_p), ("zv_csa", ctypes.c_void_p),
        ("k_csa", ctypes.c_void_p), ("v_csa", ctypes.c_void_p),
        ("cap_csa", ctypes.c_int64),
        ("zk_hca", ctypes.c_void_p), ("zv_hca", ctypes.c_void_p),
        ("k_hca", ctypes.c_void_p), ("v_hca", ctypes.c_void_p),
        ("cap_hca", ctypes.c_int64),
        ("kI_new", ctypes.c_void_p), ("kI_ring", ctypes.c_void_p),
        ("zI", ctypes.c_void_p), ("kI_csa", ctypes.c_void_p),
        ("dropped", ctypes.c_void_p),
    ]


class BwdArgs(ctypes.Structure):
    """Mirror of shattn_bwd_args (same field order; C alignment rules)."""
    _fields_ = [
        ("struct_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("W", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("gate_mode", ctypes.c_int32),
        ("m_hca", ctypes.c_int32), ("m_csa", ctypes.c_int32), ("k", ctypes.c_int32),
        ("reserved0", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("k_raw", ctypes.c_void_p), ("v_raw", ctypes.c_void_p),
        ("dout", ctypes.c_void_p), ("gates", ctypes.c_void_p),
        ("zk_hca", ctypes.c_void_p), ("zv_hca", ctypes.c_void_p),
        ("k_hca", ctypes.c_void_p), ("v_hca", ctypes.c_void_p),
        ("zk_csa", ctypes.c_void_p), ("zv_csa", ctypes.c_void_p),
        ("k_csa", ctypes.c_void_p), ("v_csa", ctypes.c_void_p),
        ("idx", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("dzk_hca", ctypes.c_void_p), ("dzv_hca", ctypes.c_void_p),
        ("dzk_csa", ctypes.c_void_p), ("dzv_csa", ctypes.c_void_p),
        ("dgates", ctypes.c_void_p),
        ("dk_hca", ctypes.c_void_p), ("dv_hca", ctypes.c_void_p),
        ("dk_csa", ctypes.c_void_p), ("dv_csa", ctypes.c_void_p),
    ]


_lib = None
_lock = threading.Lock()


def load_library(path: str = LIB_PATH):
    """Load libhybridattn.so and declare its signatures (raises if missing)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built; run `python -m sparse_hybrid_attention_amd.build_lib` "
                "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(path)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        lib.hca_compress_kv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
        lib.hca_compress_kv.restype = i32
        lib.hca_compress_kv_dual.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32,
                                             i32, i32, vp]
        lib.hca_compress_kv_dual.restype = i32
        lib.csa_index_topk_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
        lib.csa_index_topk_workspace_size.restype = sz
        lib.csa_index_topk.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i64, i32, i32,
                                       i32, i32, vp, sz, vp]
        lib.csa_index_topk.restype = i32
        lib.csa_index_topk_varlen.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, i32, i32,
                                              i32, i32, vp, sz, vp]
        lib.csa_index_topk_varlen.restype = i32
        lib.hybrid_sparse_attn_fwd_workspace_size.argtypes = [ctypes.POINTER(FwdArgs)]
        lib.hybrid_sparse_attn_fwd_workspace_size.restype = sz
        lib.hybrid_sparse_attn_fwd.argtypes = [ctypes.POINTER(FwdArgs), vp, sz, vp]
        lib.hybrid_sparse_attn_fwd.restype = i32
        lib.hybrid_sparse_attn_fwd_noalloc.argtypes = [ctypes.POINTER(FwdArgs), vp]
        lib.hybrid_sparse_attn_fwd_noalloc.restype = i32
        lib.hybrid_sparse_attn_bwd_workspace_size.argtypes = [ctypes.POINTER(BwdArgs)]
        lib.hybrid_sparse_attn_bwd_workspace_size.restype = sz
        lib.hybrid_sparse_attn_bwd.argtypes = [ctypes.POINTER(BwdArgs), vp, sz, vp]
        lib.hybrid_sparse_attn_bwd.restype = i32
        lib.hybrid_cache_append.argtypes = [ctypes.POINTER(AppendArgs), vp]
        lib.hybrid_cache_append.restype = i32
        lib.rope_apply.argtypes = [vp, vp, i64, i32, i32, i32, i32, ctypes.c_double, i32, vp]
        lib.rope_apply.restype = i32
        lib.cache_quant4.argtypes = [vp, i64, i32, vp, vp, vp]
        lib.cache_quant4.restype = i32
        lib.cache_dequant4.argtypes = [vp, vp, i64, i32, vp, vp]
        lib.cache_dequant4.restype = i32
        lib.shattn_last_error.argtypes = []
        lib.shattn_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(rc: int):
    if rc != SHATTN_OK:
        msg = _lib.shattn_last_error().decode(errors="replace")
        raise ShattnError(rc, msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, dev=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")


# ---------------------------------------------------------------------------
def hca_compress_kv(k, v, zk, zv, m: int, out=None):
    """Block compression of K and V; returns (kc, vc) of shape [B, T//m, Hkv, d]."""
    lib = load_library()
    _need(k, "k")
    _need(v, "v", k.dtype, k.device)
    _need(zk, "zk", torch.float32, k.device)
    _need(zv, "zv", torch.float32, k.device)
    B, T, Hkv, d = k.shape
    if v.shape != k.shape:
        raise ValueError("k and v shapes differ")
    N = T // m if m > 0 else 0
    if out is None:
        kc = torch.empty((B, N, Hkv, d), dtype=k.dtype, device=k.device)
        vc = torch.empty((B, N, Hkv, d), dtype=k.dtype, device=k.device)
    else:
        kc, vc = out
    _check(lib.hca_compress_kv(_ptr(k), _ptr(v), _ptr(zk), _ptr(zv), _ptr(kc), _ptr(vc),
                               B, T, Hkv, d, m, _dtype_code(k), _stream(k)))
    return kc, vc


def hca_compress_kv_dual(k, v, zk1, zv1, m1: int, zk2, zv2, m2: int):
    """Both ratios in one pass; returns ((kc1, vc1), (kc2, vc2))."""
    lib = load_library()
    _need(k, "k")
    _need(v, "v", k.dtype, k.device)
    for name, z in (("zk1", zk1), ("zv1", zv1), ("zk2", zk2), ("zv2", zv2)):
        _need(z, name, torch.float32, k.device)
    B, T, Hkv, d = k.shape
    kc1 = torch.empty((B, T // m1, Hkv, d), dtype=k.dtype, device=k.device)
    vc1 = torch.empty_like(kc1)
    kc2 = torch.empty((B, T // m2, Hkv, d), dtype=k.dtype, device=k.device)
    vc2 = torch.empty_like(kc2)
    _check(lib.hca_compress_kv_dual(_ptr(k), _ptr(v), _ptr(zk1), _ptr(zv1), _ptr(kc1), _ptr(vc1), m1,
                                    _ptr(zk2), _ptr(zv2), _ptr(kc2), _ptr(vc2), m2, B, T, Hkv, d,
                                    _dtype_code(k), _stream(k)))
    return (kc1, vc1), (kc2, vc2)


def csa_index_topk_workspace_size(B, Tq, N, Hi, d_idx, k) -> int:
    return int(load_library().csa_index_topk_workspace_size(B, Tq, N, Hi, d_idx, k))


def csa_index_topk(qI, kI, w, q_pos0, m: int, W: int, k: int, out=None, ws=None):
    """Per-query top-k CSA entries; returns int32 [B, Tq, k] (ascending, -1 padded).

    q_pos0: an int (every sequence's row 0 at that position), or a device
    int64 tensor [B] of per-sequence positions (csa_index_topk_varlen)."""
    lib = load_library()
    _need(qI, "qI")
    _need(kI, "kI", qI.dtype, qI.device)
    _need(w, "w", torch.float32, qI.device)
    B, Tq, Hi, d_idx = qI.shape
    N = kI.shape[1]
    if kI.shape[0] != B or kI.shape[2] != d_idx or tuple(w.shape) != (B, Tq, Hi):
        raise ValueError("indexer shapes disagree")
    idx = out if out is not None else torch.empty((B, Tq, k), dtype=torch.int32, device=qI.device)
    nbytes = int(lib.csa_index_topk_workspace_size(B, Tq, N, Hi, d_idx, k))
    if ws is None and nbytes > 0:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=qI.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    if isinstance(q_pos0, torch.Tensor):
        _need(q_pos0, "q_pos", torch.int64, qI.device)
        if tuple(q_pos0.shape) != (B,):
            raise ValueError("q_pos must be [B]")
        _check(lib.csa_index_topk_varlen(_ptr(qI), _ptr(kI), _ptr(w), _ptr(idx), B, Tq, N, Hi, d_idx,
                                         _ptr(q_pos0), m, W, k, _dtype_code(qI), _ptr(ws), ws_bytes,
                                         _stream(qI)))
        return idx
    _check(lib.csa_index_topk(_ptr(qI), _ptr(kI), _ptr(w), _ptr(idx), B, Tq, N, Hi, d_idx,
                              int(q_pos0), m, W, k, _dtype_code(qI), _ptr(ws), ws_bytes,
                              _stream(qI)))
    return idx


def make_fwd_args(q, k_raw, v_raw, gates, W, *, q_pos0=0, raw_pos0=0, hca=None, csa=None,
                  sm_scale=0.0, out=None, gate_logits=False, q_pos=None, raw_ring=False, rope_q=None,
                  split_part=0):
    """Build the argument struct (and the output tensor) for hybrid_sparse_attn_fwd.

    hca = (k_hca, v_hca, m_hca) or None; csa = (k_csa, v_csa, idx) or None.
    A 4-bit cache adds its (min, step) tensors: hca = (k_codes, v_codes, m_hca,
    (params_k, params_v)), csa = (k_codes, v_codes, idx, (params_k, params_v)),
    codes uint8 [B, N, Hkv, d/2] and params float32 [2] as cache_quant4 writes
    them.
    gates: [H, 3] per-head weights, or [B, Tq, H, 3] per-token weights (or,
    with gate_logits, per-token logits the kernel softmaxes over the branches).
    q_pos: device int64 [B] per-sequence positions (needs raw_ring); raw_ring:
    k_raw / v_raw are rings, position t in row t % Tr.
    rope_q: (rope_off, rope_dim, base) to rotate q by RoPE as it is loaded.
    split_part: 0 whole attention; 1 / 2 the two calls of a split launch.
    Returns (FwdArgs, out, keepalive tuple)."""
    _need(q, "q")
    dev = q.device
    _need(k_raw, "k_raw", q.dtype, dev)
    _need(v_raw, "v_raw", q.dtype, dev)
    _need(gates, "gates", torch.float32, dev)
    B, Tq, H, d = q.shape
    Tr, Hkv = k_raw.shape[1], k_raw.shape[2]
    if tuple(gates.shape) == (H, 3) and not gate_logits:
        gate_mode = 0
    elif tuple(gates.shape) == (B, Tq, H, 3):
        gate_mode = 2 if gate_logits else 1
    else:
        raise ValueError(f"gates must be [H, 3] or [B, Tq, H, 3] (logits: per token only), got {tuple(gates.shape)}")
    if out is None:
        out = torch.empty_like(q)
    a = FwdArgs()
    a.gate_mode = gate_mode
    a.struct_size = ctypes.sizeof(FwdArgs)
    a.dtype = _dtype_code(q)
    a.B, a.Tq, a.H, a.Hkv, a.d, a.W = B, Tq, H, Hkv, d, W
    a.sm_scale = sm_scale
    a.q_pos0 = int(q_pos0)
    a.q = q.data_ptr()
    a.out = out.data_ptr()
    a.raw_pos0 = int(raw_pos0)
    a.Tr = Tr
    a.k_raw, a.v_raw = k_raw.data_ptr(), v_raw.data_ptr()
    keep = [q, k_raw, v_raw, gates, out]
    def cache(t, name, params, bit):
        if params is None:
            _need(t, name, q.dtype, dev)
            if tuple(t.shape[2:]) != (Hkv, d):
                raise ValueError(f"{name} must be [B, N, Hkv, d]")
            return
        _need(t, name, torch.uint8, dev)
        if tuple(t.shape[2:]) != (Hkv, d // 2):
            raise ValueError(f"{name} (4-bit codes) must be [B, N, Hkv, d/2]")
        a.cache_q4 |= bit

    def q4params(pair, names):
        for t, n in zip(pair, names):
            _need(t, n, torch.float32, dev)
            if t.numel() != 2:
                raise ValueError(f"{n} must hold (min, step)")
            setattr(a, n, t.data_ptr())
            keep.append(t)
    if hca is not None:
        kh, vh, mh = hca[:3]
        ph = hca[3] if len(hca) > 3 else None
        cache(kh, "k_hca", ph, 1)
        cache(vh, "v_hca", ph, 1)
        if ph is not None:
            q4params(ph, ("q4_k_hca", "q4_v_hca"))
        a.k_hca, a.v_hca, a.m_hca, a.N_hca = kh.data_ptr(), vh.data_ptr(), int(mh), kh.shape[1]
        keep += [kh, vh]
    if csa is not None:
        kc, vc, idx = csa[:3]
        pc = csa[3] if len(csa) > 3 else None
        cache(kc, "k_csa", pc, 2)
        cache(vc, "v_csa", pc, 2)
        if pc is not None:
            q4params(pc, ("q4_k_csa", "q4_v_csa"))
        _need(idx, "idx", torch.int32, dev)
        a.k_csa, a.v_csa, a.idx = kc.data_ptr(), vc.data_ptr(), idx.data_ptr()
        a.N_csa, a.k = kc.shape[1], idx.shape[-1]
        keep += [kc, vc, idx]
    a.gates = gates.data_ptr()
    a.raw_ring = 1 if raw_ring else 0
    a.split_part = int(split_part)
    if rope_q is not None:
        a.rope_q = 1
        a.rope_off, a.rope_dim, a.rope_base = int(rope_q[0]), int(rope_q[1]), float(rope_q[2])
    if q_pos is not None:
        _need(q_pos, "q_pos", torch.int64, dev)
        if tuple(q_pos.shape) != (B,):
            raise ValueError("q_pos must be [B]")
        a.q_pos = q_pos.data_ptr()
        keep.append(q_pos)
    return a, out, tuple(keep)


def hybrid_sparse_attn_fwd_workspace_size(args: FwdArgs) -> int:
    return int(load_library().hybrid_sparse_attn_fwd_workspace_size(ctypes.byref(args)))


def hybrid_sparse_attn_fwd(q, k_raw, v_raw, gates, W, *, q_pos0=0, raw_pos0=0, hca=None,
                           csa=None, sm_scale=0.0, out=None, ws=None, gate_logits=False, q_pos=None,
                           raw_ring=False, rope_q=None):
    """Gated hybrid attention forward; returns out [B, Tq, H, d]."""
    lib = load_library()
    a, out, _keep = make_fwd_args(q, k_raw, v_raw, gates, W, q_pos0=q_pos0, raw_pos0=raw_pos0,
                                  hca=hca, csa=csa, sm_scale=sm_scale, out=out, gate_logits=gate_logits,
                                  q_pos=q_pos, raw_ring=raw_ring, rope_q=rope_q)
    nbytes = int(lib.hybrid_sparse_attn_fwd_workspace_size(ctypes.byref(a)))
    if ws is None and nbytes > 0:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.hybrid_sparse_attn_fwd(ctypes.byref(a), _ptr(ws), ws_bytes, _stream(q)))
    return out


def hybrid_sparse_attn_fwd_noalloc(q, k_raw, v_raw, gates, W, *, q_pos0=0, raw_pos0=0, hca=None, csa=None,
                                   sm_scale=0.0, out=None, gate_logits=False, q_pos=None, raw_ring=False,
                                   rope_q=None):
    """hybrid_sparse_attn_fwd without a caller workspace (the library's own
    per-GPU scratch array); returns out [B, Tq, H, d]."""
    lib = load_library()
    a, out, _keep = make_fwd_args(q, k_raw, v_raw, gates, W, q_pos0=q_pos0, raw_pos0=raw_pos0,
                                  hca=hca, csa=csa, sm_scale=sm_scale, out=out, gate_logits=gate_logits,
                                  q_pos=q_pos, raw_ring=raw_ring, rope_q=rope_q)
    _check(lib.hybrid_sparse_attn_fwd_noalloc(ctypes.byref(a), _stream(q)))
    return out


def make_bwd_args(q, k_raw, v_raw, gates, dout, W, *, hca=None, csa=None, sm_scale=0.0, gate_logits=False,
                  cache_grads=False):
    """Build the argument struct and the gradient tensors for hybrid_sparse_attn_bwd.

    hca = (zk_hca, zv_hca, k_hca, v_hca, m_hca) or None; csa = (zk_csa, zv_csa,
    k_csa, v_csa, m_csa, idx) or None (caches: the forward's compressed K/V).
    cache_grads: also return the gradients of the compressed caches.
    Returns (BwdArgs, dict of float32 gradient tensors, keepalive tuple)."""
    _need(q, "q")
    dev = q.device
    for t, n in ((k_raw, "k_raw"), (v_raw, "v_raw"), (dout, "dout")):
        _need(t, n, q.dtype, dev)
    _need(gates, "gates", torch.float32, dev)
    B, T, H, d = q.shape
    Hkv = k_raw.shape[2]
    if tuple(k_raw.shape) != (B, T, Hkv, d) or tuple(v_raw.shape) != (B, T, Hkv, d) or dout.shape != q.shape:
        raise ValueError("k_raw / v_raw must be [B, T, Hkv, d] and dout the shape of q")
    if tuple(gates.shape) == (H, 3) and not gate_logits:
        gate_mode = 0
    elif tuple(gates.shape) == (B, T, H, 3):
        gate_mode = 2 if gate_logits else 1
    else:
        raise ValueError(f"gates must be [H, 3] or [B, T, H, 3] (logits: per token only), got {tuple(gates.shape)}")
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"dq": torch.empty((B, T, H, d), **f32), "dk": torch.empty((B, T, Hkv, d), **f32),
         "dv": torch.empty((B, T, Hkv, d), **f32), "dgates": torch.empty(tuple(gates.shape), **f32)}
    a = BwdArgs()
    a.struct_size = ctypes.sizeof(BwdArgs)
    a.dtype = _dtype_code(q)
    a.B, a.T, a.H, a.Hkv, a.d, a.W = B, T, H, Hkv, d, W
    a.sm_scale = sm_scale
    a.gate_mode = gate_mode
    a.q, a.k_raw, a.v_raw, a.dout, a.gates = (t.data_ptr() for t in (q, k_raw, v_raw, dout, gates))
    keep = [q, k_raw, v_raw, dout, gates]
    for name, br in (("hca", hca), ("csa", csa)):
        if br is None:
            continue
        zk, zv, kc, vc, m = br[:5]
        _need(zk, "zk_" + name, torch.float32, dev)
        _need(zv, "zv_" + name, torch.float32, dev)
        _need(kc, "k_" + name, q.dtype, dev)
        _need(vc, "v_" + name, q.dtype, dev)
        m = int(m)
        if tuple(zk.shape) != (m, Hkv, d) or tuple(zv.shape) != (m, Hkv, d):
            raise ValueError(f"zk_{name} / zv_{name} must be [m, Hkv, d]")
        if tuple(kc.shape) != (B, T // m, Hkv, d) or tuple(vc.shape) != (B, T // m, Hkv, d):
            raise ValueError(f"k_{name} / v_{name} must be [B, T // m, Hkv, d]")
        setattr(a, "m_" + name, m)
        setattr(a, "zk_" + name, zk.data_ptr())
        setattr(a, "zv_" + name, zv.data_ptr())
        setattr(a, "k_" + name, kc.data_ptr())
        setattr(a, "v_" + name, vc.data_ptr())
        g["dzk_" + name] = torch.empty((m, Hkv, d), **f32)
        g["dzv_" + name] = torch.empty((m, Hkv, d), **f32)
        setattr(a, "dzk_" + name, g["dzk_" + name].data_ptr())
        setattr(a, "dzv_" + name, g["dzv_" + name].data_ptr())
        if cache_grads:
            g["dk_" + name] = torch.empty((B, T // m, Hkv, d), **f32)
            g["dv_" + name] = torch.empty((B, T // m, Hkv, d), **f32)
            setattr(a, "dk_" + name, g["dk_" + name].data_ptr())
            setattr(a, "dv_" + name, g["dv_" + name].data_ptr())
        keep += [zk, zv, kc, vc]
        if name == "csa":
            idx = br[5]
            _need(idx, "idx", torch.int32, dev)
            if tuple(idx.shape[:2]) != (B, T) or idx.dim() != 3:
                raise ValueError("idx must be [B, T, k]")
            a.idx, a.k = idx.data_ptr(), idx.shape[2]
            keep.append(idx)
    if csa is not None and a.k == 0:
        raise ValueError("idx must have k >= 1 entries per row for the CSA branch")
    a.dq, a.dk, a.dv, a.dgates = (g[n].data_ptr() for n in ("dq", "dk", "dv", "dgates"))
    return a, g, tuple(keep)


def hybrid_sparse_attn_bwd_workspace_size(args: BwdArgs) -> int:
    return int(load_library().hybrid_sparse_attn_bwd_workspace_size(ctypes.byref(args)))


def hybrid_sparse_attn_bwd(q, k_raw, v_raw, gates, dout, W, *, hca=None, csa=None, sm_scale=0.0,
                           gate_logits=False, cache_grads=False, ws=None):
    """Backward of a prefill through compression and gated hybrid attention;
    returns a dict of float32 gradients (dq, dk, dv, dgates, dzk_hca ...; see
    make_bwd_args)."""
    lib = load_library()
    a, g, _keep = make_bwd_args(q, k_raw, v_raw, gates, dout, W, hca=hca, csa=csa, sm_scale=sm_scale,
                                gate_logits=gate_logits, cache_grads=cache_grads)
    nbytes = int(lib.hybrid_sparse_attn_bwd_workspace_size(ctypes.byref(a)))
    if ws is None and nbytes > 0:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.hybrid_sparse_attn_bwd(ctypes.byref(a), _ptr(ws), ws_bytes, _stream(q)))
    return g


def make_append_args(pos, k_new, v_new, k_ring, v_ring, *, csa=None, hca=None, indexer=None, dropped=None):
    """Argument struct of hybrid_cache_append (tensors are checked here, the
    library checks the rest).  csa / hca: (m, zk, zv, k_cache, v_cache);
    indexer: (kI_new, kI_ring, zI, kI_cache) with the CSA ratio."""
    _need(k_new, "k_new")
    dev = k_new.device
    _need(pos, "pos", torch.int64, dev)
    for t, n in ((v_new, "v_new"), (k_ring, "k_ring"), (v_ring, "v_ring")):
        _need(t, n, k_new.dtype, dev)
    B, Hkv, d = k_new.shape
    W = k_ring.shape[1]
    if tuple(pos.shape) != (B,) or v_new.shape != k_new.shape or tuple(k_ring.shape) != (B, W, Hkv, d) \
            or k_ring.shape != v_ring.shape:
        raise ValueError("cache_append: pos / new rows / ring shapes disagree")
    a = AppendArgs()
    a.struct_size = ctypes.sizeof(AppendArgs)
    a.dtype = _dtype_code(k_new)
    a.B, a.Hkv, a.d, a.W = B, Hkv, d, W
    a.pos = pos.data_ptr()
    a.k_new, a.v_new, a.k_ring, a.v_ring = k_new.data_ptr(), v_new.data_ptr(), k_ring.data_ptr(), v_ring.data_ptr()
    keep = [pos, k_new, v_new, k_ring, v_ring]
    for name, br in (("csa", csa), ("hca", hca)):
        if br is None:
            continue
        m, zk, zv, kc, vc = br
        _need(zk, f"zk_{name}", torch.float32, dev)
        _need(zv, f"zv_{name}", torch.float32, dev)
        _need(kc, f"k_{name}", k_new.dtype, dev)
        _need(vc, f"v_{name}", k_new.dtype, dev)
        if tuple(zk.shape) != (m, Hkv, d) or zk.shape != zv.shape or kc.shape != vc.shape \
                or kc.shape[0] != B or tuple(kc.shape[2:]) != (Hkv, d):
            raise ValueError(f"cache_append: {name} logits / cache shapes disagree")
        setattr(a, f"m_{name}", m)
        setattr(a, f"zk_{name}", zk.data_ptr())
        setattr(a, f"zv_{name}", zv.data_ptr())
        setattr(a, f"k_{name}", kc.data_ptr())
        setattr(a, f"v_{name}", vc.data_ptr())
        setattr(a, f"cap_{name}", kc.shape[1])
        keep += [zk, zv, kc, vc]
    if indexer is not None:
        kin, kir, zI, kic = indexer
        _need(kin, "kI_new", k_new.dtype, dev)
        _need(kir, "kI_ring", k_new.dtype, dev)
        _need(zI, "zI", torch.float32, dev)
        _need(kic, "kI_csa", k_new.dtype, dev)
        d_idx = kin.shape[1]
        if csa is None or tuple(kin.shape) != (B, d_idx) or tuple(kir.shape) != (B, W, d_idx) \
                or tuple(zI.shape) != (csa[0], d_idx) or tuple(kic.shape) != (B, csa[3].shape[1], d_idx):
            raise ValueError("cache_append: indexer-key shapes disagree (or no CSA ratio)")
        a.d_idx = d_idx
        a.kI_new, a.kI_ring, a.zI, a.kI_csa = kin.data_ptr(), kir.data_ptr(), zI.data_ptr(), kic.data_ptr()
        keep += [kin, kir, zI, kic]
    if dropped is not None:
        _need(dropped, "dropped", torch.int32, dev)
        a.dropped = dropped.data_ptr()
        keep.append(dropped)
    return a, keep


def cache_append(pos, k_new, v_new, k_ring, v_ring, *, csa=None, hca=None, indexer=None, dropped=None):
    """One decode step of cache maintenance (rings and caches updated in place)."""
    lib = load_library()
    a, _keep = make_append_args(pos, k_new, v_new, k_ring, v_ring, csa=csa, hca=hca, indexer=indexer,
                                dropped=dropped)
    _check(lib.hybrid_cache_append(ctypes.byref(a), _stream(k_new)))


def rope_apply(x, pos, *, rope_off: int = 0, rope_dim: int = None, base: float = 10000.0):
    """Rotary position embedding in place on channels [rope_off, rope_off +
    rope_dim) of every head.  x: [..., heads, d] contiguous; pos: int64 with
    one position per row (x.numel() / (heads * d) rows; negative: unchanged)."""
    _need(x, "x")
    _need(pos, "pos", torch.int64, x.device)
    if x.dim() < 2:
        raise ValueError("rope_apply: x must be [..., heads, d]")
    heads, d = x.shape[-2], x.shape[-1]
    rows = x.numel() // (heads * d) if heads * d else 0
    if pos.numel() != rows:
        raise ValueError(f"rope_apply: {pos.numel()} positions for {rows} rows")
    if rope_dim is None:
        rope_dim = d - rope_off
    lib = load_library()
    _check(lib.rope_apply(_ptr(x), _ptr(pos), rows, heads, d, rope_off, rope_dim, float(base), _dtype_code(x),
                          _stream(x)))
    return x


def cache_quant4(x, codes=None, params=None):
    """4-bit storage of a cache tensor: returns (codes uint8 [ceil(n/2)],
    params float32 [2] = (min, step)), both on x's device."""
    _need(x, "x")
    n = x.numel()
    if codes is None:
        codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=x.device)
    if params is None:
        params = torch.empty(2, dtype=torch.float32, device=x.device)
    _need(codes, "codes", torch.uint8, x.device)
    _need(params, "params", torch.float32, x.device)
    if codes.numel() != (n + 1) // 2 or params.numel() != 2:
        raise ValueError("cache_quant4: codes needs ceil(n/2) bytes and params 2 floats")
    lib = load_library()
    _check(lib.cache_quant4(_ptr(x), n, _dtype_code(x), _ptr(codes), _ptr(params), _stream(x)))
    return codes, params


def cache_dequant4(codes, params, out):
    """Decode cache_quant4's codes into out (its dtype and element count)."""
    _need(out, "out")
    _need(codes, "codes", torch.uint8, out.device)
    _need(params, "params", torch.float32, out.device)
    n = out.numel()
    if codes.numel() != (n + 1) // 2 or params.numel() != 2:
        raise ValueError("cache_dequant4: codes needs ceil(n/2) bytes and params 2 floats")
    lib = load_library()
    _check(lib.cache_dequant4(_ptr(codes), _ptr(params), n, _dtype_code(out), _ptr(out), _stream(out)))
    return out


class HybridPipeline:
    """One pass of the forward hot path with every buffer allocated up front.

    Prefill: compress K/V for CSA (m_csa) and HCA (m_hca), score + select the
    CSA entries, gated attention.  Decode: the caches are given; select, then
    attend.  `run()` only enqueues the kernels (C calls with prepared
    arguments) on the current stream; it allocates nothing.
    """

    def __init__(self, *, q, gates, W, k_raw, v_raw, q_pos0=0, raw_pos0=0,
                 zk_csa=None, zv_csa=None, m_csa=None, zk_hca=None, zv_hca=None, m_hca=None,
                 qI=None, kI=None, w=None, k=None,
                 k_csa=None, v_csa=None, k_hca=None, v_hca=None, q4_hca=None, q4_csa=None,
                 rope_q=None, rope_fused=True, overlap=False):
        """Decode with 4-bit caches: k_hca / v_hca (k_csa / v_csa) are the
        codes [B, N, Hkv, d/2] and q4_hca (q4_csa) their (params_k, params_v).
        rope_q = (rope_off, rope_dim, base): RoPE of q at each row's position,
        inside the attention's Q load (rope_fused) or as a rope_apply launch
        on q before it (which turns q in place at every run).
        overlap: when the attention splits its key list (decode), its window
        and HCA items run on a second stream while the indexer runs, and the
        CSA items and the merge follow on this stream.  Off by default: at the
        1M-token decode shape the indexer fills the chip, and the items run
        beside it slow it by more than they save."""
        lib = load_library()
        self.lib = lib
        dev = q.device
        self.stream = torch.cuda.current_stream(dev)
        self.calls = []      # (name, function, args)
        self.keep = [q, gates, k_raw, v_raw, qI, kI, w]
        dt = _dtype_code(q)
        B, Tq, H, d = q.shape
        Tr, Hkv = k_raw.shape[1], k_raw.shape[2]
        s = ctypes.c_void_p(self.stream.cuda_stream)
        # compression (prefill): caches are produced from the raw K/V, both
        # ratios in one pass when the fused kernel supports them
        if zk_csa is not None:
            k_csa = torch.empty((B, Tr // m_csa, Hkv, d), dtype=q.dtype, device=dev)
            v_csa = torch.empty_like(k_csa)
            self.keep += [zk_csa, zv_csa]
        if zk_hca is not None:
            k_hca = torch.empty((B, Tr // m_hca, Hkv, d), dtype=q.dtype, device=dev)
            v_hca = torch.empty_like(k_hca)
            self.keep += [zk_hca, zv_hca]
        if zk_csa is not None and zk_hca is not None and 8 % m_csa == 0 and m_hca % 8 == 0 and m_hca <= 1024:
            self.calls.append(("compress_dual", lib.hca_compress_kv_dual,
                               (_ptr(k_raw), _ptr(v_raw), _ptr(zk_csa), _ptr(zv_csa), _ptr(k_csa), _ptr(v_csa),
                                m_csa, _ptr(zk_hca), _ptr(zv_hca), _ptr(k_hca), _ptr(v_hca), m_hca, B, Tr, Hkv,
                                d, dt, s)))
        else:
            if zk_csa is not None:
                self.calls.append(("compress_csa", lib.hca_compress_kv,
                                   (_ptr(k_raw), _ptr(v_raw), _ptr(zk_csa), _ptr(zv_csa), _ptr(k_csa),
                                    _ptr(v_csa), B, Tr, Hkv, d, m_csa, dt, s)))
            if zk_hca is not None:
                self.calls.append(("compress_hca", lib.hca_compress_kv,
                                   (_ptr(k_raw), _ptr(v_raw), _ptr(zk_hca), _ptr(zv_hca), _ptr(k_hca),
                                    _ptr(v_hca), B, Tr, Hkv, d, m_hca, dt, s)))
        self.k_csa, self.v_csa, self.k_hca, self.v_hca = k_csa, v_csa, k_hca, v_hca
        idx = None
        if qI is not None:
            Bq, Tq_i, Hi, d_idx = qI.shape
            N = kI.shape[1]
            idx = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
            nbytes = int(lib.csa_index_topk_workspace_size(B, Tq, N, Hi, d_idx, k))
            ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
            self.keep.append(ws)
            self.calls.append(("index_topk", lib.csa_index_topk,
                               (_ptr(qI), _ptr(kI), _ptr(w), _ptr(idx), B, Tq, N, Hi, d_idx,
                                int(q_pos0), m_csa, W, k, _dtype_code(qI), _ptr(ws) if nbytes else None,
                                nbytes, s)))
        self.idx = idx
        hca = None if k_hca is None else (k_hca, v_hca, m_hca) + (() if q4_hca is None else (q4_hca,))
        csa = None if idx is None else (k_csa, v_csa, idx) + (() if q4_csa is None else (q4_csa,))
        self.q4_hca, self.q4_csa = q4_hca is not None, q4_csa is not None
        if rope_q is not None and not rope_fused:
            pos = (torch.arange(Tq, dtype=torch.int64, device=dev) + int(q_pos0)).repeat(B)
            self.keep.append(pos)
            self.calls.append(("rope_q", lib.rope_apply,
                               (_ptr(q), _ptr(pos), B * Tq, H, d, int(rope_q[0]), int(rope_q[1]),
                                float(rope_q[2]), dt, s)))
        a, out, keep = make_fwd_args(q, k_raw, v_raw, gates, W, q_pos0=q_pos0, raw_pos0=raw_pos0,
                                     hca=hca, csa=csa, rope_q=rope_q if rope_fused else None)
        self.args = a
        self.out = out
        self.keep += list(keep)
        nbytes = int(lib.hybrid_sparse_attn_fwd_workspace_size(ctypes.byref(a)))
        self.attn_ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        wsp = _ptr(self.attn_ws) if nbytes else None
        self.part1 = None
        if overlap and nbytes > 0:
            # the same launch in two calls on one workspace: window and HCA
            # items on a second stream (they do not read idx), CSA items and
            # the merge here after the indexer and after the first call
            a1, _o1, k1 = make_fwd_args(q, k_raw, v_raw, gates, W, q_pos0=q_pos0, raw_pos0=raw_pos0, hca=hca,
                                        csa=csa, rope_q=rope_q if rope_fused else None, out=out, split_part=1)
            a.split_part = 2
            self.stream2 = torch.cuda.Stream(device=dev)
            self.ev_start = torch.cuda.Event()
            self.ev_part1 = torch.cuda.Event()
            self.part1 = (lib.hybrid_sparse_attn_fwd,
                          (ctypes.byref(a1), wsp, nbytes, ctypes.c_void_p(self.stream2.cuda_stream)))
            self.keep += [a1] + list(k1)
        self.calls.append(("attention", lib.hybrid_sparse_attn_fwd, (ctypes.byref(a), wsp, nbytes, s)))

    def names(self):
        return [c[0] for c in self.calls]

    def run(self, events=None):
        """Enqueue one pass.  events: optional list of len(calls)+1 torch events
        recorded around the calls on the pipeline's stream."""
        if events is not None:
            events[0].record(self.stream)
        if self.part1 is not None:
            self.ev_start.record(self.stream)
            self.stream2.wait_event(self.ev_start)
            fn, args = self.part1
            rc = fn(*args)
            if rc != SHATTN_OK:
                raise ShattnError(rc, "attention (window and HCA items): " +
                                  self.lib.shattn_last_error().decode(errors="replace"))
            self.ev_part1.record(self.stream2)
        for j, (name, fn, args) in enumerate(self.calls):
            if name == "attention" and self.part1 is not None:
                self.stream.wait_event(self.ev_part1)
            rc = fn(*args)
            if rc != SHATTN_OK:
                raise ShattnError(rc, f"{name}: " + self.lib.shattn_last_error().decode(errors="replace"))
            if events is not None:
                events[j + 1].record(self.stream)
        return self.out
