"""Host-side checks of the C interface (no GPU needed): the library loads and
exports every symbol include/hybrid_attn.h declares, the ctypes struct mirrors
the C layout, and every invalid call returns its documented error code before
touching the GPU."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from sparse_hybrid_attention_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hybrid_attn.h")

# fake, 256-byte aligned device addresses: never dereferenced because every
# call below fails validation on the host
P = ctypes.c_void_p(0x7F0000000000)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from sparse_hybrid_attention_amd import build_lib
        build_lib.build()
    return binding.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SHATTN_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert set(syms) == set(binding.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for s in syms:
        assert s in exported, s
        assert getattr(lib, s) is not None
    # nothing else leaks out of the library
    assert exported == set(syms)


def test_no_unresolved_library_symbols(lib):
    # every kernel the launchers reference is defined in the library itself
    out = subprocess.run(["nm", "-C", "--undefined-only", binding.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    assert not [l for l in out.splitlines() if "shattn" in l]


@pytest.mark.parametrize("cls,cname", [(binding.FwdArgs, "shattn_fwd_args"),
                                       (binding.AppendArgs, "shattn_append_args"),
                                       (binding.BwdArgs, "shattn_bwd_args")])
def test_struct_layout_matches_c(lib, tmp_path, cls, cname):
    fields = [f for f, _ in cls._fields_]
    src = tmp_path / "layout.c"
    body = "\n".join(f'printf("{f} %zu\\n", offsetof({cname}, {f}));' for f in fields)
    src.write_text(f"""#include <stdio.h>
#include <stddef.h>
#include "hybrid_attn.h"
int main(void) {{ printf("size %zu\\n", sizeof({cname})); {body} return 0; }}
""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True).stdout.splitlines())
    assert int(out["size"]) == ctypes.sizeof(cls)
    for f in fields:
        assert int(out[f]) == getattr(cls, f).offset, f


def err(lib):
    return lib.shattn_last_error().decode()


def test_compress_errors(lib):
    f = lib.hca_compress_kv
    assert f(P, P, P, P, P, P, 1, 64, 2, 128, 4, 7, None) == binding.SHATTN_EINVAL
    assert "dtype" in err(lib)
    assert f(P, P, P, P, P, P, 1, 64, 2, 96, 4, 0, None) == binding.SHATTN_EUNSUPPORTED
    assert f(P, P, P, P, P, P, 1, 64, 2, 128, 0, 0, None) == binding.SHATTN_EINVAL
    assert f(P, P, P, P, P, P, 1, 64, 2, 128, 2000, 0, None) == binding.SHATTN_EUNSUPPORTED
    assert f(None, P, P, P, P, P, 1, 64, 2, 128, 4, 0, None) == binding.SHATTN_EINVAL
    assert f(ctypes.c_void_p(0x7F0000000008), P, P, P, P, P, 1, 64, 2, 128, 4, 0, None) == binding.SHATTN_EINVAL
    assert "aligned" in err(lib)
    # nothing to do: T < m is a successful no-op
    assert f(None, None, None, None, None, None, 1, 3, 2, 128, 4, 0, None) == binding.SHATTN_OK


def test_index_errors(lib):
    f = lib.csa_index_topk
    ok = dict(B=1, Tq=16, N=64, Hi=4, d_idx=64, q_pos0=0, m=4, W=8, k=8, dtype=0)

    def call(**kw):
        a = dict(ok, **kw)
        return f(P, P, P, P, a["B"], a["Tq"], a["N"], a["Hi"], a["d_idx"], a["q_pos0"], a["m"], a["W"],
                 a["k"], a["dtype"], None, 0, None)
    assert call(Hi=3) == binding.SHATTN_EUNSUPPORTED
    assert call(d_idx=32) == binding.SHATTN_EUNSUPPORTED
    assert call(k=0) == binding.SHATTN_EINVAL
    assert call(k=5000) == binding.SHATTN_EUNSUPPORTED
    assert call(m=0) == binding.SHATTN_EINVAL
    assert call(dtype=3) == binding.SHATTN_EINVAL
    assert call(q_pos0=-1) == binding.SHATTN_EINVAL
    # decode-shaped call needs a workspace
    assert lib.csa_index_topk_workspace_size(16, 1, 262144, 4, 64, 1024) > 0
    assert call(B=16, Tq=1, N=262144, k=1024) == binding.SHATTN_EWORKSPACE
    assert "workspace" in err(lib)
    # prefill with N <= 2048 keeps every score in LDS: no workspace
    assert lib.csa_index_topk_workspace_size(2, 4096, 2048, 4, 64, 64) == 0
    # ... except at 16 indexer heads, which always take the list pipeline
    assert lib.csa_index_topk_workspace_size(2, 600, 150, 16, 128, 40) >= 8 * 1200 * 40
    assert lib.csa_index_topk_workspace_size(2, 600, 0, 16, 128, 40) == 0
    # longer prefill keeps per-query candidate lists ((key, entry) pairs, at
    # least k per query) in the workspace: it grows with the query rows
    ws1 = lib.csa_index_topk_workspace_size(1, 4096, 8192, 4, 64, 64)
    ws2 = lib.csa_index_topk_workspace_size(2, 4096, 8192, 4, 64, 64)
    assert ws1 >= 8 * 4096 * 64 and ws2 >= 2 * ws1 - 4096
    assert call(B=1, Tq=4096, N=8192, k=64) == binding.SHATTN_EWORKSPACE
    assert f(None, P, P, P, 1, 16, 64, 4, 64, 0, 4, 8, 8, 0, None, 0, None) == binding.SHATTN_EINVAL


def test_probe_library_is_separate(lib):
    # the device measurement probes live in their own library, declared in
    # probe/probes.h; the attention library exports none of them
    probe_lib = os.path.join(os.path.dirname(binding.LIB_PATH), "libshattn_probe.so")
    header = os.path.join(ROOT, "sparse_hybrid_attention_amd", "probe", "probes.h")
    declared = set(re.findall(r"SHATTN_PROBE_API\s+[\w\s\*]+?\b(\w+)\s*\(", open(header).read()))
    assert declared == {"shattn_probe_mfma", "shattn_probe_gather", "shattn_probe_stream"}
    out = subprocess.run(["nm", "-D", "--defined-only", probe_lib], capture_output=True, text=True,
                         check=True).stdout
    assert {l.split()[-1] for l in out.splitlines() if " T " in l} == declared
    main = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True,
                          check=True).stdout
    assert "probe" not in main
    pl = ctypes.CDLL(probe_lib)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    pl.shattn_probe_mfma.argtypes = [i32, i32, i32, vp, vp]
    pl.shattn_probe_gather.argtypes = [vp, i64, i32, i64, i32, i64, i32, i32, vp, vp]
    f = pl.shattn_probe_mfma
    assert f(0, 16, 0, P, None) == -1
    assert f(16, 0, 0, P, None) == -1
    assert f(16, 16, 2, P, None) == -1
    assert f(16, 16, 0, None, None) == -1
    g = pl.shattn_probe_gather
    assert g(P, 1024, 96, 256, 1, 100, 4, 64, P, None) == -1      # row size
    assert g(P, 1024, 256, 128, 1, 100, 4, 64, P, None) == -1     # stride below the row
    assert g(P, 0, 256, 256, 1, 100, 4, 64, P, None) == -1        # no rows
    assert g(P, 1024, 256, 256, 1, 100, 3, 64, P, None) == -1     # depth
    assert g(None, 1024, 256, 256, 1, 100, 4, 64, P, None) == -1  # table
    assert g(P, 1026, 256, 256, 4, 100, 4, 64, P, None) == -1     # slices must divide the rows
    assert g(P, 1024, 256, 256, 9, 100, 4, 64, P, None) == -1     # at most 8 slices


def fwd(**kw):
    a = binding.FwdArgs()
    a.struct_size = ctypes.sizeof(binding.FwdArgs)
    a.dtype, a.B, a.Tq, a.H, a.Hkv, a.d, a.W = 0, 1, 16, 4, 2, 128, 8
    a.q = a.out = a.k_raw = a.v_raw = a.gates = P.value
    a.Tr = 16
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def test_attention_errors(lib):
    f = lib.hybrid_sparse_attn_fwd

    def call(**kw):
        return f(ctypes.byref(fwd(**kw)), None, 0, None)
    assert call(struct_size=8) == binding.SHATTN_EINVAL
    assert call(H=5) == binding.SHATTN_EINVAL
    assert "multiple" in err(lib)
    assert call(d=80) == binding.SHATTN_EUNSUPPORTED
    assert call(H=130, Hkv=1) == binding.SHATTN_EUNSUPPORTED
    assert call(dtype=9) == binding.SHATTN_EINVAL
    assert call(W=0) == binding.SHATTN_EINVAL
    assert call(gate_mode=3) == binding.SHATTN_EINVAL
    assert call(gate_mode=-1) == binding.SHATTN_EINVAL
    assert call(Tr=10) == binding.SHATTN_EINVAL          # window rows missing
    assert "window rows" in err(lib)
    assert call(raw_pos0=4) == binding.SHATTN_EINVAL     # first rows missing
    assert call(k=8, N_csa=100) == binding.SHATTN_EINVAL  # CSA without caches / idx
    assert call(k=5000, N_csa=0, idx=P.value) == binding.SHATTN_EUNSUPPORTED
    assert call(m_hca=4, N_hca=10) == binding.SHATTN_EINVAL
    assert call(q=0x7F0000000004) == binding.SHATTN_EINVAL
    assert call(sm_scale=float("nan")) == binding.SHATTN_EINVAL
    # decode-shaped split launch needs a workspace
    a = fwd(B=1, Tq=1, H=32, Hkv=1, W=128, Tr=128, q_pos0=1048703, raw_pos0=1048576, m_hca=128, N_hca=8192,
            k_hca=P.value, v_hca=P.value)
    assert lib.hybrid_sparse_attn_fwd_workspace_size(ctypes.byref(a)) > 0
    assert f(ctypes.byref(a), None, 0, None) == binding.SHATTN_EWORKSPACE
    # per-sequence positions read the window from rings
    assert call(q_pos=P.value) == binding.SHATTN_EINVAL           # q_pos without a ring
    assert "raw_ring" in err(lib)
    assert call(raw_ring=2) == binding.SHATTN_EINVAL
    assert call(reserved0=1) == binding.SHATTN_EINVAL
    assert call(raw_ring=1, q_pos=0x7F0000000004) == binding.SHATTN_EINVAL   # misaligned q_pos
    assert call(raw_ring=1, q_pos=P.value, Tr=22) == binding.SHATTN_EINVAL   # ring shorter than W + Tq - 1
    assert "ring" in err(lib)
    ring = fwd(raw_ring=1, q_pos=P.value, Tr=23, B=1, Tq=16)
    assert lib.hybrid_sparse_attn_fwd_workspace_size(ctypes.byref(ring)) == 0
    # 4-bit caches: known bits only, their (min, step) given, bf16 only
    hq = dict(m_hca=4, N_hca=2, k_hca=P.value, v_hca=P.value)
    assert call(cache_q4=4) == binding.SHATTN_EINVAL
    assert call(reserved1=1) == binding.SHATTN_EINVAL
    assert call(cache_q4=1, **hq) == binding.SHATTN_EINVAL
    assert "(min, step)" in err(lib)
    assert call(cache_q4=1, q4_k_hca=P.value, q4_v_hca=0x7F0000000002, **hq) == binding.SHATTN_EINVAL
    assert call(dtype=1, cache_q4=1, q4_k_hca=P.value, q4_v_hca=P.value, **hq) == binding.SHATTN_EUNSUPPORTED
    # RoPE of q at load: even channel range inside d, finite base > 0
    rq = dict(rope_q=1, rope_off=64, rope_dim=64, rope_base=10000.0)
    assert call(**dict(rq, rope_q=2)) == binding.SHATTN_EINVAL
    assert call(**dict(rq, rope_off=63)) == binding.SHATTN_EINVAL
    assert call(**dict(rq, rope_dim=66)) == binding.SHATTN_EINVAL
    assert call(**dict(rq, rope_base=0.0)) == binding.SHATTN_EINVAL
    assert call(**dict(rq, rope_base=float("inf"))) == binding.SHATTN_EINVAL
    assert call(reserved2=1) == binding.SHATTN_EINVAL
    assert call(reserved3=1) == binding.SHATTN_EINVAL
    assert call(split_part=3) == binding.SHATTN_EINVAL
    assert call(split_part=1) == binding.SHATTN_OK        # no split: the first call does nothing
    # empty problem is a no-op
    assert call(B=0) == binding.SHATTN_OK


def test_index_varlen_errors(lib):
    f = lib.csa_index_topk_varlen
    args = lambda qp, **kw: (P, P, P, P, kw.get("B", 2), 1, 64, 4, 64, qp, 4, 8, 8, 0, None, 0, None)
    assert f(*args(None)) == binding.SHATTN_EINVAL
    assert "q_pos" in err(lib)
    assert f(*args(ctypes.c_void_p(0x7F0000000004))) == binding.SHATTN_EINVAL
    assert f(*args(None, B=0)) == binding.SHATTN_OK     # nothing to do


def bwd(**kw):
    a = binding.BwdArgs()
    a.struct_size = ctypes.sizeof(binding.BwdArgs)
    a.dtype, a.B, a.T, a.H, a.Hkv, a.d, a.W = 0, 2, 256, 4, 2, 128, 16
    a.m_hca, a.m_csa, a.k = 64, 4, 8
    for f in ("q", "k_raw", "v_raw", "dout", "gates", "zk_hca", "zv_hca", "k_hca", "v_hca", "zk_csa", "zv_csa",
              "k_csa", "v_csa", "idx", "dq", "dk", "dv", "dzk_hca", "dzv_hca", "dzk_csa", "dzv_csa", "dgates"):
        setattr(a, f, P.value)
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


def test_backward_errors(lib):
    f = lib.hybrid_sparse_attn_bwd

    def call(**kw):
        return f(ctypes.byref(bwd(**kw)), None, 0, None)
    assert f(None, None, 0, None) == binding.SHATTN_EINVAL
    assert call(struct_size=8) == binding.SHATTN_EINVAL
    assert call(reserved0=1) == binding.SHATTN_EINVAL
    assert call(dtype=4) == binding.SHATTN_EINVAL
    assert call(H=3) == binding.SHATTN_EINVAL
    assert call(d=96) == binding.SHATTN_EUNSUPPORTED
    assert call(W=0) == binding.SHATTN_EINVAL
    assert call(gate_mode=3) == binding.SHATTN_EINVAL
    assert call(m_csa=0) == binding.SHATTN_EINVAL              # CSA branch without its ratio
    assert call(m_hca=2048) == binding.SHATTN_EUNSUPPORTED
    assert call(sm_scale=float("inf")) == binding.SHATTN_EINVAL
    assert call(idx=None) == binding.SHATTN_EINVAL
    assert call(zk_hca=None) == binding.SHATTN_EINVAL
    assert call(dzv_csa=None) == binding.SHATTN_EINVAL
    assert call(dq=None) == binding.SHATTN_EINVAL
    assert call(k_raw=0x7F0000000008) == binding.SHATTN_EINVAL    # 16-byte alignment
    assert call(idx=0x7F0000000002) == binding.SHATTN_EINVAL      # 4-byte alignment
    # absent branches need none of their pointers
    a = bwd(m_hca=0, k=0, zk_hca=None, zv_hca=None, k_hca=None, v_hca=None, zk_csa=None, zv_csa=None,
            k_csa=None, v_csa=None, idx=None, dzk_hca=None, dzv_hca=None, dzk_csa=None, dzv_csa=None)
    need = lib.hybrid_sparse_attn_bwd_workspace_size(ctypes.byref(a))
    assert need >= 2 * 256 * 4 * 24                  # softmax statistics: 24 bytes per (row, head)
    assert f(ctypes.byref(a), None, 0, None) == binding.SHATTN_EWORKSPACE
    assert f(ctypes.byref(a), P, need - 1, None) == binding.SHATTN_EWORKSPACE
    assert "workspace" in err(lib)
    # returning the cache gradients shrinks the workspace
    full = bwd()
    given = bwd(dk_hca=P.value, dv_hca=P.value, dk_csa=P.value, dv_csa=P.value)
    assert (lib.hybrid_sparse_attn_bwd_workspace_size(ctypes.byref(full)) -
            lib.hybrid_sparse_attn_bwd_workspace_size(ctypes.byref(given))) >= 2 * 2 * (4 + 64) * 2 * 128 * 4
    assert lib.hybrid_sparse_attn_bwd_workspace_size(ctypes.byref(bwd(d=96))) == 0


def append(**kw):
    a = binding.AppendArgs()
    a.struct_size = ctypes.sizeof(binding.AppendArgs)
    a.dtype = binding.DTYPE_BF16
    a.B, a.Hkv, a.d, a.W = 16, 1, 128, 128
    a.m_csa, a.m_hca, a.d_idx = 4, 128, 64
    for f in ("pos", "k_new", "v_new", "k_ring", "v_ring", "zk_csa", "zv_csa", "k_csa", "v_csa", "zk_hca",
              "zv_hca", "k_hca", "v_hca", "kI_new", "kI_ring", "zI", "kI_csa"):
        setattr(a, f, P.value)
    a.cap_csa, a.cap_hca = 1024, 64
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_cache_append_errors(lib):
    f = lib.hybrid_cache_append

    def call(**kw):
        return f(ctypes.byref(append(**kw)), None)
    assert f(None, None) == binding.SHATTN_EINVAL
    assert call(struct_size=8) == binding.SHATTN_EINVAL
    assert call(reserved0=1) == binding.SHATTN_EINVAL
    assert call(dtype=5) == binding.SHATTN_EINVAL
    assert call(d=96) == binding.SHATTN_EUNSUPPORTED
    assert call(d_idx=32) == binding.SHATTN_EUNSUPPORTED
    assert call(m_hca=256) == binding.SHATTN_EUNSUPPORTED      # block longer than the ring
    assert "W=128" in err(lib)
    assert call(m_csa=0) == binding.SHATTN_EINVAL              # indexer keys without the CSA ratio
    assert call(cap_csa=-1) == binding.SHATTN_EINVAL
    assert call(pos=None) == binding.SHATTN_EINVAL
    assert call(pos=0x7F0000000004) == binding.SHATTN_EINVAL   # int64 array must be 8-byte aligned
    assert call(k_ring=0x7F0000000008) == binding.SHATTN_EINVAL
    assert call(zk_hca=None) == binding.SHATTN_EINVAL
    assert call(kI_csa=None) == binding.SHATTN_EINVAL
    assert call(dropped=0x7F0000000002) == binding.SHATTN_EINVAL
    assert call(B=-1) == binding.SHATTN_EINVAL
    # an empty batch is a no-op
    assert call(B=0) == binding.SHATTN_OK


def test_rope_errors(lib):
    f = lib.rope_apply
    X, P = 0x7F0000000000, 0x7F0000001000   # never dereferenced: every call below fails validation

    def call(x=X, pos=P, rows=4, heads=2, d=128, off=64, rd=64, base=10000.0, dtype=binding.DTYPE_BF16):
        return f(x, pos, rows, heads, d, off, rd, base, dtype, None)
    assert call(dtype=7) == binding.SHATTN_EINVAL
    assert call(rows=-1) == binding.SHATTN_EINVAL
    assert call(heads=0) == binding.SHATTN_EINVAL
    assert call(rd=63) == binding.SHATTN_EINVAL               # odd channel count
    assert call(rd=0) == binding.SHATTN_EINVAL
    assert call(off=66) == binding.SHATTN_EINVAL              # range past d
    assert "inside d=128" in err(lib)
    assert call(off=-2) == binding.SHATTN_EINVAL
    assert call(base=0.0) == binding.SHATTN_EINVAL
    assert call(base=float("inf")) == binding.SHATTN_EINVAL
    assert call(x=None) == binding.SHATTN_EINVAL
    assert call(pos=P + 4) == binding.SHATTN_EINVAL           # int64 array must be 8-byte aligned
    assert call(x=X + 1) == binding.SHATTN_EINVAL             # bf16 elements must be aligned
    # no rows: a no-op
    assert call(rows=0, x=None, pos=None) == binding.SHATTN_OK


def test_quant4_errors(lib):
    q, dq = lib.cache_quant4, lib.cache_dequant4
    X, C, P = 0x7F0000000000, 0x7F0000002000, 0x7F0000004000   # never dereferenced
    assert q(X, 10, 7, C, P, None) == binding.SHATTN_EINVAL        # dtype
    assert q(X, -1, binding.DTYPE_BF16, C, P, None) == binding.SHATTN_EINVAL
    assert q(None, 10, binding.DTYPE_BF16, C, P, None) == binding.SHATTN_EINVAL
    assert q(X, 10, binding.DTYPE_BF16, None, P, None) == binding.SHATTN_EINVAL
    assert q(X + 1, 10, binding.DTYPE_BF16, C, P, None) == binding.SHATTN_EINVAL   # misaligned elements
    assert q(X, 10, binding.DTYPE_F32, C, P + 2, None) == binding.SHATTN_EINVAL    # params 4-byte aligned
    assert q(None, 0, binding.DTYPE_BF16, None, None, None) == binding.SHATTN_OK   # empty: no-op
    assert dq(C, P, 10, 9, X, None) == binding.SHATTN_EINVAL
    assert dq(None, P, 10, binding.DTYPE_BF16, X, None) == binding.SHATTN_EINVAL
    assert dq(C, P, 10, binding.DTYPE_F32, X + 2, None) == binding.SHATTN_EINVAL
    assert "aligned" in err(lib)
    assert dq(None, None, 0, binding.DTYPE_BF16, None, None) == binding.SHATTN_OK


def test_library_refuses_to_fall_back(tmp_path, monkeypatch):
    # a missing library is an error, never a silent CPU path
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        binding.load_library(str(tmp_path / "missing.so"))
