"""Plain float64 CPU oracle of the hybrid sparse attention forward pass.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the CPU-baseline leg of the
benchmark).  It never runs on the product path and shares no code with the HIP
library.

Pages cited (titles as published):
  [Tiny-R2]  "Tiny-R2: A Hybrid Architecture Combining SWA, CSA, HCA, mHC and
             DSMoE Under the DeepSeek V4 Design Paradigm" (project README).
  [V4-blog]  "deepseek-v4" (astro-blog post), section "1. hybrid attn".
  [V4-code]  CSDN article with example PyTorch code for CSA and HCA,
             sections "1. HCA ... 机制实现" and "2. CSA ... 机制实现".
  [V4-arch]  zwxr.cn article on the DeepSeek-V4 architecture figure,
             section "4. SWA 滑动窗口注意力的边界处理".
  [CS336]    CS336 course notes, "Attention Heads 变体" and
             "Attention Alternatives".

Storage convention (shared with the C interface only by specification, not by
code): tensors are numpy arrays in their storage form, ``np.uint16`` holding
bfloat16 bit patterns when ``dtype == DTYPE_BF16`` and ``np.float32`` when
``dtype == DTYPE_F32``.  Logits, indexer weights and gates are float32 always.
Every computation below decodes its inputs exactly to float64 and works in
float64; results that mirror a stored tensor are rounded once, to nearest
even, to the storage dtype.

Readings taken where the pages are silent (each repeated at its function):
  R1  Indexer score of query row t against CSA entry c is
      sum_h w[t,h] * max(0, qI[t,h] . kI[c]), heads summed in order h = 0..Hi-1.
  R2  A compressed entry c of ratio m covers raw positions [c*m, (c+1)*m);
      N = floor(T/m), a trailing partial block is dropped.
  R3  The window of the query at position t is the W positions t-W+1 .. t,
      clipped at 0.  Compressed entries (CSA candidates and HCA entries) are
      visible to t only when they lie wholly before that window:
      (c+1)*m <= t-W+1.
  R4  Top-k keeps the min(k, #visible) visible entries ordered by
      (score descending, entry index ascending); output is ascending entry
      index, padded with -1.  One selection per query row, shared by all
      attention heads.
  R5  Branch key sets: SWA = window; HCA = window + all visible HCA entries;
      CSA = window + the selected CSA entries.  Each branch is one softmax
      over its whole key set, scale 1/sqrt(d) unless given.
  R6  out = g[h,0]*O_HCA + g[h,1]*O_CSA + g[h,2]*O_SWA with the per-head gates
      as given (no renormalisation); an absent branch contributes nothing.
  R7  KV head of query head h is h // (H // Hkv).
  R8  Decode cache maintenance: the raw window is a ring of W rows per
      sequence, the token at position t in slot t % W.  When that token
      completes a block of ratio m ((t + 1) % m == 0), entry c = (t+1)/m - 1
      is the block compression of positions [c*m, (c+1)*m) (needs m <= W, so
      the ring still holds the whole block).  Indexer keys of CSA entries are
      the same compression of per-token indexer keys with their own logits.
      An entry at or beyond a cache's capacity is not stored.
  R9  Per-token gates ([Tiny-R2] 3.2 diagram: branch_gate = Linear + Softmax
      before the weighted sum): gates may be given per (token, head) as
      weights, or as logits whose softmax over the three branches (in the
      order [HCA, CSA, SWA], all three, present or not) gives the weights.
  R10 Rotary position embedding ([Tiny-R2] architecture diagram: RoPE on the
      prepared query, the window keys, the selected CSA keys and the HCA keys;
      parameter block: a rope part of the head dim next to a non-rope part;
      [CS336] "位置编码" paragraph: position as a rotation angle, so that a
      query-key product depends on the position difference).  Channels
      [off, off + R) of every head are rotated in adjacent pairs
      (off + 2i, off + 2i + 1) by the angle pos * base^(-2i/R), as
      (a, b) -> (a cos - b sin, a sin + b cos); base 10000 unless given (the
      pages give none); every other channel is unchanged.  The position of
      each row is the caller's (for a compressed entry: whichever position the
      model assigns it); a row with a negative position is left unchanged.
  R12 Backward pass (the Tiny-R2 training step differentiates the path):
      the gradient of the float64 forward value of the output (before its
      storage rounding) with respect to Q, the raw K/V rows, the compressed
      caches, the compression logits and the gates, given dL/dout.  The
      top-k selection is a fixed input (a selection is not differentiable);
      the storage rounding of the compressed caches is taken as the identity
      (the gradient reaching a cache flows through the block compression to
      the raw rows and the logits).
  R11 4-bit cache storage ([V4-code] section "1. HCA": the merged cache is
      quantised with one minimum and one maximum over the whole tensor, step
      (max - min) / 15, codes rounded and clamped to 0..15, decoded as
      code * step + min; the page keeps one code per byte and names packing
      two per byte as the real layout).  Reading: the decision is taken in
      float32 (x - min) / step with round-half-even, as the page's tensor
      arithmetic does; two codes per byte, element 2j in the low nibble of
      byte j; a constant tensor (step 0) gets code 0 everywhere and decodes to
      its value.
"""
from __future__ import annotations

import math

import numpy as np

DTYPE_BF16 = 0
DTYPE_F32 = 1
DTYPE_F64 = 2   # oracle only: float64 storage (no rounding anywhere), for derivative checks

__all__ = [
    "DTYPE_BF16", "DTYPE_F32", "DTYPE_F64",
    "bf16_bits_to_f64", "f64_to_bf16_bits", "to_f64", "to_storage",
    "block_weights", "compress", "compress_kv",
    "window_bounds", "visible_count",
    "indexer_scores", "select_topk", "index_topk", "index_topk_row",
    "attend", "attn_row", "hybrid_attn_fwd",
    "gate_weights",
    "cache_append",
    "rope",
    "quant4", "dequant4",
    "compress_backward", "attn_row_backward", "hybrid_attn_bwd", "hybrid_path_bwd",
]


# --------------------------------------------------------------------------
# Storage dtypes
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bfloat16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values once, to nearest even, to bfloat16 bit patterns.

    Works from the float64 value directly (no detour through float32, which
    could round twice).  Finite inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)                 # x = mant * 2**expo, |mant| in [0.5, 1)
    # bfloat16 keeps 8 significant bits for normal numbers; below 2**-126 the
    # spacing is fixed at 2**-133 (subnormals).
    normal = expo >= -125
    q_norm = np.ldexp(np.rint(mant * 256.0), expo - 8)
    q_sub = np.ldexp(np.rint(np.ldexp(x, 133)), -133)
    q = np.where(normal, q_norm, q_sub)
    return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def to_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == DTYPE_BF16:
        return bf16_bits_to_f64(a)
    if dtype == DTYPE_F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == DTYPE_F64:
        return np.asarray(a, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype}")


def to_storage(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == DTYPE_BF16:
        return f64_to_bf16_bits(x)
    if dtype == DTYPE_F32:
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == DTYPE_F64:
        return np.asarray(x, dtype=np.float64).copy()
    raise ValueError(f"unknown dtype {dtype}")


# --------------------------------------------------------------------------
# Step 1: block compression  ([V4-code] section 1, the block-merge method:
# a learned [block_size, channels] parameter is softmaxed over the block
# positions and used as per-channel weights of a sum over the block;
# [V4-blog] "CSA" 4:1 diagram; m = 4 for CSA, m = 128 for HCA).
# --------------------------------------------------------------------------
def block_weights(z: np.ndarray) -> np.ndarray:
    """Softmax of the logits z[i, g, ch] over the block position i (axis 0)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max(axis=0, keepdims=True))
    return e / e.sum(axis=0, keepdims=True)


def compress(x: np.ndarray, z: np.ndarray, m: int) -> np.ndarray:
    """xc[b, c, g, ch] = sum_{i<m} P[i, g, ch] * x[b, c*m + i, g, ch] (float64).

    x: [B, T, Hkv, d] float64; z: [m, Hkv, d] logits.  Reading R2: the number
    of entries is floor(T / m); a trailing partial block is dropped.
    """
    B, T, Hkv, d = x.shape
    if z.shape != (m, Hkv, d):
        raise ValueError("logits must be [m, Hkv, d]")
    n_blocks = T // m
    p = block_weights(z)
    blocks = x[:, : n_blocks * m].reshape(B, n_blocks, m, Hkv, d)
    return (blocks * p[None, None]).sum(axis=2)


def compress_kv(k, v, zk, zv, m: int, dtype: int):
    """Compress K with zk and V with zv; return both in the storage dtype."""
    kc = compress(to_f64(k, dtype), zk, m)
    vc = compress(to_f64(v, dtype), zv, m)
    return to_storage(kc, dtype), to_storage(vc, dtype)


# --------------------------------------------------------------------------
# Visibility (reading R3; [V4-blog] "SWA": recent raw tokens beside the
# compressed history; [V4-arch] 4.4: out-of-range window positions at the
# start of the sequence contribute nothing)
# --------------------------------------------------------------------------
def window_bounds(t: int, W: int):
    """Absolute positions [lo, hi) of the window of the query at position t."""
    return max(0, t - W + 1), t + 1


def visible_count(t: int, W: int, m: int, n_entries: int) -> int:
    """Number of entries c (a prefix 0..n-1) with (c+1)*m <= t - W + 1."""
    start = t - W + 1
    if start <= 0:
        return 0
    return min(n_entries, start // m)


# --------------------------------------------------------------------------
# Step 2: lightning-indexer scores ([V4-blog] "CSA": the indexer finds the
# compressed entries most relevant to the current query; reading R1 gives the
# score formula)
# --------------------------------------------------------------------------
def indexer_scores(q_row: np.ndarray, w_row: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """s[c] = sum_h w[h] * max(0, q[h] . keys[c]) in float64, h in order."""
    s = np.zeros(keys.shape[0], dtype=np.float64)
    for h in range(q_row.shape[0]):
        dots = (keys * q_row[h][None, :]).sum(axis=1)
        s = s + w_row[h] * np.maximum(dots, 0.0)
    return s


# --------------------------------------------------------------------------
# Step 2b: per-query top-k (reading R4; [V4-blog] "CSA": Top-K compressed
# entries for the current query)
# --------------------------------------------------------------------------
def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Ascending indices of the top min(k, n) of scores, -1 padded to k.

    Order is (score descending, index ascending); -0.0 and +0.0 compare equal.
    """
    n = scores.shape[0]
    k_eff = min(k, n)
    order = np.lexsort((np.arange(n), -scores))
    out = np.full(k, -1, dtype=np.int32)
    out[:k_eff] = np.sort(order[:k_eff])
    return out


def index_topk_row(qI_row, w_row, kI_b, t: int, m: int, W: int, k: int):
    """Selection for one query row at absolute position t (float64 inputs)."""
    n_vis = visible_count(t, W, m, kI_b.shape[0])
    scores = indexer_scores(qI_row, w_row, kI_b[:n_vis])
    return select_topk(scores, k), scores


def index_topk(qI, kI, w, q_pos0: int, m: int, W: int, k: int, dtype: int,
               rows=None):
    """Top-k CSA selection for every query row.

    qI: [B, Tq, Hi, d_idx], kI: [B, N, d_idx] (storage dtype); w: [B, Tq, Hi]
    float32.  Returns int32 [B, Tq, k] (or [len(rows), k] for a list of
    (b, i) rows).
    """
    q = to_f64(qI, dtype)
    kk = to_f64(kI, dtype)
    ww = np.asarray(w, dtype=np.float32).astype(np.float64)
    B, Tq = q.shape[:2]
    if rows is None:
        out = np.empty((B, Tq, k), dtype=np.int32)
        for b in range(B):
            for i in range(Tq):
                out[b, i], _ = index_topk_row(q[b, i], ww[b, i], kk[b],
                                              q_pos0 + i, m, W, k)
        return out
    out = np.empty((len(rows), k), dtype=np.int32)
    for r, (b, i) in enumerate(rows):
        out[r], _ = index_topk_row(q[b, i], ww[b, i], kk[b], q_pos0 + i, m, W, k)
    return out


# --------------------------------------------------------------------------
# Step 3: softmax attention over one key set ([V4-code] attention: scores
# divided by sqrt(head_dim), softmax, weighted sum of values; [V4-blog] "SWA":
# compressed and raw entries enter one attention together)
# --------------------------------------------------------------------------
def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float):
    """Textbook softmax attention of one query over n keys (float64).

    Returns (output [d], weights [n]).
    """
    logits = scale * (keys * q[None, :]).sum(axis=1)
    e = np.exp(logits - logits.max())
    p = e / e.sum()
    return (p[:, None] * vals).sum(axis=0), p


def attn_row(q_row, t, *, W, raw_pos0, k_raw_b, v_raw_b, scale,
             hca=None, csa=None, idx_row=None, want=("hca", "csa", "swa")):
    """Per-branch outputs for one query row (all heads), float64.

    q_row: [H, d]; k_raw_b/v_raw_b: [Tr, Hkv, d]; hca = (k_hca_b, v_hca_b, m)
    with [N, Hkv, d] caches; csa = (k_csa_b, v_csa_b) with the row's selected
    indices idx_row (-1 padded).  Returns dict branch -> (O [H, d], weights
    list per head).
    """
    H, d = q_row.shape
    Hkv = k_raw_b.shape[1]
    G = H // Hkv
    lo, hi = window_bounds(t, W)
    r0, r1 = lo - raw_pos0, hi - raw_pos0
    if r0 < 0 or r1 > k_raw_b.shape[0]:
        raise ValueError("window rows fall outside the raw K/V rows given")
    res = {}
    for br in want:
        out = np.zeros((H, d))
        weights = []
        for h in range(H):
            g = h // G
            ks = [k_raw_b[r0:r1, g]]
            vs = [v_raw_b[r0:r1, g]]
            if br == "hca":
                k_h, v_h, m_h = hca
                n_vis = visible_count(t, W, m_h, k_h.shape[0])
                ks.append(k_h[:n_vis, g])
                vs.append(v_h[:n_vis, g])
            elif br == "csa":
                k_c, v_c = csa
                sel = idx_row[idx_row >= 0]
                ks.append(k_c[sel, g])
                vs.append(v_c[sel, g])
            o, p = attend(q_row[h], np.concatenate(ks), np.concatenate(vs), scale)
            out[h] = o
            weights.append(p)
        res[br] = (out, weights)
    return res


def gate_weights(gates, gate_mode: int, b: int, i: int) -> np.ndarray:
    """[H, 3] float64 gate weights of query row (b, i) (readings R6, R9).

    gate_mode 0: gates [H, 3], the same for every row; 1: gates [B, Tq, H, 3]
    per row; 2: per-row logits [B, Tq, H, 3], weights = softmax over the 3
    branches of each head."""
    g = np.asarray(gates, dtype=np.float32).astype(np.float64)
    if gate_mode == 0:
        return g
    if gate_mode == 1:
        return g[b, i]
    if gate_mode == 2:
        x = g[b, i]
        e = np.exp(x - x.max(axis=-1, keepdims=True))
        return e / e.sum(axis=-1, keepdims=True)
    raise ValueError(f"unknown gate_mode {gate_mode}")


def hybrid_attn_fwd(q, k_raw, v_raw, gates, *, W, dtype, q_pos0=0, raw_pos0=0,
                    hca=None, csa=None, scale=None, rows=None, branches=False, gate_mode=0):
    """Gated hybrid attention output (reading R6, [Tiny-R2] 3.1.2 mode table
    and 3.2 diagram: a per-branch gate and a weighted sum of the three
    attentions, order [HCA, CSA, SWA]).

    q: [B, Tq, H, d]; k_raw/v_raw: [B, Tr, Hkv, d]; gates: float32 [H, 3]
    (gate_mode 0) or [B, Tq, H, 3] per-row weights (1) or logits (2).
    hca = (k_hca, v_hca, m_hca) or None; csa = (k_csa, v_csa, idx) or None
    (idx int32 [B, Tq, k]).  A branch passed as None contributes nothing.
    Returns the output in the storage dtype ([B, Tq, H, d], or [len(rows), H, d]
    for a list of (b, i) rows); with branches=True also the float64 per-branch
    outputs.
    """
    qf = to_f64(q, dtype)
    kr = to_f64(k_raw, dtype)
    vr = to_f64(v_raw, dtype)
    B, Tq, H, d = qf.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    hca_f = None
    if hca is not None:
        hca_f = (to_f64(hca[0], dtype), to_f64(hca[1], dtype), int(hca[2]))
    csa_f = None
    if csa is not None:
        csa_f = (to_f64(csa[0], dtype), to_f64(csa[1], dtype), np.asarray(csa[2]))
    want = ["swa"]
    if hca_f is not None:
        want.append("hca")
    if csa_f is not None:
        want.append("csa")
    row_list = rows if rows is not None else [(b, i) for b in range(B) for i in range(Tq)]
    out = np.zeros((len(row_list), H, d))
    per_branch = {br: np.zeros((len(row_list), H, d)) for br in want}
    for r, (b, i) in enumerate(row_list):
        t = q_pos0 + i
        res = attn_row(
            qf[b, i], t, W=W, raw_pos0=raw_pos0, k_raw_b=kr[b], v_raw_b=vr[b],
            scale=scale,
            hca=None if hca_f is None else (hca_f[0][b], hca_f[1][b], hca_f[2]),
            csa=None if csa_f is None else (csa_f[0][b], csa_f[1][b]),
            idx_row=None if csa_f is None else csa_f[2][b, i],
            want=want)
        acc = np.zeros((H, d))
        g = gate_weights(gates, gate_mode, b, i)
        for col, br in ((0, "hca"), (1, "csa"), (2, "swa")):
            if br in res:
                acc = acc + g[:, col][:, None] * res[br][0]
                per_branch[br][r] = res[br][0]
        out[r] = acc
    if rows is None:
        out = out.reshape(B, Tq, H, d)
        per_branch = {k: v.reshape(B, Tq, H, d) for k, v in per_branch.items()}
    stored = to_storage(out, dtype)
    if branches:
        return stored, per_branch
    return stored


# --------------------------------------------------------------------------
# Decode cache maintenance ([V4-blog] "1. hybrid attn", the paragraph on the
# separate caches: the raw window K/V ages out as decode advances, the
# compressed entries live as long as the sequence).  Reading R8.
# --------------------------------------------------------------------------
def cache_append(pos, k_new, v_new, k_ring, v_ring, *, W: int, dtype: int, branches=(),
                 kI_new=None, kI_ring=None, kI_branch=None) -> int:
    """Append one token per sequence; update rings and caches in place.

    pos[b]: position of sequence b's new token.  k_new, v_new: [B, Hkv, d]
    and k_ring, v_ring: [B, W, Hkv, d] in the storage dtype.  branches: tuples
    (m, zk, zv, kc, vc) with logits [m, Hkv, d] and caches [B, cap, Hkv, d].
    kI_new [B, d_idx], kI_ring [B, W, d_idx] and kI_branch = (m, zI, kIc) with
    zI [m, d_idx], kIc [B, cap, d_idx] maintain the indexer keys the same way.
    Returns the number of (sequence, cache) entries not stored (capacity).
    A sequence with pos[b] < 0 (an inactive batch slot) is left untouched.
    """
    dropped = 0
    B = len(pos)
    for b in range(B):
        t = int(pos[b])
        if t < 0:
            continue
        s = t % W
        k_ring[b, s] = k_new[b]
        v_ring[b, s] = v_new[b]
        if kI_ring is not None:
            kI_ring[b, s] = kI_new[b]
        jobs = [(m, ((zk, k_ring, kc), (zv, v_ring, vc))) for (m, zk, zv, kc, vc) in branches]
        if kI_branch is not None:
            m, zI, kIc = kI_branch
            jobs.append((m, ((np.asarray(zI)[:, None, :], kI_ring[:, :, None, :], kIc[:, :, None, :]),)))
        for m, parts in jobs:
            if m > W:
                raise ValueError("block ratio larger than the ring")
            if (t + 1) % m != 0:
                continue
            c = (t + 1) // m - 1
            if c >= parts[0][2].shape[1]:
                dropped += 1
                continue
            slots = [p % W for p in range(c * m, c * m + m)]
            for z, ring, cache in parts:
                x = to_f64(ring[b, slots], dtype)[None]           # [1, m, Hkv, ch]
                cache[b, c] = to_storage(compress(x, z, m)[0, 0], dtype)
    return dropped


# --------------------------------------------------------------------------
# Rotary position embedding (reading R10: [Tiny-R2] architecture diagram and
# parameter block; [CS336] "位置编码" paragraph).
# --------------------------------------------------------------------------
def rope(x, pos, *, rope_off: int, rope_dim: int, dtype: int, base: float = 10000.0):
    """x: [rows, heads, d] in storage form; pos: [rows] int64 (negative: row
    unchanged).  Returns the rotated tensor in storage form (R10)."""
    xf = to_f64(np.asarray(x), dtype).copy()
    pos = np.asarray(pos, dtype=np.int64)
    assert xf.ndim == 3 and pos.shape == (xf.shape[0],)
    assert rope_dim > 0 and rope_dim % 2 == 0 and 0 <= rope_off and rope_off + rope_dim <= xf.shape[2]
    freq = np.array([float(base) ** (-2.0 * i / rope_dim) for i in range(rope_dim // 2)])
    for r in range(xf.shape[0]):
        p = int(pos[r])
        if p < 0:
            continue
        for i in range(rope_dim // 2):
            ang = p * freq[i]
            c, s_ = math.cos(ang), math.sin(ang)
            ca, cb = rope_off + 2 * i, rope_off + 2 * i + 1
            a = xf[r, :, ca].copy()
            b = xf[r, :, cb].copy()
            xf[r, :, ca] = a * c - b * s_
            xf[r, :, cb] = a * s_ + b * c
    return to_storage(xf, dtype)


# --------------------------------------------------------------------------
# 4-bit cache storage (reading R11: [V4-code] section "1. HCA", the storage
# of the merged cache).  The code decision is float32 arithmetic on purpose.
# --------------------------------------------------------------------------
def quant4(x, dtype: int):
    """x: any shape, storage form.  Returns (packed codes uint8 [ceil(n/2)],
    min float32, step float32)."""
    xf = to_f64(np.asarray(x), dtype).astype(np.float32).reshape(-1)
    n = xf.size
    if n == 0:
        return np.zeros(0, np.uint8), np.float32(0), np.float32(0)
    mn, mx = np.float32(xf.min()), np.float32(xf.max())
    step = np.float32((mx - mn) / np.float32(15))
    if step == 0:
        codes = np.zeros(n, np.uint8)
    else:
        t = (xf - mn) / step                       # float32, correctly rounded
        codes = np.clip(np.rint(t), 0, 15).astype(np.uint8)
    if n % 2:
        codes = np.concatenate([codes, np.zeros(1, np.uint8)])
    packed = (codes[0::2] | (codes[1::2] << np.uint8(4))).astype(np.uint8)
    return packed, mn, step


def dequant4(packed, mn, step, n: int, dtype: int):
    """Inverse of quant4: code * step + min, rounded once to the storage dtype."""
    packed = np.asarray(packed, np.uint8)
    codes = np.empty(2 * packed.size, np.uint8)
    codes[0::2] = packed & np.uint8(15)
    codes[1::2] = packed >> np.uint8(4)
    vals = codes[:n].astype(np.float64) * float(step) + float(mn)
    return to_storage(vals, dtype)


# --------------------------------------------------------------------------
# Backward pass (reading R12): the chain rule through the forward definitions
# above, one query row and one branch at a time.
# --------------------------------------------------------------------------
def compress_backward(x: np.ndarray, z: np.ndarray, m: int, dxc: np.ndarray):
    """Gradients of xc = compress(x, z, m) given dxc = dL/dxc (float64).

    xc[b, c] = sum_i P[i] x[b, c*m + i] per channel, P = softmax over i of z:
      dx[b, c*m + i] = P[i] dxc[b, c]  (rows past the last full block: 0),
      dP[i] = sum over (b, c) of dxc[b, c] x[b, c*m + i],
      dz[i] = P[i] (dP[i] - sum_l P[l] dP[l]).
    Returns (dx [B, T, Hkv, d], dz [m, Hkv, d])."""
    B, T, Hkv, d = x.shape
    n = T // m
    p = block_weights(z)
    blocks = x[:, : n * m].reshape(B, n, m, Hkv, d)
    dx = np.zeros_like(x, dtype=np.float64)
    dx[:, : n * m] = (p[None, None] * dxc[:, :, None]).reshape(B, n * m, Hkv, d)
    dp = (blocks * dxc[:, :, None]).sum(axis=(0, 1))
    dz = p * (dp - (p * dp).sum(axis=0, keepdims=True))
    return dx, dz


def attn_row_backward(q_row, t, dO, *, W, raw_pos0, k_raw_b, v_raw_b, scale, hca=None, csa=None,
                      idx_row=None, want=("hca", "csa", "swa")):
    """Backward of attn_row for one query row (all heads), float64.

    dO[br]: [H, d] gradient reaching branch br's output.  Returns the branch
    outputs O[br] ([H, d], for the gate gradient) and the gradients as a
    dict: dq [H, d]; dk_raw / dv_raw [Tr, Hkv, d]; dk_hca / dv_hca and
    dk_csa / dv_csa [N, Hkv, d] (present branches only).  Per head and branch
    with keys K, values V (the branch's key set), s = scale K q, P = softmax(s),
    O = P V:  dV_j = P_j dO;  dP_j = dO . V_j;  dS_j = P_j (dP_j - dO . O);
    dq = scale sum_j dS_j K_j;  dK_j = scale dS_j q."""
    H, d = q_row.shape
    Hkv = k_raw_b.shape[1]
    G = H // Hkv
    lo, hi = window_bounds(t, W)
    r0, r1 = lo - raw_pos0, hi - raw_pos0
    if r0 < 0 or r1 > k_raw_b.shape[0]:
        raise ValueError("window rows fall outside the raw K/V rows given")
    grads = {"dq": np.zeros((H, d)), "dk_raw": np.zeros(k_raw_b.shape), "dv_raw": np.zeros(v_raw_b.shape)}
    if hca is not None:
        grads["dk_hca"] = np.zeros(hca[0].shape)
        grads["dv_hca"] = np.zeros(hca[1].shape)
    if csa is not None:
        grads["dk_csa"] = np.zeros(csa[0].shape)
        grads["dv_csa"] = np.zeros(csa[1].shape)
    outs = {}
    for br in want:
        out = np.zeros((H, d))
        for h in range(H):
            g = h // G
            # (source, row) of every key of the branch's set, window first
            srcs = [("raw", r) for r in range(r0, r1)]
            if br == "hca":
                n_vis = visible_count(t, W, hca[2], hca[0].shape[0])
                srcs += [("hca", c) for c in range(n_vis)]
            elif br == "csa":
                srcs += [("csa", int(c)) for c in idx_row[idx_row >= 0]]
            tabs = {"raw": (k_raw_b, v_raw_b)}
            if hca is not None:
                tabs["hca"] = hca[:2]
            if csa is not None:
                tabs["csa"] = csa[:2]
            K = np.stack([tabs[sname][0][r, g] for sname, r in srcs])
            V = np.stack([tabs[sname][1][r, g] for sname, r in srcs])
            s = scale * (K * q_row[h][None, :]).sum(axis=1)
            e = np.exp(s - s.max())
            p = e / e.sum()
            o = (p[:, None] * V).sum(axis=0)
            out[h] = o
            do = dO[br][h]
            dp = (V * do[None, :]).sum(axis=1)
            ds = p * (dp - np.dot(do, o))
            grads["dq"][h] += scale * (ds[:, None] * K).sum(axis=0)
            for j, (sname, r) in enumerate(srcs):
                grads["dk_" + sname][r, g] += scale * ds[j] * q_row[h]
                grads["dv_" + sname][r, g] += p[j] * do
        outs[br] = out
    return outs, grads


def hybrid_attn_bwd(q, k_raw, v_raw, gates, dout, *, W, dtype, q_pos0=0, raw_pos0=0, hca=None, csa=None,
                    scale=None, gate_mode=0):
    """Gradients of hybrid_attn_fwd's float64 output (reading R12) given
    dout = dL/dout [B, Tq, H, d] (float64).  Inputs as for hybrid_attn_fwd.

    Returns a dict of float64 arrays: dq; dk_raw, dv_raw; dk_hca, dv_hca
    (with hca); dk_csa, dv_csa (with csa); dgates of the gates' shape (for
    gate_mode 2 the gradient reaches the logits through the branch softmax:
    dlogit = w (dw - sum w dw))."""
    qf = to_f64(q, dtype)
    kr = to_f64(k_raw, dtype)
    vr = to_f64(v_raw, dtype)
    B, Tq, H, d = qf.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    hca_f = None if hca is None else (to_f64(hca[0], dtype), to_f64(hca[1], dtype), int(hca[2]))
    csa_f = None if csa is None else (to_f64(csa[0], dtype), to_f64(csa[1], dtype), np.asarray(csa[2]))
    want = ["swa"] + (["hca"] if hca_f is not None else []) + (["csa"] if csa_f is not None else [])
    gdt = np.asarray(gates, dtype=np.float32).astype(np.float64)
    res = {"dq": np.zeros(qf.shape), "dk_raw": np.zeros(kr.shape), "dv_raw": np.zeros(vr.shape),
           "dgates": np.zeros(gdt.shape)}
    if hca_f is not None:
        res["dk_hca"] = np.zeros(hca_f[0].shape)
        res["dv_hca"] = np.zeros(hca_f[1].shape)
    if csa_f is not None:
        res["dk_csa"] = np.zeros(csa_f[0].shape)
        res["dv_csa"] = np.zeros(csa_f[1].shape)
    dout = np.asarray(dout, dtype=np.float64)
    cols = {"hca": 0, "csa": 1, "swa": 2}
    for b in range(B):
        for i in range(Tq):
            t = q_pos0 + i
            g = gate_weights(gates, gate_mode, b, i)
            dO = {br: g[:, cols[br]][:, None] * dout[b, i] for br in want}
            outs, gr = attn_row_backward(
                qf[b, i], t, dO, W=W, raw_pos0=raw_pos0, k_raw_b=kr[b], v_raw_b=vr[b], scale=scale,
                hca=None if hca_f is None else (hca_f[0][b], hca_f[1][b], hca_f[2]),
                csa=None if csa_f is None else (csa_f[0][b], csa_f[1][b]),
                idx_row=None if csa_f is None else csa_f[2][b, i], want=want)
            res["dq"][b, i] = gr["dq"]
            for name in ("dk_raw", "dv_raw", "dk_hca", "dv_hca", "dk_csa", "dv_csa"):
                if name in gr:
                    res[name][b] += gr[name]
            # gate weights: dL/dw[h, col] = dout . O_col (absent branches: 0)
            dw = np.zeros((H, 3))
            for br in want:
                dw[:, cols[br]] = (dout[b, i] * outs[br]).sum(axis=1)
            if gate_mode == 0:
                res["dgates"] += dw
            elif gate_mode == 1:
                res["dgates"][b, i] = dw
            else:
                res["dgates"][b, i] = g * (dw - (g * dw).sum(axis=1, keepdims=True))
    return res


def hybrid_path_bwd(q, k, v, gates, dout, *, W, dtype, idx=None, hca=None, csa=None, scale=None, gate_mode=0):
    """Backward of the whole prefill path (reading R12): block compression of
    K and V for each present branch (hca = (zk, zv, m), csa = (zk, zv, m);
    caches stored in the storage dtype as in the forward), gated attention
    with the CSA selection idx given, then the compression backward.

    Returns float64 gradients: dq; dk, dv (raw rows: window part plus every
    branch's compression part); dzk_hca, dzv_hca, dzk_csa, dzv_csa (present
    branches); dgates; and the cache gradients dk_hca ... dv_csa."""
    kf, vf = to_f64(k, dtype), to_f64(v, dtype)
    hca_c = csa_c = None
    if hca is not None:
        kh, vh = compress_kv(k, v, hca[0], hca[1], hca[2], dtype)
        hca_c = (kh, vh, hca[2])
    if csa is not None:
        kc, vc = compress_kv(k, v, csa[0], csa[1], csa[2], dtype)
        csa_c = (kc, vc, idx)
    res = hybrid_attn_bwd(q, k, v, gates, dout, W=W, dtype=dtype, hca=hca_c, csa=csa_c, scale=scale,
                          gate_mode=gate_mode)
    res["dk"] = res["dk_raw"].copy()
    res["dv"] = res["dv_raw"].copy()
    for name, br in (("hca", hca), ("csa", csa)):
        if br is None:
            continue
        zk, zv, m = br
        dxk, dzk = compress_backward(kf, np.asarray(zk, np.float64), m, res["dk_" + name])
        dxv, dzv = compress_backward(vf, np.asarray(zv, np.float64), m, res["dv_" + name])
        res["dk"] += dxk
        res["dv"] += dxv
        res["dzk_" + name] = dzk
        res["dzv_" + name] = dzv
    return res
