/*
 * hybrid_attn.h -- C interface of the MI355X (gfx950) hybrid sparse attention
 * forward pass: HCA (heavily compressed), CSA (compressed + sparse-selected) and
 * SWA (sliding window) branches mixed by gates (per head or per token), the
 * decode-time maintenance of the raw window ring and the compressed caches,
 * the rotary position embedding applied to Q and K before the path, and the
 * 4-bit storage of a compressed cache.
 *
 * Pages this interface follows (cited by title and section):
 *   [V4-blog] "deepseek-v4" (astro-blog post), section "1. hybrid attn":
 *             CSA = 4:1 compression + lightning indexer top-K + sparse attention;
 *             HCA = ratio 128, dense attention over the compressed entries;
 *             SWA = the most recent 128 raw tokens, attended together with the
 *             compressed history in one attention; the caches are kept apart.
 *   [V4-code] CSDN article with CSA/HCA example code, section "1. HCA":
 *             block merge = softmax over block positions of a learned
 *             [block_size, channels] parameter, weighted sum over the block;
 *             attention scale 1/sqrt(head_dim).
 *   [Tiny-R2] Tiny-R2 README, sections 3.1.2 (modes HCA [1,0,0], CSA [0,1,0],
 *             SWA [0,0,1]) and 3.2 (branch gate + weighted sum, config fields
 *             block_size / window_size / num_tokens_to_keep).
 *   [CS336]   CS336 notes, "Attention Heads 变体" (MQA / GQA head sharing),
 *             "位置编码" paragraph (RoPE: position as a rotation angle).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer allocated and owned by the caller.
 *    The library never allocates or frees device memory and keeps no state
 *    between calls (apart from the thread-local error string and the device
 *    array of hybrid_sparse_attn_fwd_noalloc).
 *  - dtype: SHATTN_DTYPE_BF16 (bfloat16) or SHATTN_DTYPE_F32 applies to every
 *    tensor operand except logits, indexer weights and gates, which are always
 *    float32.  Accumulation is float32; stored results are rounded once to
 *    nearest even.
 *  - Layouts are dense row-major with the shapes given below; pointers must be
 *    16-byte aligned.
 *  - Positions: query row i has absolute position q_pos0 + i.  A compressed
 *    entry c of ratio m covers raw positions [c*m, (c+1)*m).  The window of the
 *    query at t is positions max(0, t-W+1) .. t.  A compressed entry is visible
 *    to t only when it lies wholly before that window: (c+1)*m <= t-W+1.
 *  - stream is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *    work; they never synchronise the device.  Calls are reentrant.
 *  - Return value: SHATTN_OK (0) or a negative error code.  Every argument is
 *    validated on the host before any HIP call, so an invalid call enqueues
 *    nothing.  shattn_last_error() returns a message for the calling thread's
 *    last failure.
 *  - Identical inputs give bitwise identical outputs (no floating-point
 *    atomics in any reduction).
 */
#ifndef HYBRID_ATTN_H
#define HYBRID_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define SHATTN_API __attribute__((visibility("default")))
#else
#define SHATTN_API
#endif

#define SHATTN_DTYPE_BF16 0
#define SHATTN_DTYPE_F32 1

#define SHATTN_OK 0
#define SHATTN_EINVAL (-1)       /* invalid argument (null pointer, bad shape) */
#define SHATTN_EUNSUPPORTED (-2) /* valid but outside what the kernels support */
#define SHATTN_EWORKSPACE (-3)   /* workspace missing or too small */
#define SHATTN_EHIP (-4)         /* a HIP launch failed; message has the reason */

/*
 * Block compression of K and V ([V4-code] section 1, block merge; [V4-blog]
 * "CSA" 4:1 diagram; m = 4 for CSA and m = 128 for HCA).
 *
 *   P[i,g,ch]      = softmax over i < m of z[i,g,ch]         (float32)
 *   kc[b,c,g,ch]   = sum_{i<m} Pk[i,g,ch] * k[b, c*m+i, g, ch]
 *   vc[b,c,g,ch]   = sum_{i<m} Pv[i,g,ch] * v[b, c*m+i, g, ch]
 *
 *   k, v   : [B, T, Hkv, d]          dtype
 *   zk, zv : [m, Hkv, d]             float32 logits (may be the same pointer)
 *   kc, vc : [B, floor(T/m), Hkv, d] dtype, written; a trailing partial block
 *            of T % m rows is not compressed.
 * Supported: d in {64, 128}; 1 <= m <= 1024; Hkv >= 1; B, T >= 0.
 */
SHATTN_API int hca_compress_kv(const void* k, const void* v, const float* zk, const float* zv,
                    void* kc, void* vc, int B, int T, int Hkv, int d, int m, int dtype,
                    void* stream);

/*
 * The same block compression for two ratios in one pass over K and V (each raw
 * row is read once): ratio m1 into kc1/vc1 ([B, floor(T/m1), Hkv, d], logits
 * zk1/zv1 [m1, Hkv, d]) and ratio m2 into kc2/vc2 ([B, floor(T/m2), Hkv, d],
 * logits zk2/zv2 [m2, Hkv, d]).  Results equal two hca_compress_kv calls.
 * Supported: m1 in {1, 2, 4, 8}; m2 a multiple of 8, at most 1024; d in {64, 128}.
 * Rows past the last full m2-block are compressed for ratio m1 only, with
 * extra launches (one per sequence).
 */
SHATTN_API int hca_compress_kv_dual(const void* k, const void* v, const float* zk1, const float* zv1,
                                    void* kc1, void* vc1, int m1, const float* zk2, const float* zv2,
                                    void* kc2, void* vc2, int m2, int B, int T, int Hkv, int d, int dtype,
                                    void* stream);

/*
 * Lightning indexer + per-query top-k over the CSA entries ([V4-blog] "CSA":
 * the indexer finds, for the current query, the Top-K most relevant
 * compressed entries; [Tiny-R2] 3.2 importance_score / topk selection).
 *
 *   score[b,i,c] = sum_{h<Hi} w[b,i,h] * max(0, qI[b,i,h,:] . kI[b,c,:])
 *
 * for the entries c visible to query row i (position q_pos0 + i; visibility
 * uses ratio m and window W as above).  idx[b,i,:] receives the
 * k_eff = min(k, #visible) visible entries ranked first by (score descending,
 * entry index ascending), written in ascending entry index and padded with -1.
 * The ranking is decided on exact scores: a float32 MFMA pass screens the
 * candidates and every candidate within the float32 error bound of the k-th
 * score is re-scored in float64, so the selected set equals the one a float64
 * evaluation of the formula selects.
 *
 *   qI  : [B, Tq, Hi, d_idx] dtype      kI : [B, N, d_idx] dtype
 *   w   : [B, Tq, Hi]        float32    idx: [B, Tq, k] int32, written
 *   ws  : device workspace of at least csa_index_topk_workspace_size() bytes,
 *         256-byte aligned (may be NULL when that size is 0); its contents are
 *         scratch.  Sizes: 0 for N <= 2048 with Hi < 16 and for N = 0; for
 *         longer prefill (and Hi = 16) about 8 * B * Tq * L bytes, L =
 *         per-query candidate list length (a few times k); for decode shapes
 *         (B * Tq <= 64, N >= 8192) about 4 * B * Tq * N bytes.
 * Long prefill (N > 2048, or any N > 0 with Hi = 16) is decided per query
 * from a list of the entries whose float32 score reaches a threshold
 * estimated from every S-th entry; queries whose list cannot decide are
 * recomputed by streaming all entries, so the result never depends on the
 * estimate.
 * Supported: Hi in {1, 2, 4, 8, 16}; d_idx in {64, 128}; 1 <= k <= 2048;
 *            m >= 1; W >= 1; N >= 0.
 */
SHATTN_API size_t csa_index_topk_workspace_size(int B, int Tq, int N, int Hi, int d_idx, int k);
SHATTN_API int csa_index_topk(const void* qI, const void* kI, const float* w, int32_t* idx, int B,
                   int Tq, int N, int Hi, int d_idx, int64_t q_pos0, int m, int W, int k,
                   int dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * csa_index_topk with one position per sequence (decode of sequences at
 * different positions, [V4-blog] "1. hybrid attn": the compressed caches live
 * with each sequence): query row i of sequence b has position q_pos[b] + i.
 * q_pos is a DEVICE int64 array [B], 8-byte aligned; a negative q_pos[b]
 * marks an inactive sequence (its rows are written all -1).  N may be the
 * capacity of the kI cache: an entry is read only when it is visible at the
 * row's position, so entries not yet written are never read.  Everything
 * else (shapes, workspace, errors, the exact selection) as csa_index_topk.
 */
SHATTN_API int csa_index_topk_varlen(const void* qI, const void* kI, const float* w, int32_t* idx, int B,
                                     int Tq, int N, int Hi, int d_idx, const int64_t* q_pos, int m, int W,
                                     int k, int dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * Gated hybrid attention forward ([V4-blog] "SWA": the raw window and the
 * compressed history enter one attention; [Tiny-R2] 3.1.2 / 3.2: three
 * branches mixed by a per-head gate, order [HCA, CSA, SWA]).
 *
 * For query row i (position t) and head h (KV head g = h / (H/Hkv)), with
 * logits sm_scale * q.k and one softmax per key set:
 *   O_SWA = attention over the window rows of k_raw / v_raw
 *   O_HCA = attention over the window rows + every visible HCA entry
 *   O_CSA = attention over the window rows + the entries idx[b,i,:] (those
 *           with 0 <= idx < N_csa; -1 marks padding)
 *   out   = g[0]*O_HCA + g[1]*O_CSA + g[2]*O_SWA, with the gate weights g of
 *           (row, head) by gate_mode: 0 = gates[h, :] ([H, 3], per head);
 *           1 = gates[b, i, h, :] ([B, Tq, H, 3], per token); 2 = softmax over
 *           the three branches of the logits gates[b, i, h, :] ([B, Tq, H, 3];
 *           the branch gate's Linear + Softmax of [Tiny-R2] 3.2, softmax fused)
 * The HCA branch is present iff m_hca > 0 and the CSA branch iff k > 0; an
 * absent branch contributes nothing (its gate column is ignored).  A present
 * branch with no entries (N = 0, pointers may then be NULL) still contributes
 * its window-only attention.  idx rows list distinct entries.
 * Raw K/V row r holds absolute position raw_pos0 + r; every window row the
 * queries need must lie in [raw_pos0, raw_pos0 + Tr).  Decode with sequences
 * at different positions ([V4-blog] "1. hybrid attn": the raw window and the
 * compressed caches are kept apart, the raw rows age out): q_pos gives each
 * sequence's position and raw_ring = 1 reads the window from the rings
 * hybrid_cache_append maintains; the compressed caches hold the entries
 * visible at each sequence's own position (N_hca / N_csa may be their
 * capacity: entries a position cannot see are never read).
 */
typedef struct shattn_fwd_args {
    int32_t struct_size; /* must equal sizeof(shattn_fwd_args) */
    int32_t dtype;
    int32_t B, Tq, H, Hkv, d, W;
    float sm_scale;      /* 0 -> 1/sqrt(d) */
    int32_t gate_mode;   /* 0, 1 or 2: how gates is read (see above) */
    int64_t q_pos0;
    const void* q;       /* [B, Tq, H, d] */
    void* out;           /* [B, Tq, H, d], written */
    int64_t raw_pos0;
    int32_t Tr;
    int32_t m_hca;       /* HCA ratio; 0 = HCA branch absent */
    const void* k_raw;   /* [B, Tr, Hkv, d] */
    const void* v_raw;   /* [B, Tr, Hkv, d] */
    int32_t N_hca;
    int32_t N_csa;
    const void* k_hca;   /* [B, N_hca, Hkv, d] */
    const void* v_hca;
    int32_t m_csa;       /* informational; selection already encodes visibility */
    int32_t k;           /* entries per row in idx; 0 = CSA branch absent */
    const void* k_csa;   /* [B, N_csa, Hkv, d] */
    const void* v_csa;
    const int32_t* idx;  /* [B, Tq, k] */
    const float* gates;  /* float32: [H, 3] (gate_mode 0) or [B, Tq, H, 3] (1, 2) */
    const int64_t* q_pos; /* NULL, or DEVICE int64 [B]: position of query row 0 of
                             each sequence (q_pos0 is then unused); a negative
                             entry marks an inactive sequence whose output rows
                             are left untouched.  Needs raw_ring = 1. */
    int32_t raw_ring;    /* 0: raw row r holds position raw_pos0 + r.
                            1: k_raw / v_raw are rings of Tr rows per sequence
                            (as hybrid_cache_append keeps them): position t is
                            in row t % Tr; raw_pos0 is unused and Tr >= W + Tq - 1. */
    int32_t reserved0;   /* must be 0 */
    int32_t cache_q4;    /* bit 0: k_hca / v_hca hold 4-bit codes, bit 1: k_csa /
                            v_csa do ([V4-code] section 1, 4-bit storage of the
                            merged cache): codes as cache_quant4 writes them
                            ([B, N, Hkv, d/2] bytes, element 2j in the low nibble
                            of byte j of a row), decoded inside the attention's
                            loads to the values cache_dequant4 gives.  bf16 only. */
    int32_t reserved1;   /* must be 0 */
    const float* q4_k_hca; /* DEVICE float32 [2] (min, step) of each coded tensor, */
    const float* q4_v_hca; /*   as cache_quant4 writes them (bits of cache_q4 set) */
    const float* q4_k_csa;
    const float* q4_v_csa;
    int32_t rope_q;      /* 1: rotate the query's channels [rope_off, rope_off +
                            rope_dim) by RoPE at each query row's position as
                            the attention loads it: the values rope_apply would
                            store, so q need not be rotated beforehand.
                            rope_off and rope_dim even, base finite and > 0. */
    int32_t rope_off;
    int32_t rope_dim;
    int32_t reserved2;   /* must be 0 */
    double rope_base;
    int32_t split_part;  /* 0: the whole attention.  A launch that splits the
                            key list (hybrid_sparse_attn_fwd_workspace_size() >
                            0: decode) can run as two calls on one workspace:
                            1 = the window and HCA items, which do not read
                            idx (so they may run while the indexer writes it,
                            on another stream); 2 = the CSA items and the merge
                            of every item's partial state, ordered after call
                            1 by the caller.  Without a split, call 1 does
                            nothing and call 2 the whole attention. */
    int32_t reserved3;   /* must be 0 */
} shattn_fwd_args;

/* Workspace bytes hybrid_sparse_attn_fwd needs for these arguments (0 when the
 * launch needs none). */
SHATTN_API size_t hybrid_sparse_attn_fwd_workspace_size(const shattn_fwd_args* a);
/* Supported: d in {64, 128}; H % Hkv == 0 with H/Hkv <= 64; W >= 1;
 *            k <= 4096. */
SHATTN_API int hybrid_sparse_attn_fwd(const shattn_fwd_args* a, void* ws, size_t ws_bytes, void* stream);

/*
 * hybrid_sparse_attn_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace taken from a
 * device array inside the library (32 MiB per GPU, held by each GPU the
 * library runs on until the process ends).  This call itself allocates
 * nothing.  The array is located on the calling thread's current device,
 * which must be the device the tensors and the stream belong to.  Arguments
 * whose hybrid_sparse_attn_fwd_workspace_size() exceeds 32 MiB return
 * SHATTN_EUNSUPPORTED.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (concurrent streams, threads) race and must be
 * serialised by the caller.
 */
SHATTN_API int hybrid_sparse_attn_fwd_noalloc(const shattn_fwd_args* a, void* stream);

/*
 * Backward pass of a prefill through the whole path: block compression of K
 * and V for each present branch, gated hybrid attention, as
 * hybrid_sparse_attn_fwd defines it with q_pos0 = raw_pos0 = 0 and Tq = Tr = T
 * ([V4-code] section 1 block merge; [V4-blog] "1. hybrid attn"; [Tiny-R2]
 * 3.1.2 / 3.2 branch gate).  Gradients are those of the forward's value with
 * the CSA selection idx held fixed (a top-k has none) and the storage
 * rounding of the compressed caches taken as the identity:
 *   per branch b with gate weight w_b, P_bj the branch softmax and
 *   D_b = dout . O_b:  dS_j = sum_b w_b P_bj (dout . v_j - D_b);
 *   dq = scale sum_j dS_j k_j;  dk_j = scale sum dS_j q;  dv_j = sum w_b P_bj dout;
 *   window keys belong to every present branch, HCA entries to HCA, selected
 *   CSA entries to CSA; cache gradients flow to the raw rows (P_i dkc) and to
 *   the logits (dz_i = P_i (dP_i - sum_l P_l dP_l), dP_i = sum dkc . x_i);
 *   gates: dw_b = D_b (per head: summed over rows; logits: through the
 *   branch softmax).
 * All gradients are float32 and overwrite their buffers.  Arithmetic is
 * float32 with no floating-point atomics (bitwise-reproducible).
 */
typedef struct shattn_bwd_args {
    int32_t struct_size; /* must equal sizeof(shattn_bwd_args) */
    int32_t dtype;       /* of q, k_raw, v_raw, dout and the caches */
    int32_t B, T, H, Hkv, d, W;
    float sm_scale;      /* 0 -> 1/sqrt(d) */
    int32_t gate_mode;   /* 0, 1 or 2 as in hybrid_sparse_attn_fwd */
    int32_t m_hca;       /* HCA ratio; 0 = HCA branch absent */
    int32_t m_csa;       /* CSA ratio (>= 1 when k > 0) */
    int32_t k;           /* entries per row in idx; 0 = CSA branch absent */
    int32_t reserved0;   /* must be 0 */
    const void* q;       /* [B, T, H, d] */
    const void* k_raw;   /* [B, T, Hkv, d], positions 0 .. T-1 */
    const void* v_raw;
    const void* dout;    /* [B, T, H, d]: dL/dout */
    const float* gates;  /* as in hybrid_sparse_attn_fwd */
    const float* zk_hca; /* [m_hca, Hkv, d] compression logits of the HCA caches */
    const float* zv_hca;
    const void* k_hca;   /* [B, T / m_hca, Hkv, d]: hca_compress_kv(k_raw, v_raw, zk_hca, zv_hca) */
    const void* v_hca;
    const float* zk_csa; /* [m_csa, Hkv, d] */
    const float* zv_csa;
    const void* k_csa;   /* [B, T / m_csa, Hkv, d] */
    const void* v_csa;
    const int32_t* idx;  /* [B, T, k]: the forward's selection; -1 = padding.
                            Entries must be distinct; entries not visible to
                            their row are ignored (csa_index_topk writes none). */
    float* dq;           /* [B, T, H, d] */
    float* dk;           /* [B, T, Hkv, d]: window part plus every compression's part */
    float* dv;
    float* dzk_hca;      /* [m_hca, Hkv, d] (HCA present) */
    float* dzv_hca;
    float* dzk_csa;      /* [m_csa, Hkv, d] (CSA present) */
    float* dzv_csa;
    float* dgates;       /* gates' shape: [H, 3] (mode 0) or [B, T, H, 3] */
    float* dk_hca;       /* optional (NULL = not returned): [B, T / m_hca, Hkv, d] */
    float* dv_hca;       /*   gradients of the compressed caches */
    float* dk_csa;       /* optional: [B, T / m_csa, Hkv, d] */
    float* dv_csa;
} shattn_bwd_args;

/* Workspace bytes hybrid_sparse_attn_bwd needs (0 for invalid arguments):
 * 24 B per (row, head) for the softmax statistics, the cache gradients not
 * returned, and the compression-logit partial sums. */
SHATTN_API size_t hybrid_sparse_attn_bwd_workspace_size(const shattn_bwd_args* a);
/* Supported: d in {64, 128}; H % Hkv == 0; W >= 1; ratios <= 1024;
 * B T H < 2^31.  Workspace 16-byte aligned, at least the size above
 * (SHATTN_EWORKSPACE otherwise). */
SHATTN_API int hybrid_sparse_attn_bwd(const shattn_bwd_args* a, void* ws, size_t ws_bytes, void* stream);

/*
 * Decode cache maintenance, one new token per sequence ([V4-blog] "1. hybrid
 * attn": the raw window K/V and the compressed caches are kept apart; the raw
 * rows age out as decode advances, the compressed entries stay; the block
 * merge of [V4-code] section 1 as in hca_compress_kv).
 *
 * For each sequence b whose new token has absolute position t = pos[b] >= 0:
 *   - ring row t % W of k_ring / v_ring (and kI_ring) takes k_new[b] /
 *     v_new[b] (and kI_new[b]);
 *   - for each present ratio m (m_csa, m_hca) with (t + 1) % m == 0, entry
 *     c = (t + 1) / m - 1 of that ratio's K and V caches becomes the block
 *     compression of positions [c*m, (c+1)*m) with that ratio's logits: the
 *     first m - 1 rows from the ring (written by earlier calls), the last from
 *     k_new / v_new.  With d_idx > 0 the CSA entry's indexer key is the same
 *     compression of the per-token indexer keys with logits zI.
 *   - An entry with c >= its cache's capacity is not written; for each such
 *     (sequence, cache) -- the K/V pair of a ratio counts once, the
 *     indexer-key cache once -- *dropped grows by 1 (when dropped != NULL).
 * A sequence with pos[b] < 0 is left untouched (inactive batch slot).  The
 * caller advances pos between calls; calls for one sequence must be issued
 * in position order on one stream (each reads ring rows the earlier ones
 * wrote).  Rows of the ring older than t - W + 1 are overwritten.
 *
 *   pos            : [B] int64, DEVICE memory, 8-byte aligned
 *   k_new, v_new   : [B, Hkv, d]           dtype
 *   k_ring, v_ring : [B, W, Hkv, d]        dtype, row t % W written
 *   zk_*, zv_*     : [m, Hkv, d]           float32 logits of each ratio
 *   k_csa, v_csa   : [B, cap_csa, Hkv, d]  dtype;  k_hca, v_hca: [B, cap_hca, Hkv, d]
 *   kI_new         : [B, d_idx]; kI_ring: [B, W, d_idx]; kI_csa: [B, cap_csa, d_idx]
 *   zI             : [m_csa, d_idx]        float32
 *   dropped        : int32 counter in DEVICE memory (incremented atomically), or NULL
 * Supported: d in {64, 128}; d_idx in {0, 64, 128} (d_idx > 0 needs m_csa > 0);
 *            0 <= m_csa, m_hca <= min(W, 1024) (0 = no cache of that ratio);
 *            B <= 65535.
 */
typedef struct shattn_append_args {
    int32_t struct_size;   /* must equal sizeof(shattn_append_args) */
    int32_t dtype;
    int32_t B, Hkv, d, W;
    int32_t m_csa, m_hca, d_idx;
    int32_t reserved0;     /* must be 0 */
    const int64_t* pos;
    const void* k_new;
    const void* v_new;
    void* k_ring;
    void* v_ring;
    const float* zk_csa;
    const float* zv_csa;
    void* k_csa;
    void* v_csa;
    int64_t cap_csa;
    const float* zk_hca;
    const float* zv_hca;
    void* k_hca;
    void* v_hca;
    int64_t cap_hca;
    const void* kI_new;
    void* kI_ring;
    const float* zI;
    void* kI_csa;
    int32_t* dropped;
} shattn_append_args;

SHATTN_API int hybrid_cache_append(const shattn_append_args* a, void* stream);

/*
 * Rotary position embedding, in place, on a range of channels of every head
 * (the prologue step before the attention: applied to Q, to the raw window
 * K rows and to the compressed K entries).
 *
 * Pages: [Tiny-R2] architecture diagram (RoPE on the prepared query, the
 * window keys, the selected CSA keys and the HCA keys) and parameter block
 * (a rope part of the head dim beside a non-rope part); [CS336] "位置编码"
 * paragraph (position as a rotation angle, so that a query-key product
 * depends on the position difference).  The pages fix neither the pairing
 * nor the base; the reading taken: channels rope_off + 2i and
 * rope_off + 2i + 1 (0 <= i < rope_dim / 2) of each head turn by the angle
 * pos * base^(-2i / rope_dim), (a, b) -> (a cos - b sin, a sin + b cos);
 * the other channels are unchanged.  Arithmetic: the angle is formed in
 * turns (pos * f_i / 2 pi) in float64 and its whole turns dropped there; the
 * sine and cosine of the remaining fraction (the hardware's float32 sine and
 * cosine, which take turns) and the rotation are float32; the result is
 * rounded once to the storage dtype.
 *
 *   x    : [rows, heads, d]  dtype, DEVICE memory, rotated in place
 *   pos  : [rows] int64, DEVICE memory, 8-byte aligned: the position of each
 *          row (for a compressed entry, the position the model assigns it);
 *          a row with pos < 0 is left unchanged
 *   base : finite, > 0 (10000 is the usual choice)
 * Errors (SHATTN_EINVAL): unknown dtype, rows < 0, heads < 1, d < 2, an odd
 * or empty rope_dim, a channel range outside [0, d), a bad base, null or
 * misaligned pointers with rows > 0.  rows == 0 is a no-op.
 */
SHATTN_API int rope_apply(void* x, const int64_t* pos, int64_t rows, int32_t heads, int32_t d,
                          int32_t rope_off, int32_t rope_dim, double base, int32_t dtype, void* stream);

/*
 * 4-bit storage of a compressed cache (K or V of CSA / HCA, any shape): one
 * minimum and one step over the whole tensor, two codes per byte.
 *
 * Page: [V4-code] section "1. HCA" (the merged cache is stored in 4 bits:
 * minimum and maximum over the tensor, step = (max - min) / 15, codes rounded
 * and clamped to 0..15, decoded as code * step + min; packing two codes per
 * byte is named there as the real layout).  Reading: the code of element i is
 * rint((x[i] - min) / step) clamped to [0, 15], computed in float32 with
 * round-half-even; step == 0 (a constant tensor) gives code 0 everywhere.
 *
 * cache_quant4:
 *   x      : [n] dtype, DEVICE memory (finite values)
 *   codes  : [ceil(n / 2)] uint8, DEVICE memory, written: element 2j in the low
 *            nibble of byte j, element 2j + 1 in the high nibble (0 past n)
 *   params : [2] float32, DEVICE memory, 4-byte aligned, written: (min, step);
 *            it doubles as the scratch of the min / max reduction, and the
 *            first four bytes of codes (when codes is 4-byte aligned and holds
 *            at least four bytes) hold a workgroup counter until the codes are
 *            written, so a second call must not use the same params or codes
 *            while one is in flight
 * cache_dequant4:
 *   out[i] = code_i * step + min, the product exact and the sum rounded to
 *   float64, then rounded once (nearest even) to dtype; codes / params as
 *   written by cache_quant4 (or any (min, step) pair the caller stores).
 * Errors (SHATTN_EINVAL): unknown dtype, n < 0, null or misaligned pointers
 * with n > 0.  n == 0 is a no-op (params untouched).
 */
SHATTN_API int cache_quant4(const void* x, int64_t n, int32_t dtype, uint8_t* codes, float* params,
                            void* stream);
SHATTN_API int cache_dequant4(const uint8_t* codes, const float* params, int64_t n, int32_t dtype, void* out,
                              void* stream);

/* Message describing the calling thread's last failure ("" if none). */
SHATTN_API const char* shattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HYBRID_ATTN_H */
