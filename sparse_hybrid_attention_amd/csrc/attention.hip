// Gated hybrid (HCA / CSA / SWA) attention forward on gfx950.
//
// Method ([V4-blog] "SWA": the recent raw window and the compressed history
// enter one attention; [V4-blog] "HCA" / "CSA": all compressed entries vs the
// top-k selected ones; [Tiny-R2] 3.1.2 / 3.2: three branches mixed by a
// per-head gate; [V4-code] attention scale 1/sqrt(head_dim); [CS336] GQA/MQA
// head sharing; FlashAttention-style online softmax).
//
// Design:
//  * One workgroup = (sequence b, KV head g, a tile of QW query rows) with the
//    G = H/Hkv query heads of that KV head: 64 "columns" (query, head), 16 per
//    wave.  All columns of a workgroup share the window and HCA keys, so those
//    K/V tiles are staged once in LDS and read by every wave.
//  * Transposed MFMA formulation: S^T = K Q^T (rows = 32 keys per tile,
//    columns = the wave's 16 (query, head) pairs) and O^T = V^T P^T.  The key
//    rows of the two 16-row S^T tiles are interleaved so that the C layout of
//    S^T is already the B-operand layout of P^T: no LDS round trip for P.
//  * bf16 K/V tiles arrive by direct global->LDS loads into XOR-swizzled rows
//    (no register staging); V^T operands come from transposing LDS reads.
//    Tiles are double-buffered and the pipeline runs on across the branches
//    of a workgroup (the last tile of one key source overlaps the first tile
//    of the next).  32-key tiles keep LDS at 32 KB and VGPRs at ~160 per
//    wave, so three workgroups share a CU.
//  * One running online-softmax state per column (log2 domain, the scale
//    folded into the exponent's FMA) and one gated output accumulator.  The
//    HCA entries are attended alone first (their raw state parks in the
//    output accumulator), then the window once: O_SWA is the window state and
//    O_HCA the merge of the window and HCA states, which needs only their
//    maxima and sums.  The CSA entries then continue the window's state
//    (O_CSA).  Every key is attended once per branch that contains it and the
//    window is never recomputed.  out = g0 O_HCA + g1 O_CSA + g2 O_SWA is
//    rounded once.
//  * CSA keys: when the selections of a tile's queries cover most visible
//    entries (small N, G < 8) the CSA entries are attended densely with a
//    per-(query, entry) selection bitmap in LDS ("dense-masked"); otherwise
//    each wave gathers the selected rows of its queries into its own LDS
//    tile ("gather").  Both give the same mathematical result.
//  * A branch whose gate is 0 for every head of the workgroup is skipped.
//  * Long key lists with few workgroups (decode) are split along the key
//    list; each split writes (m, l, acc) partial states to the workspace and a
//    combine kernel merges them in split order (deterministic).
//  * Workgroups are remapped so that each XCD (own L2) runs a contiguous
//    range of (sequence, head, query tile) work.
//  * 4-bit compressed caches ([V4-code] section 1, 4-bit storage of the
//    merged cache): a kernel variant (Q4) loads the codes of HCA / CSA rows
//    into registers and decodes them through 256-entry byte tables in LDS
//    (each entry the two bf16 values of a code byte, code * step + min
//    rounded once) into the same swizzled bf16 tiles; everything after the
//    loads is unchanged.
#include <algorithm>
#include <cmath>
#include <mutex>

#include <type_traits>

#include "common.h"

namespace shattn {

long long n_visible_host(long long t, int W, int m, int N) {
    const long long s = t - W + 1;
    if (s <= 0) return 0;
    const long long n = s / m;
    return n < N ? n : N;
}

namespace {

constexpr int KT = 32;  // keys per shared LDS tile (one MFMA chunk; small tiles keep 3 workgroups per CU)
constexpr int KC = 32;  // keys per MFMA chunk

enum CsaMode { CSA_NONE = 0, CSA_DENSE = 1, CSA_GATHER = 2 };

struct AttnParams {
    const void* q;
    void* out;
    const void* k_raw;
    const void* v_raw;
    const void* k_hca;
    const void* v_hca;
    const void* k_csa;
    const void* v_csa;
    const int32_t* idx;
    const float* gates;
    int gate_mode;     // 0: [H, 3]; 1: [B, Tq, H, 3] weights; 2: [B, Tq, H, 3] logits
    float* ws;  // split partial states (split mode only)
    long long q_pos0, raw_pos0;
    const int64_t* q_pos;  // per-sequence position of query row 0 (device [B]) or null: q_pos0 for all
    int ring;              // raw K/V: 0 = row r holds position raw_pos0 + r; 1 = ring, position t in row t % Tr
    int B, Tq, H, Hkv, G, W, Tr;
    int m_hca, N_hca, N_csa, k;
    float scale_log2;
    int QW;        // query rows per workgroup
    int nqt;       // query tiles per (b, g)
    int csa_mode;
    int bm_words;  // bitmap words per query (dense mode)
    int lds_bm;    // byte offsets in dynamic LDS
    int lds_gather;
    int lds_gather_stride;
    // split mode (0 = off): work item list over [window | HCA | CSA] keys
    int nsplit;
    int split_keys;
    int split_csa;   // selected CSA entries per split item (gathers are slower per key)
    int n_win_items, n_hca_items;
    int item_lo, item_n;   // the items [item_lo, item_lo + item_n) of every (b, g, query tile) this launch runs
    int has_hca, has_csa;  // branch present (its gate column is used)
    int ncol;              // columns (query, head) per workgroup = 16 * waves
    // 4-bit compressed caches: bit 0 HCA, bit 1 CSA hold codes (two per byte)
    int q4;
    const float* q4p[4];   // (min, step) of the k_hca, v_hca, k_csa, v_csa codes
    int lds_lut;           // byte offset of the four 256-entry decode tables
    // RoPE of the query at load (rope_q): channels [rope_off, rope_off + rope_dim)
    int rope_q, rope_off, rope_dim;
    double rope_step;      // 2 log2(base) / rope_dim
};

// ---------------------------------------------------------------- per-dtype MFMA
template <typename T, int D> struct Tr;

template <int D> struct Tr<bf16_t, D> {
    static constexpr int KS = D / 32;     // S^T k-steps
    static constexpr int DT = D / 16;     // O^T dim tiles
    static constexpr int KPAD = D + 8;    // K tile row stride (elements)
    static constexpr int VST = KT + 8;    // shared V^T row stride (elements)
    static constexpr int GVST = KC + 8;   // gather V^T row stride
    static constexpr int VEC = 8;
    typedef bf16x8_t QF;

    __device__ static void load_q(const bf16_t* qrow, int q4, bool ok, QF* qf) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ok) {
                qf[ks] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * ks + 8 * q4);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) qf[ks][j] = (__bf16)0.0f;
            }
        }
    }
    // RoPE of the loaded query (position pos): the lane holds dims 32 ks + 8 q4
    // .. +7 of the row, whole channel pairs when rope_off is even
    __device__ static void rope_q(const AttnParams& p, const bf16_t*, long long pos, int q4, QF* qf) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int ch = 32 * ks + 8 * q4 + 2 * jj;
                if (ch < p.rope_off || ch >= p.rope_off + p.rope_dim) continue;
                float s, c, r0, r1;
                rope_sincos(pos, (ch - p.rope_off) >> 1, p.rope_step, &s, &c);
                rope_turn((float)qf[ks][2 * jj], (float)qf[ks][2 * jj + 1], s, c, &r0, &r1);
                qf[ks][2 * jj] = __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_rne(r0));
                qf[ks][2 * jj + 1] = __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_rne(r1));
            }
    }
    // key offset (within the 32-key chunk) of this lane's score j
    __device__ static int key_of(int q4, int j) { return 8 * q4 + j; }
    // bit j = visibility of key_of(q4, j), from a chunk mask over its 32 keys
    __device__ static uint32_t lane_bits(uint32_t m, int q4) { return (m >> (8 * q4)) & 0xFFu; }

    // S^T for keys [c, c+32) of a K tile (row stride KPAD).  s[j] <-> key_of(q4, j).
    __device__ static void scores(const bf16_t* Ks, int c, int lane, const QF* qf, float* s) {
        const int rho = lane & 15, q4 = lane >> 4;
        const int key0 = c + 8 * (rho >> 2) + (rho & 3);
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(Ks + key0 * KPAD + 32 * ks + 8 * q4);
            const bf16x8_t a1 =
                *reinterpret_cast<const bf16x8_t*>(Ks + (key0 + 4) * KPAD + 32 * ks + 8 * q4);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = s0[r];
            s[4 + r] = s1[r];
        }
    }
    // acc += V^T P^T for keys [c, c+32) of a V^T tile with row stride vst.
    __device__ static void pv(const bf16_t* Vt, int vst, int c, int lane, const float* p,
                              f32x4_t* acc) {
        const int rho = lane & 15, q4 = lane >> 4;
        bf16x8_t b;
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = (__bf16)p[j];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Vt + (16 * dt + rho) * vst + c + 8 * q4);
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[dt], 0, 0, 0);
        }
    }
    // Stage rows into LDS: K row-major (stride KPAD), V transposed (stride vst).
    // rows[kk] = element offset of key kk's row in k / v, or -1 (zero row).
    __device__ static void stage(bf16_t* Ks, bf16_t* Vt, int vst, const bf16_t* __restrict__ kg,
                                 const bf16_t* __restrict__ vg, const long long* rows, int nkeys,
                                 int tid, int nthr) {
        constexpr int PIECES = D / 8;
        for (int u = tid; u < nkeys * PIECES; u += nthr) {
            const int kk = u / PIECES, pc = u - kk * PIECES;
            const long long r = rows[kk];
            const uint4 val = r >= 0 ? ld16(kg + r + pc * 8) : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(Ks + kk * KPAD + pc * 8) = val;
        }
        // V: units of 4 keys x 8 dims, written as 8 rows of 4 keys (8 bytes)
        const int nquads = nkeys / 4;
        for (int u = tid; u < nquads * PIECES; u += nthr) {
            const int kq = u / PIECES, oc = u - kq * PIECES;
            uint4 x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const long long r = rows[4 * kq + e];
                x[e] = r >= 0 ? ld16(vg + r + oc * 8) : make_uint4(0, 0, 0, 0);
            }
            const uint32_t w[4][4] = {{x[0].x, x[0].y, x[0].z, x[0].w},
                                      {x[1].x, x[1].y, x[1].z, x[1].w},
                                      {x[2].x, x[2].y, x[2].z, x[2].w},
                                      {x[3].x, x[3].y, x[3].z, x[3].w}};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int wi = j >> 1;
                uint32_t lo, hi;
                if ((j & 1) == 0) {
                    lo = (w[0][wi] & 0xFFFFu) | (w[1][wi] << 16);
                    hi = (w[2][wi] & 0xFFFFu) | (w[3][wi] << 16);
                } else {
                    lo = (w[0][wi] >> 16) | (w[1][wi] & 0xFFFF0000u);
                    hi = (w[2][wi] >> 16) | (w[3][wi] & 0xFFFF0000u);
                }
                *reinterpret_cast<uint2*>(Vt + (oc * 8 + j) * vst + 4 * kq) = make_uint2(lo, hi);
            }
        }
    }
    __device__ static void store_out(bf16_t* o, const float* v4) {
        *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3]));
    }
    static constexpr int shared_bytes() { return (KT * KPAD + D * VST) * 2; }
    static constexpr int gather_bytes() { return (KC * KPAD + D * GVST) * 2 + KC * 8; }
};

template <int D> struct Tr<float, D> {
    static constexpr int KS = D / 4;
    static constexpr int DT = D / 16;
    static constexpr int KPAD = D + 4;
    static constexpr int VST = KPAD;   // V kept row-major for fp32
    static constexpr int GVST = KPAD;
    static constexpr int VEC = 4;
    typedef float QF;

    __device__ static void load_q(const float* qrow, int q4, bool ok, QF* qf) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = ok ? qrow[4 * ks + q4] : 0.f;
    }
    // RoPE of the loaded query (position pos): the lane holds dim 4 ks + q4;
    // its pair partner is read from the row
    __device__ static void rope_q(const AttnParams& p, const float* qrow, long long pos, int q4, QF* qf) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int ch = 4 * ks + q4;
            if (ch < p.rope_off || ch >= p.rope_off + p.rope_dim) continue;
            float s, c, r0, r1;
            rope_sincos(pos, (ch - p.rope_off) >> 1, p.rope_step, &s, &c);
            rope_turn(qrow[ch & ~1], qrow[ch | 1], s, c, &r0, &r1);
            qf[ks] = (ch & 1) ? r1 : r0;
        }
    }
    __device__ static int key_of(int q4, int j) { return 16 * (j >> 2) + 4 * (j & 3) + q4; }
    __device__ static uint32_t lane_bits(uint32_t m, int q4) {
        uint32_t r = 0u;
#pragma unroll
        for (int j = 0; j < 8; ++j) r |= ((m >> key_of(q4, j)) & 1u) << j;
        return r;
    }

    __device__ static void scores(const float* Ks, int c, int lane, const QF* qf, float* s) {
        const int rho = lane & 15, q4 = lane >> 4;
        const int key0 = c + 4 * (rho & 3) + (rho >> 2);
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(Ks[key0 * KPAD + 4 * ks + q4], qf[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(Ks[(key0 + 16) * KPAD + 4 * ks + q4], qf[ks], s1,
                                                      0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = s0[r];
            s[4 + r] = s1[r];
        }
    }
    __device__ static void pv(const float* Vs, int vst, int c, int lane, const float* p,
                              f32x4_t* acc) {
        const int rho = lane & 15, q4 = lane >> 4;
#pragma unroll
        for (int st = 0; st < 8; ++st) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const float a = Vs[(c + 4 * st + q4) * vst + 16 * dt + rho];
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, p[st], acc[dt], 0, 0, 0);
            }
        }
    }
    __device__ static void stage(float* Ks, float* Vs, int vst, const float* __restrict__ kg,
                                 const float* __restrict__ vg, const long long* rows, int nkeys,
                                 int tid, int nthr) {
        constexpr int PIECES = D / 4;
        for (int u = tid; u < nkeys * PIECES; u += nthr) {
            const int kk = u / PIECES, pc = u - kk * PIECES;
            const long long r = rows[kk];
            const uint4 a = r >= 0 ? ld16(kg + r + pc * 4) : make_uint4(0, 0, 0, 0);
            const uint4 b = r >= 0 ? ld16(vg + r + pc * 4) : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(Ks + kk * KPAD + pc * 4) = a;
            *reinterpret_cast<uint4*>(Vs + kk * vst + pc * 4) = b;
        }
    }
    __device__ static void store_out(float* o, const float* v4) {
        *reinterpret_cast<float4*>(o) = make_float4(v4[0], v4[1], v4[2], v4[3]);
    }
    static constexpr int shared_bytes() { return (KT * KPAD + KT * VST) * 4; }
    static constexpr int gather_bytes() { return (KC * KPAD + KC * GVST) * 4 + KC * 8; }
};

// ---------------------------------------------------------------- online softmax
template <int DT> struct State {
    float m;  // running max (log2 domain), identical across the 4 lane groups of a column
    float l;  // this lane's partial sum of weights
    f32x4_t acc[DT];
    __device__ void init() {
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int i = 0; i < DT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
};

// Reductions over the four lanes l, l^16, l^32, l^48 that hold one column.
// v_permlane16_swap / v_permlane32_swap exchange rows of 16 / halves of 32
// lanes in registers: swapping a value with itself leaves lane l holding the
// values of lanes l and l^16 (resp. l^32) in the two results.
__device__ __forceinline__ float col_max(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// fixed order: (l0 + l16) + (l32 + l48) on every lane of the column
__device__ __forceinline__ float col_sum(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One online-softmax step over NCH 32-key chunks (keys [c, c + 32 NCH) of a
// tile).  s[8 ch + j] is this lane's raw score of key key_of(q4, j) of chunk
// ch; bit 8 ch + j of mb says whether that key is attended (FULL: every key
// of the step is attended by every column of the wave); scale = softmax
// scale * log2(e) > 0.  The scale is applied inside the exponent's FMA and to
// the (monotone) column max.
template <int D, int NCH, bool FULL, typename PV>
__device__ __forceinline__ void softmax_pv(State<D / 16>& st, const float* s, uint32_t mb, float scale,
                                           PV&& pv) {
    constexpr int NJ = 8 * NCH;
    float x[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if constexpr (FULL) {
            x[j] = s[j];
        } else {
            // bit j of mb selects s[j], else -inf: sign-extended bit + bitfield insert
            const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)mb, j, 1);
            x[j] = __uint_as_float((__float_as_uint(s[j]) & sel) | (0xFF800000u & ~sel));
        }
    }
    float mloc = x[0];
#pragma unroll
    for (int j = 1; j < NJ; ++j) mloc = fmaxf(mloc, x[j]);
    mloc = col_max(mloc) * scale;
    // Lazy rescaling: the reference m of a column only moves when a new
    // maximum exceeds it by more than 8 (log2 units); weights are then at most
    // 2^8, which float32 sums and bf16 P operands hold without loss of
    // relative precision, and the reference cancels in acc / l.
    if (__builtin_expect(__any(mloc > st.m + 8.0f), 0)) {
        const float mnew = fmaxf(st.m, mloc);
        const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(st.m - mnew);
        st.l *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) st.acc[dt][r] *= alpha;
        st.m = mnew;
    }
    const float muse = st.m == -INFINITY ? 0.f : st.m;
    float p[NJ];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        p[j] = __builtin_amdgcn_exp2f(fmaf(x[j], scale, -muse));
        ps += p[j];
    }
    st.l += ps;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) pv(ch, p + 8 * ch, st.acc);
}

__device__ __forceinline__ long long n_visible(long long t, int W, int m, int N) {
    const long long s = t - W + 1;
    if (s <= 0) return 0;
    const long long n = s / m;
    return n < N ? n : N;
}

// ---------------------------------------------------------------- tile staging
// Register staging of one KT-key tile (global -> registers -> LDS), so the next
// tile's loads are in flight while the current tile is computed.
template <typename T, int D, int NT> struct Stage;

template <int D, int NT> struct Stage<float, D, NT> {
    static constexpr int PIECES = D / 4;
    static constexpr int KU = KT * PIECES;
    static constexpr int KP = (KU + NT - 1) / NT;
    uint4 k[KP], v[KP];
    __device__ void load(const float* __restrict__ kb, const float* __restrict__ vb, int rs, int nvalid, int tid) {
#pragma unroll
        for (int j = 0; j < KP; ++j) {
            const int u = tid + j * NT;
            const int kk = u / PIECES, pc = u % PIECES;
            const bool ok = kk < nvalid && (KU % NT == 0 || u < KU);
            const int off = (ok ? kk : 0) * rs + pc * 4;
            const uint4 x = ld16(kb + off), y = ld16(vb + off);
            k[j] = ok ? x : make_uint4(0, 0, 0, 0);
            v[j] = ok ? y : make_uint4(0, 0, 0, 0);
        }
    }
    __device__ void store(float* Ks, float* Vs, int tid) const {
        constexpr int KPAD = D + 4;
#pragma unroll
        for (int j = 0; j < KP; ++j) {
            const int u = tid + j * NT;
            if (KU % NT == 0 || u < KU) {
                const int kk = u / PIECES, pc = u % PIECES;
                *reinterpret_cast<uint4*>(Ks + kk * KPAD + pc * 4) = k[j];
                *reinterpret_cast<uint4*>(Vs + kk * KPAD + pc * 4) = v[j];
            }
        }
    }
};

// ---------------------------------------------------------------- tile I/O
// How a KT-key tile of one K/V source gets into LDS and into the MFMA operands.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) const uint32_t lds_cu32_t;   // decode table entries in LDS

template <typename T, int D, int NW> struct TileIO;

// bf16: K and V tiles are [KT][D] row-major in LDS, their 16-byte pieces
// XOR-swizzled per row, filled by direct global->LDS loads (each wave load
// writes 64 lanes x 16 bytes = RPI whole rows) with no register staging.
//  * K A-operand reads (16 rows per lane group, one piece each) and V^T
//    reads (4 rows x 32 bytes per lane group) hit distinct banks.
//  * V^T operands come from transposing LDS reads: within each 16-lane
//    group, lane i of ds_read_b64_tr_b16 receives element (i mod 4) of the 4
//    elements read by lane 4k + i/4 in slot k.  Lane s reading 4 elements of
//    key row (8 g + s/4) at dims 4 (s mod 4) .. +3 makes lane i hold keys
//    8 g + k, dim i: the A layout of O^T = V^T P^T.
// Reads of a bf16 K/V tile laid out as above ([rows][D], 16-byte pieces of
// row r at slot piece ^ swz(r)): S^T from K pieces, O^T += V^T P^T with
// transposing reads of V.
template <int D> struct TileReadBf16 {
    static constexpr int PIECES = D / 8;        // 16-byte pieces per row
    static constexpr int ROWB = D * 2;          // bytes per row
    static constexpr int RPI = 1024 / ROWB;     // rows per wave load (64 lanes x 16 bytes)
    static constexpr int KS = D / 32;
    static constexpr int DT = D / 16;
    int kro[KS];                 // byte offsets of this lane's K pieces (chunk-relative)
    int vro[4];                  // byte offsets of this lane's V^T reads (chunk-relative, dims < 64)
    int vhs;                     // byte step to this lane's V^T reads of dims 64..127

    __device__ static int swz_k(int row) { return ((row & 3) | (((row >> 3) & 3) << 2)) & (PIECES - 1); }
    // V: rows 8g + r (lane group g of a transposing read) use pieces 2 (r ^ t) + {0, 1};
    // at d = 128 bit 3 of the row also flips the upper half of the pieces, so
    // lane groups 0 / 1 (and 2 / 3) of one read use different LDS bank halves
    __device__ static int swz_v(int row) { return ((2 * (row & 3)) | (((row >> 3) & 1) << 3)) & (PIECES - 1); }

    __device__ void init_read(int lane) {
        const int rho = lane & 15, q4 = lane >> 4;
        const int key0 = 8 * (rho >> 2) + (rho & 3);  // S^T row rho of a chunk's first tile
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kro[ks] = key0 * ROWB + (((4 * ks + q4) ^ swz_k(key0)) * 16);
        const int g4 = lane >> 4, sl = lane & 15;
        const int vrow = 8 * g4 + (sl >> 2);
        const int hb = PIECES > 8 ? (g4 & 1) : 0;   // the row's upper-half flip (d = 128)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            vro[dt] = vrow * ROWB + (2 * (dt ^ (sl >> 2)) + ((sl & 3) >> 1)) * 16 + 8 * (sl & 1) + hb * 128;
        vhs = hb ? -128 : 128;
    }
    // S^T for keys [c, c+32) of the K tile at kbuf.  s[j] <-> key 8 q4 + j of the chunk.
    __device__ void scores_at(const char* kbuf, int c, const bf16x8_t* qf, float* s) const {
        const char* kb = kbuf + c * ROWB;
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(kb + kro[ks]);
            const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(kb + kro[ks] + 4 * ROWB);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], s1, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = s0[r];
            s[4 + r] = s1[r];
        }
    }
    // acc += V^T P^T for keys [c, c+32) of the V tile at vbuf
    __device__ void pv_at(const char* vbuf, int c, const float* p, f32x4_t* acc) const {
        const char* vb = vbuf + c * ROWB;
        bf16x8_t bop;
#pragma unroll
        for (int j = 0; j < 8; ++j) bop[j] = (__bf16)p[j];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const char* a = vb + vro[dt & 3] + (dt >> 2) * vhs;
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a + 4 * ROWB));
            const i16x4_t lohi[2] = {lo, hi};
            bf16x8_t aop;
            __builtin_memcpy(&aop, lohi, 16);
            acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bop, acc[dt], 0, 0, 0);
        }
    }
};

template <int D, int NW> struct TileIO<bf16_t, D, NW> : TileReadBf16<D> {
    typedef TileReadBf16<D> R;
    using R::PIECES;
    using R::ROWB;
    using R::RPI;
    using R::swz_k;
    using R::swz_v;
    static constexpr int NLOADS = KT / RPI;             // wave loads per matrix per tile
    static constexpr int NI = (NLOADS + NW - 1) / NW;   // of them per wave (at most)
    static constexpr int MAT_BYTES = KT * ROWB;
    static_assert(NLOADS * RPI == KT, "tile split");
    uint32_t boff_k[NI], boff_v[NI];  // byte offsets of this lane's global pieces
    int grow[NI];                     // their tile rows
    int wave;

    __device__ void init(int tid, int rs) {
        const int lane = tid & 63;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            // wave load j * NW + wave (when it exists) covers rows RPI * that .. +RPI
            const int row = (j * NW + wave) * RPI + lane / PIECES;
            const int pc = lane % PIECES;  // LDS slot piece; it holds global piece pc ^ swz(row)
            grow[j] = row;
            boff_k[j] = (uint32_t)(row * rs + (pc ^ swz_k(row)) * 8) * 2u;
            boff_v[j] = (uint32_t)(row * rs + (pc ^ swz_v(row)) * 8) * 2u;
        }
        this->init_read(lane);
    }
    // start loading rows [0, nvalid) of a tile (rows past nvalid repeat row 0).
    // Addresses are a wave-uniform base plus a 32-bit per-lane byte offset.
    __device__ void issue(const bf16_t* kb, const bf16_t* vb, int nvalid, char* buf) const {
        const char* kbb = reinterpret_cast<const char*>(kb);
        const char* vbb = reinterpret_cast<const char*>(vb);
        if (nvalid >= KT) {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if (NLOADS % NW != 0 && j * NW + wave >= NLOADS) break;   // uniform per wave
                char* dst = buf + (j * NW + wave) * 1024;
                __builtin_amdgcn_global_load_lds(kbb + boff_k[j], (lds_void_t*)dst, 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vbb + boff_v[j], (lds_void_t*)(dst + MAT_BYTES), 16, 0, 0);
            }
        } else {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                if (NLOADS % NW != 0 && j * NW + wave >= NLOADS) break;
                const bool ok = grow[j] < nvalid;
                char* dst = buf + (j * NW + wave) * 1024;
                __builtin_amdgcn_global_load_lds(kbb + (ok ? boff_k[j] : 0u), (lds_void_t*)dst, 16, 0, 0);
                __builtin_amdgcn_global_load_lds(vbb + (ok ? boff_v[j] : 0u), (lds_void_t*)(dst + MAT_BYTES), 16, 0,
                                                 0);
            }
        }
    }
    // the issued loads have landed in LDS (a barrier must follow)
    __device__ void commit(char*) const { __builtin_amdgcn_s_waitcnt(0); }

    // 4-bit sources: a tile's codes travel global -> registers in 16-byte
    // pieces of 32 codes, loaded while the previous tile is computed, and are
    // decoded at commit_q4 through the byte tables into the tile layout above.
    static constexpr int QPR = D / 32;                          // code pieces per row
    static constexpr int QP = 2 * KT * QPR;                     // code pieces per tile (K and V)
    static constexpr int NQ = (QP + NW * 64 - 1) / (NW * 64);   // of them per thread
    uint4 qc[NQ];
    lds_cu32_t* qlut_k;
    lds_cu32_t* qlut_v;
    int qtid;
    __device__ void init_q4(int tid) { qtid = tid; }
    // rows [0, nvalid) of a tile of codes at kb / vb (row stride rsb bytes);
    // rows past nvalid repeat row 0
    __device__ void issue_q4(const char* kb, const char* vb, long long rsb, int nvalid, lds_cu32_t* lk,
                             lds_cu32_t* lv) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int pid = qtid + j * NW * 64;
            if (QP % (NW * 64) != 0 && pid >= QP) break;
            const int mat = pid / (KT * QPR), r = pid - mat * (KT * QPR);
            const int row = r / QPR, pc = r - row * QPR;
            qc[j] = ld16((mat ? vb : kb) + (long long)(row < nvalid ? row : 0) * rsb + pc * 16);
        }
        qlut_k = lk;
        qlut_v = lv;
    }
    __device__ void commit_q4(char* buf) const {
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int pid = qtid + j * NW * 64;
            if (QP % (NW * 64) != 0 && pid >= QP) break;
            const int mat = pid / (KT * QPR), r = pid - mat * (KT * QPR);
            const int row = r / QPR, pc = r - row * QPR;
            lds_cu32_t* lut = mat ? qlut_v : qlut_k;
            const int sw = mat ? swz_v(row) : swz_k(row);
            char* rb = buf + mat * MAT_BYTES + row * ROWB;
            const uint32_t w[4] = {qc[j].x, qc[j].y, qc[j].z, qc[j].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint4 o = make_uint4(lut[w[u] & 255u], lut[(w[u] >> 8) & 255u], lut[(w[u] >> 16) & 255u],
                                           lut[w[u] >> 24]);
                *reinterpret_cast<uint4*>(rb + (((4 * pc + u) ^ sw) * 16)) = o;
            }
        }
    }
    __device__ void scores(const char* buf, int c, const bf16x8_t* qf, float* s) const {
        this->scores_at(buf, c, qf, s);
    }
    __device__ void pv(const char* buf, int c, const float* p, f32x4_t* acc) const {
        this->pv_at(buf + MAT_BYTES, c, p, acc);
    }
    static constexpr int buf_bytes() { return 2 * MAT_BYTES; }
};

// Per-wave chunk of KC gathered K and V rows (entries listed by lanes 0..KC-1)
// loaded straight into the wave's own LDS tiles, in the tile layout above.
template <int D> struct GatherBf16 : TileReadBf16<D> {
    typedef TileReadBf16<D> R;
    using R::PIECES;
    using R::ROWB;
    using R::RPI;
    using R::swz_k;
    using R::swz_v;
    static constexpr int NL = KC / RPI;       // wave loads per matrix
    static constexpr int MAT_BYTES = KC * ROWB;
    static_assert(NL * RPI == KC, "chunk split");
    int lrow[NL];                   // chunk row of this lane's piece in load j
    uint32_t poff_k[NL], poff_v[NL];  // byte offset of that piece within its row

    __device__ void init(int lane) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int row = j * RPI + lane / PIECES;
            const int pc = lane % PIECES;
            lrow[j] = row;
            poff_k[j] = (uint32_t)((pc ^ swz_k(row)) * 16);
            poff_v[j] = (uint32_t)((pc ^ swz_v(row)) * 16);
        }
        this->init_read(lane);
    }
    // load one matrix's chunk rows: this lane's piece of load j comes from
    // base + rowoff[j] + poff[j] (rowoff[j]: byte offset of chunk row lrow[j]'s
    // entry; a wave-uniform base plus 32-bit lane offsets)
    __device__ void issue(const char* base, const uint32_t* rowoff, const uint32_t* poff, char* dst) const {
#pragma unroll
        for (int j = 0; j < NL; ++j)
            __builtin_amdgcn_global_load_lds(base + (rowoff[j] + poff[j]), (lds_void_t*)(dst + j * 1024), 16, 0, 0);
    }
};

// fp32: register staging (global -> registers -> LDS), K row-major, V
// row-major, MFMA 16x16x4 operands read directly.
template <int D, int NW> struct TileIO<float, D, NW> {
    typedef Tr<float, D> TR;
    Stage<float, D, NW * 64> stg;
    int tid, lane, rs;
    __device__ void init(int tid_, int rs_) {
        tid = tid_;
        lane = tid_ & 63;
        rs = rs_;
    }
    __device__ void issue(const float* kb, const float* vb, int nvalid, char*) { stg.load(kb, vb, rs, nvalid, tid); }
    __device__ void commit(char* buf) const {
        stg.store(reinterpret_cast<float*>(buf), reinterpret_cast<float*>(buf) + KT * TR::KPAD, tid);
    }
    __device__ void scores(const char* buf, int c, const float* qf, float* s) const {
        TR::scores(reinterpret_cast<const float*>(buf), c, lane, qf, s);
    }
    __device__ void pv(const char* buf, int c, const float* p, f32x4_t* acc) const {
        TR::pv(reinterpret_cast<const float*>(buf) + KT * TR::KPAD, TR::VST, c, lane, p, acc);
    }
    static constexpr int buf_bytes() { return (KT * TR::KPAD + KT * TR::VST) * 4; }
};

// bits [a, b] of a 32-bit mask (empty when b < a or the range misses [0, 31])
__device__ __forceinline__ uint32_t range_mask(int a, int b) {
    a = a < 0 ? 0 : a;
    b = b > 31 ? 31 : b;
    if (b < a) return 0u;
    const uint32_t hi = b == 31 ? 0xFFFFFFFFu : ((2u << b) - 1u);
    return hi & ~((1u << a) - 1u);
}

// Gate weights of (query row qi of batch b, head h): per head, per row, or
// the softmax over the three branches of per-row logits.
__device__ __forceinline__ void load_gates(const AttnParams& p, int b, int qi, int h, float* g) {
    const float* src = p.gate_mode == 0 ? p.gates + h * 3 : p.gates + (((long long)b * p.Tq + qi) * p.H + h) * 3;
    g[0] = src[0];
    g[1] = src[1];
    g[2] = src[2];
    if (p.gate_mode == 2) {
        const float m = fmaxf(g[0], fmaxf(g[1], g[2]));
        const float e0 = expf(g[0] - m), e1 = expf(g[1] - m), e2 = expf(g[2] - m);
        const float inv = 1.0f / (e0 + e1 + e2);
        g[0] = e0 * inv;
        g[1] = e1 * inv;
        g[2] = e2 * inv;
    }
}

// ---------------------------------------------------------------- main kernel
enum { ITEM_WIN = 0, ITEM_HCA = 1, ITEM_CSA = 2 };

// GATHER: CSA entries are gathered per wave (else: attended densely with the
// selection bitmap, or absent); the two variants are separate kernels so that
// each carries only its own CSA code.  Q4 (bf16 only): the HCA and / or CSA
// caches may be 4-bit codes (p.q4).
template <typename T, int D, int NW, bool GATHER, bool Q4>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(AttnParams p) {
    static_assert(!Q4 || std::is_same<T, bf16_t>::value, "4-bit caches decode to bf16");
    typedef Tr<T, D> TR;
    constexpr int DT = D / 16;
    constexpr int NT = NW * 64;
    typedef TileIO<T, D, NW> TIO;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    auto tbuf = [&](int par) { return smem + par * TIO::buf_bytes(); };  // double-buffered K/V tiles
    __shared__ int sflag[4];
    __shared__ int emax_s;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = lane & 15, q4 = lane >> 4;

    // work decomposition: (b, g, query tile) [, split item].  Workgroups are
    // dealt round-robin to the 8 XCDs (each with its own L2); the work id is
    // remapped so that every XCD runs a contiguous range of work ids: the
    // query tiles of one (b, g), which share window rows and compressed
    // entries, then meet in one L2.
    // (split mode: a launch may run a range of the items; wid names the
    // item's absolute partial-state slot)
    const long long wl = xcd_work_id(blockIdx.x, gridDim.x);
    long long wg = wl;
    int item = 0;
    if (p.nsplit) {
        item = p.item_lo + (int)(wl % p.item_n);
        wg = wl / p.item_n;
    }
    const long long wid = p.nsplit ? wg * p.nsplit + item : wl;
    // later query tiles first: they attend the most CSA entries, so the
    // lightest work runs last and the tail of the launch is short
    const int qt = p.nqt - 1 - (int)(wg % p.nqt);
    const long long bg = wg / p.nqt;
    const int g = (int)(bg % p.Hkv);
    const int b = (int)(bg / p.Hkv);
    const int i0 = qt * p.QW;
    const int nq = min(p.QW, p.Tq - i0);
    // position of the sequence's query row 0; a negative per-sequence
    // position marks an inactive batch slot (its output rows are not written)
    const long long pos0 = p.q_pos ? (long long)p.q_pos[b] : p.q_pos0;
    if (pos0 < 0) return;

    const int col = wave * 16 + n;
    const int ql = col / p.G;
    const int hl = col - ql * p.G;
    const bool valid = (ql < nq);
    const int h = g * p.G + hl;
    const int qi = i0 + (valid ? ql : 0);
    const long long t = pos0 + qi;

    const T* qrow = reinterpret_cast<const T*>(p.q) + (((long long)b * p.Tq + qi) * p.H + (valid ? h : 0)) * D;
    typename TR::QF qf[TR::KS];
    TR::load_q(qrow, q4, valid, qf);
    if (p.rope_q && valid) TR::rope_q(p, qrow, t, q4, qf);

    float gate[3] = {0.f, 0.f, 0.f};
    if (valid) load_gates(p, b, qi, h, gate);
    // decode tables of the 4-bit caches: entry x of table s holds the bf16
    // values of codes x & 15 and x >> 4 of tensor s (code * step + min formed
    // in float64 and rounded once, as cache_dequant4 decodes)
    lds_cu32_t* luts = (lds_cu32_t*)(smem + p.lds_lut);
    if constexpr (Q4) {
        // only the tables this workgroup's key ranges read (a split item
        // covers one branch)
        int need = p.q4;
        if (p.nsplit) need &= item < p.n_win_items ? 0 : (item < p.n_win_items + p.n_hca_items ? 1 : 2);
        for (int i = tid; i < 4 * 256; i += NT) {
            const int st = i >> 8;
            if (!((need >> (st >> 1)) & 1)) continue;
            const double mn = p.q4p[st][0], step = p.q4p[st][1];
            const uint32_t lo = f64_to_bf16_rne(fma((double)(i & 15), step, mn));
            const uint32_t hi = f64_to_bf16_rne(fma((double)((i >> 4) & 15), step, mn));
            reinterpret_cast<uint32_t*>(smem + p.lds_lut)[i] = lo | (hi << 16);
        }
    }
    if (tid < 4) sflag[tid] = 0;
    if (tid == 0) emax_s = -1;
    __syncthreads();
    if (valid && gate[0] != 0.f) sflag[0] = 1;
    if (valid && gate[1] != 0.f) sflag[1] = 1;
    __syncthreads();
    const bool use_hca = p.has_hca && sflag[0] != 0;
    const bool use_csa = p.has_csa && sflag[1] != 0;

    const long long t_first = pos0 + i0;
    const long long t_last = pos0 + i0 + nq - 1;
    const long long win_lo = t - p.W + 1 > 0 ? t - p.W + 1 : 0;  // this column's window start

    // One running online-softmax state S and one output accumulator oacc per
    // column (two d-wide float32 arrays live); the branch schedule below folds
    // each branch into oacc, normalised and gated, as soon as it is complete.
    State<DT> S;
    S.init();
    f32x4_t oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto fold = [&](float gcoef) {   // oacc += gcoef * S / sum(S)
        const float l = col_sum(S.l);
        const float c = valid ? gcoef / l : 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[dt][r] = fmaf(c, S.acc[dt][r], oacc[dt][r]);
    };

    // which key ranges this workgroup covers (split mode: one item)
    bool do_win = true, do_hca = use_hca, do_csa = use_csa;
    long long hca_lo = 0, hca_hi = 0x7FFFFFFFFFFFLL, csa_lo = 0, csa_hi = -1;
    if (p.nsplit) {
        do_win = item < p.n_win_items;
        do_hca = use_hca && item >= p.n_win_items && item < p.n_win_items + p.n_hca_items;
        do_csa = use_csa && item >= p.n_win_items + p.n_hca_items;
        if (do_hca) {
            hca_lo = (long long)(item - p.n_win_items) * p.split_keys;
            hca_hi = hca_lo + p.split_keys;
        }
        if (do_csa) {
            csa_lo = (long long)(item - p.n_win_items - p.n_hca_items) * p.split_csa;
            csa_hi = csa_lo + p.split_csa;
        }
    }

    // ---- window geometry; the first window tile starts loading now, under the
    // bitmap set-up
    const long long w_lo = t_first - p.W + 1 > 0 ? t_first - p.W + 1 : 0;
    const int wlen = (int)(t_last + 1 - w_lo);
    const int rs = p.Hkv * D;  // row stride of every K/V tensor (elements)
    const long long hoff = (long long)g * D;
    // window rows [w_lo, t_last]: one contiguous run of raw rows, or with a
    // ring two runs, [0, wlen1) from ring row w_lo % Tr to the ring's end and
    // [wlen1, wlen) from ring row 0 (its base pointer is offset so that
    // window index k reads ring row k - wlen1)
    const long long r_lo = p.ring ? w_lo % p.Tr : w_lo - p.raw_pos0;
    const int wlen1 = p.ring ? (int)min((long long)wlen, p.Tr - r_lo) : wlen;
    const T* kraw = reinterpret_cast<const T*>(p.k_raw) + ((long long)b * p.Tr + r_lo) * rs + hoff;
    const T* vraw = reinterpret_cast<const T*>(p.v_raw) + ((long long)b * p.Tr + r_lo) * rs + hoff;
    const T* kraw2 = reinterpret_cast<const T*>(p.k_raw) + ((long long)b * p.Tr - wlen1) * rs + hoff;
    const T* vraw2 = reinterpret_cast<const T*>(p.v_raw) + ((long long)b * p.Tr - wlen1) * rs + hoff;
    int h_hi = do_hca ? (int)n_visible(t_last, p.W, p.m_hca, p.N_hca) : 0;
    if ((long long)h_hi > hca_hi) h_hi = (int)hca_hi;
    const int h_lo = do_hca ? (int)hca_lo : 0;
    // a 4-bit cache row is D / 2 bytes: its pointer arithmetic runs in bf16
    // units with row stride rs / 4 and head offset hoff / 4; lut_x is its K
    // decode table (V: lut_x + 1), -1 for rows in the dtype
    const bool hq = Q4 && (p.q4 & 1), cq = Q4 && (p.q4 & 2);
    const int hrs = hq ? rs / 4 : rs, crs = cq ? rs / 4 : rs;
    const int lut_h = hq ? 0 : -1, lut_c = cq ? 2 : -1;
    const T* khca = reinterpret_cast<const T*>(p.k_hca) + (long long)b * p.N_hca * hrs + (hq ? hoff / 4 : hoff);
    const T* vhca = reinterpret_cast<const T*>(p.v_hca) + (long long)b * p.N_hca * hrs + (hq ? hoff / 4 : hoff);
    TIO tio;
    tio.init(tid, rs);
    bool q4_pending = false;   // the tile in flight is 4-bit codes (in registers)
    if constexpr (Q4) tio.init_q4(tid);
    // start loading rows [row0, row0 + nvalid) of a source (row stride srs, in T units)
    // row stride (T units) and decode table of each key source
    auto src_rs = [&](int type) { return type == ITEM_HCA ? hrs : (type == ITEM_CSA ? crs : rs); };
    auto src_lut = [&](int type) { return type == ITEM_HCA ? lut_h : (type == ITEM_CSA ? lut_c : -1); };
    auto issue_src = [&](const T* kb, const T* vb, int type, int row0, int nvalid,
                         char* buf) __attribute__((always_inline)) {
        const int srs = src_rs(type), lut = src_lut(type);
        if constexpr (Q4) {
            q4_pending = lut >= 0;
            if (lut >= 0) {
                tio.issue_q4(reinterpret_cast<const char*>(kb + (long long)row0 * srs),
                             reinterpret_cast<const char*>(vb + (long long)row0 * srs), (long long)srs * 2, nvalid,
                             luts + lut * 256, luts + (lut + 1) * 256);
                return;
            }
        }
        tio.issue(kb + (long long)row0 * srs, vb + (long long)row0 * srs, nvalid, buf);
    };
    auto commit_src = [&](char* buf) __attribute__((always_inline)) {
        if constexpr (Q4) {
            if (q4_pending) {
                tio.commit_q4(buf);
                return;
            }
        }
        tio.commit(buf);
    };
    int parity = 0;
    bool pf = false;  // the first tile of the next stream is already on its way into tbuf(parity)
    // the first stream is the HCA one when it has entries, else the window
    if (do_hca && h_hi > h_lo) {
        issue_src(khca, vhca, ITEM_HCA, h_lo, min(KT, h_hi - h_lo), tbuf(0));
        pf = true;
    } else if (do_win && wlen > 0) {
        issue_src(kraw, vraw, ITEM_WIN, 0, min(KT, wlen1), tbuf(0));
        pf = true;
    }

    // ---- CSA selection bitmap (dense-masked mode)
    const bool dense_csa = !GATHER && do_csa && p.csa_mode == CSA_DENSE;
    uint32_t* bm = reinterpret_cast<uint32_t*>(smem + p.lds_bm);
    if (dense_csa) {
        // bitmap of the selections of the workgroup's queries; the nq index rows
        // are one contiguous [nq, k] block, read 4 entries at a time (k % 4 == 0,
        // checked on the host).  A row is ascending, so entries of one bitmap
        // word are adjacent: their bits are merged before one atomicOr.
        for (int u = tid; u < p.QW * p.bm_words / 4; u += NT)
            reinterpret_cast<uint4*>(bm)[u] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
        int emax = -1;
        const int4* rows = reinterpret_cast<const int4*>(p.idx + ((long long)b * p.Tq + i0) * p.k);
        const int n4 = nq * p.k / 4;
        // up to 4 of this thread's 16-byte index groups load together
        constexpr int NPF = 4;
        for (int u0 = tid; u0 < n4; u0 += NPF * NT) {
          int4 pre[NPF];
#pragma unroll
          for (int xp = 0; xp < NPF; ++xp)
            if (u0 + xp * NT < n4) pre[xp] = rows[u0 + xp * NT];
#pragma unroll
          for (int xp = 0; xp < NPF; ++xp) {
            const int u = u0 + xp * NT;
            if (u >= n4) break;
            const int4 e4 = pre[xp];
            const int qq = (4 * u) / p.k;
            uint32_t* brow = bm + qq * p.bm_words;
            const int ev[4] = {e4.x, e4.y, e4.z, e4.w};
            int cw = -1;
            uint32_t cbits = 0u;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int e = ev[x];
                if (e >= 0 && e < p.N_csa) {
                    emax = e > emax ? e : emax;
                    if ((e >> 5) != cw) {
                        if (cw >= 0) atomicOr(&brow[cw], cbits);
                        cw = e >> 5;
                        cbits = 0u;
                    }
                    cbits |= 1u << (e & 31);
                }
            }
            if (cw >= 0) atomicOr(&brow[cw], cbits);
          }
        }
        for (int off = 32; off > 0; off >>= 1) {
            const int o = __shfl_xor(emax, off);
            emax = o > emax ? o : emax;
        }
        if (lane == 0) atomicMax(&emax_s, emax);
        __syncthreads();
    }

    // ---- geometry: every index inside a stream is a 32-bit offset from the
    // workgroup's window start (window) or from entry 0 (HCA, CSA)
    const int c_hi = dense_csa ? emax_s + 1 : 0;
    const int wv_lo = valid ? (int)(win_lo - w_lo) : 1;  // column's window [wv_lo, wv_hi]
    const int wv_hi = valid ? (int)(t - w_lo) : 0;
    int hv = (valid && do_hca) ? (int)n_visible(t, p.W, p.m_hca, p.N_hca) : 0;
    if (hv > h_hi) hv = h_hi;
    const T* kcsa = reinterpret_cast<const T*>(p.k_csa) + (long long)b * p.N_csa * crs + (cq ? hoff / 4 : hoff);
    const T* vcsa = reinterpret_cast<const T*>(p.v_csa) + (long long)b * p.N_csa * crs + (cq ? hoff / 4 : hoff);

    // ---- wave-uniform key ranges attended by every valid column of the wave:
    // chunks inside them need no per-key mask
    // (scalar arithmetic: the wave's valid queries are qa..qb, and the window
    // start, window end and visible HCA count all grow with the position)
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int qa = (16 * wave_u) / p.G;
    const int qb = min((16 * wave_u + 15) / p.G, nq - 1);
    const bool wave_any = qa < nq;
    const long long ta = pos0 + i0 + qa, tb = pos0 + i0 + qb;
    int hf = do_hca ? (int)n_visible(ta, p.W, p.m_hca, p.N_hca) : 0;
    if (hf > h_hi) hf = h_hi;
    const int wf_lo = wave_any ? (int)((tb - p.W + 1 > 0 ? tb - p.W + 1 : 0) - w_lo) : INT_MAX;
    const int wf_hi = wave_any ? (int)(ta - w_lo) : INT_MIN;
    const int hf_hi = wave_any ? hf : INT_MIN;

    // ---- a pipelined stream of KT-key tiles of one source into S: tile i+1 is
    // on its way into the other LDS buffer while tile i is computed, and the
    // last tile of a stream overlaps the first tile of the next stream
    // (nkb, nvb, [nk_begin, nk_end)), so the pipeline does not drain between
    // branches
    auto stream = [&](const T* kb, const T* vb, int k_begin, int k_end, int type, const T* nkb, const T* nvb,
                      int nk_begin, int nk_end, int ntype) __attribute__((always_inline)) {
        const int n = k_end > k_begin ? (k_end - k_begin + KT - 1) / KT : 0;
        if (n == 0) return;
        if (!pf) issue_src(kb, vb, type, k_begin, min(KT, k_end - k_begin), tbuf(parity));
        pf = false;
        commit_src(tbuf(parity));
        __syncthreads();
        for (int i = 0; i < n; ++i) {
            const int k0 = k_begin + i * KT;
            const char* buf = tbuf(parity);
            if (i + 1 < n) {
                const int k1 = k0 + KT;
                issue_src(kb, vb, type, k1, min(KT, k_end - k1), tbuf(parity ^ 1));
            } else if (nk_end > nk_begin) {
                issue_src(nkb, nvb, ntype, nk_begin, min(KT, nk_end - nk_begin), tbuf(parity ^ 1));
                pf = true;
            }
            auto pvf = [&](int ch, const float* pp, f32x4_t* acc) { tio.pv(buf, ch * KC, pp, acc); };
            {
                // one softmax step over the whole KT = 2 KC key tile.  One code
                // path for every tile (the softmax state stays in place): a tile
                // inside the range of every column of the wave takes an all-ones
                // mask without computing it.
                bool full;
                if (type == ITEM_WIN) full = k0 >= wf_lo && k0 + KT - 1 <= min(wf_hi, k_end - 1);
                else if (type == ITEM_HCA) full = k0 + KT <= hf_hi;
                else full = false;
                constexpr int NCH = KT / KC;  // 32-key chunks per tile
                uint32_t mb = NCH == 2 ? 0xFFFFu : 0xFFu;
                if (!full) {
                    uint32_t m[NCH];
#pragma unroll
                    for (int ch = 0; ch < NCH; ++ch) {
                        const int kc0 = k0 + ch * KC;
                        if (type == ITEM_WIN) m[ch] = range_mask(wv_lo - kc0, min(wv_hi, k_end - 1) - kc0);
                        else if (type == ITEM_HCA) m[ch] = range_mask(0, hv - kc0 - 1);
                    }
                    if (type == ITEM_CSA) {
                        const bool ok = valid && k0 < c_hi;
                        if constexpr (NCH == 2) {
                            const uint2 w2 = ok ? *reinterpret_cast<const uint2*>(bm + ql * p.bm_words + (k0 >> 5))
                                                : make_uint2(0u, 0u);
                            m[0] = w2.x;
                            m[NCH - 1] = w2.y;
                        } else {
                            m[0] = ok ? bm[ql * p.bm_words + (k0 >> 5)] : 0u;
                        }
                    }
                    mb = 0u;
#pragma unroll
                    for (int ch = 0; ch < NCH; ++ch) mb |= TR::lane_bits(m[ch], q4) << (8 * ch);
                }
                float sc[8 * NCH];
#pragma unroll
                for (int ch = 0; ch < NCH; ++ch) tio.scores(buf, ch * KC, qf, sc + 8 * ch);
                softmax_pv<D, NCH, false>(S, sc, mb, p.scale_log2, pvf);
            }
            parity ^= 1;
            if (i + 1 < n) commit_src(tbuf(parity));
            __syncthreads();
        }
    };

    // ---- the window, in one run of raw rows or two (ring wrap-around), then
    // the stream that follows it
    auto window = [&](const T* nkb, const T* nvb, int nk_begin, int nk_end,
                      int ntype) __attribute__((always_inline)) {
        if (wlen1 < wlen) {
            stream(kraw, vraw, 0, wlen1, ITEM_WIN, kraw2, vraw2, wlen1, wlen, ITEM_WIN);
            stream(kraw2, vraw2, wlen1, wlen, ITEM_WIN, nkb, nvb, nk_begin, nk_end, ntype);
        } else {
            stream(kraw, vraw, 0, wlen, ITEM_WIN, nkb, nvb, nk_begin, nk_end, ntype);
        }
    };

    // ---- CSA gather, bf16: per-wave K/V chunk tiles in LDS (aliasing the
    // stream buffers) and a two-slot ring of entry lists, all loaded by DMA,
    // so that every vector-memory operation of the loop is a direct-to-LDS
    // load and the waits below can count them.  Chunk ci: scores from the K
    // tile; the entries of chunk ci + 1 (read from the ring) give the next
    // K rows, which go out with the entry list of chunk ci + 2; softmax; PV
    // from the V tile, then the next V rows go out.  V(ci) is in flight
    // during the scores and softmax, K(ci + 1) during the PV; the last chunk
    // issues nothing more and waits for everything.  The tiles are
    // restrict pointers: the compiler then knows that loads into one never
    // write another and adds no waits of its own beyond these.
    auto gather_dma = [&]() {
      if constexpr (std::is_same<T, bf16_t>::value) {
        typedef GatherBf16<D> GB;
        constexpr int NL = GB::NL;   // loads per K or V chunk tile
        GB gio;
        gio.init(lane);
        const uint32_t rsb = (uint32_t)p.Hkv * D * 2;   // bytes between entries (host: N_csa * rsb < 2^32)
        const char* kc = reinterpret_cast<const char*>(p.k_csa) + (long long)b * p.N_csa * rsb + hoff * 2;
        const char* vc = reinterpret_cast<const char*>(p.v_csa) + (long long)b * p.N_csa * rsb + hoff * 2;
        const int ql_a = (wave * 16) / p.G;
        const int ql_b = min((wave * 16 + 15) / p.G, nq - 1);
        int j_lo = 0, j_hi = p.k;
        if (p.nsplit) {
            j_lo = (int)csa_lo;
            j_hi = csa_hi < p.k ? (int)csa_hi : p.k;
        }
        const int nj = j_hi > j_lo ? (j_hi - j_lo + KC - 1) / KC : 0;
        const int nchunks = ql_b >= ql_a ? (ql_b - ql_a + 1) * nj : 0;
        if (nchunks == 0 || p.N_csa == 0) return;   // no entries: nothing to attend (or to load)
        // chunk c (clamped to the last) -> its query and first list position
        auto chunk_at = [&](int c, int& qq, int& jb) {
            c = min(c, nchunks - 1);
            qq = ql_a + c / nj;
            jb = j_lo + (c - (qq - ql_a) * nj) * KC;
        };
        auto run = [&](char* __restrict__ tk, char* __restrict__ tv, char* __restrict__ te)
                       __attribute__((always_inline)) {
            // the entry list of chunk c into ring slot c & 1 (256 bytes: lane l
            // writes the 4 bytes at 4 l; lanes >= KC repeat lanes < KC, and
            // positions past the list repeat its last entry)
            auto issue_entries = [&](int c) {
                int qq, jb;
                chunk_at(c, qq, jb);
                const int pos = min(jb + (lane & (KC - 1)), j_hi - 1);
                const int* src = p.idx + ((long long)b * p.Tq + i0 + qq) * p.k + pos;
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(src), (lds_void_t*)(te + (c & 1) * 256),
                                                 4, 0, 0);
            };
            // row offsets of chunk c's loads for this lane (entries past the
            // list, negative or beyond the cache read row 0 and are masked)
            // and the chunk's valid-row bits (bit r: row r)
            auto read_entries = [&](int c, uint32_t* ro, unsigned long long& vr) {
                int qq, jb;
                chunk_at(c, qq, jb);
                const int nv = j_hi - jb;   // rows below nv hold list positions
                const int* ent = reinterpret_cast<const int*>(te + (c & 1) * 256);
#pragma unroll
                for (int j = 0; j < NL; ++j) {
                    const int r = gio.lrow[j];
                    const int e = ent[r];
                    ro[j] = (r < nv && e >= 0 && e < p.N_csa) ? (uint32_t)e * rsb : 0u;
                }
                const int r = lane & (KC - 1);
                const int e = ent[r];
                vr = __ballot(lane < KC && r < nv && e >= 0 && e < p.N_csa);
            };
            __builtin_amdgcn_s_waitcnt(0);
            issue_entries(0);
            issue_entries(1);
            wait_vmcnt<1>();   // the entries of chunk 0
            wave_lds_sync();
            uint32_t ro[NL];
            unsigned long long vrows;
            read_entries(0, ro, vrows);
            gio.issue(kc, ro, gio.poff_k, tk);
            gio.issue(vc, ro, gio.poff_v, tv);
            for (int ci = 0; ci < nchunks; ++ci) {
                // in flight, oldest first: K(ci) [NL], entries(ci + 1) [1], V(ci) [NL]
                wait_vmcnt<NL>();
                wave_lds_sync();
                const int qq = ql_a + ci / nj;
                float sc[8];
                gio.scores_at(tk, 0, qf, sc);
                wave_lds_sync();   // this wave's K reads are complete
                const bool more = ci + 1 < nchunks;
                unsigned long long vr_n = 0ull;
                if (more) {
                    read_entries(ci + 1, ro, vr_n);
                    gio.issue(kc, ro, gio.poff_k, tk);   // K tile is free again
                    issue_entries(ci + 2);
                }
                const uint32_t mb = (valid && ql == qq) ? (uint32_t)(vrows >> (8 * q4)) & 0xFFu : 0u;
                softmax_pv<D, 1, false>(S, sc, mb, p.scale_log2, [&](int, const float* pp, f32x4_t* acc) {
                    // in flight, oldest first: V(ci) [NL], then (more) K(ci + 1)
                    // [NL] and entries(ci + 2) [1]
                    if (more) wait_vmcnt<NL + 1>();
                    else wait_vmcnt<0>();
                    wave_lds_sync();
                    gio.pv_at(tv, 0, pp, acc);
                });
                wave_lds_sync();   // this wave's V reads are complete
                if (more) gio.issue(vc, ro, gio.poff_v, tv);   // V tile is free again
                vrows = vr_n;
            }
            __builtin_amdgcn_s_waitcnt(0);
        };
        char* gk = smem + p.lds_gather + wave * p.lds_gather_stride;
        run(gk, gk + GB::MAT_BYTES, gk + 2 * GB::MAT_BYTES);
      }
    };

    // ---- CSA gather of 4-bit rows: the same per-wave tiles and entry walk as
    // gather_dma, but the rows' codes travel global -> registers (loaded one
    // chunk ahead, during this chunk's scores, softmax and PV) and are decoded
    // through the CSA tables into the bf16 tile layout at the top of the chunk.
    auto gather_q4 = [&]() {
      if constexpr (std::is_same<T, bf16_t>::value) {
        typedef GatherBf16<D> GB;
        char* gk = smem + p.lds_gather + wave * p.lds_gather_stride;
        char* gv = gk + GB::MAT_BYTES;
        GB gio;
        gio.init(lane);
        constexpr int QPR = D / 32;            // 16-byte code pieces per row
        constexpr int NLQ = KC * QPR / 64;     // pieces per lane per matrix
        static_assert(NLQ * 64 == KC * QPR, "chunk split");
        const long long ers = (long long)p.Hkv * (D / 2);   // bytes between entries
        const char* kc = reinterpret_cast<const char*>(kcsa);
        const char* vc = reinterpret_cast<const char*>(vcsa);
        lds_cu32_t* lk = luts + 2 * 256;
        lds_cu32_t* lv = luts + 3 * 256;
        const int ql_a = (wave * 16) / p.G;
        const int ql_b = min((wave * 16 + 15) / p.G, nq - 1);
        int j_lo = 0, j_hi = p.k;
        if (p.nsplit) {
            j_lo = (int)csa_lo;
            j_hi = csa_hi < p.k ? (int)csa_hi : p.k;
        }
        const int nj = j_hi > j_lo ? (j_hi - j_lo + KC - 1) / KC : 0;
        const int nchunks = ql_b >= ql_a ? (ql_b - ql_a + 1) * nj : 0;
        if (nchunks == 0 || p.N_csa == 0) return;
        auto entry = [&](int ci) -> int {
            const int qq = ql_a + ci / nj;
            const int j = j_lo + (ci - (qq - ql_a) * nj) * KC + lane;
            int e = -1;
            if (lane < KC && j < j_hi) {
                e = p.idx[((long long)b * p.Tq + i0 + qq) * p.k + j];
                if (e < 0 || e >= p.N_csa) e = -1;
            }
            return e;
        };
        uint4 ck[NLQ], cv[NLQ];
        // codes of the chunk whose entries lanes < KC hold (e >= 0)
        auto load = [&](int e) {
#pragma unroll
            for (int j = 0; j < NLQ; ++j) {
                const int pid = j * 64 + lane;
                const int row = pid / QPR, pc = pid - row * QPR;
                const long long off = (long long)__shfl(e, row) * ers + pc * 16;
                ck[j] = ld16(kc + off);
                cv[j] = ld16(vc + off);
            }
        };
        auto expand = [&]() {
#pragma unroll
            for (int j = 0; j < NLQ; ++j) {
                const int pid = j * 64 + lane;
                const int row = pid / QPR, pc = pid - row * QPR;
#pragma unroll
                for (int mat = 0; mat < 2; ++mat) {
                    const uint4 c4 = mat ? cv[j] : ck[j];
                    const uint32_t w[4] = {c4.x, c4.y, c4.z, c4.w};
                    lds_cu32_t* lut = mat ? lv : lk;
                    const int sw = mat ? GB::swz_v(row) : GB::swz_k(row);
                    char* rb = (mat ? gv : gk) + row * GB::ROWB;
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const uint4 o = make_uint4(lut[w[u] & 255u], lut[(w[u] >> 8) & 255u],
                                                   lut[(w[u] >> 16) & 255u], lut[w[u] >> 24]);
                        *reinterpret_cast<uint4*>(rb + (((4 * pc + u) ^ sw) * 16)) = o;
                    }
                }
            }
        };
        int e_cur = entry(0);
        load(max(e_cur, 0));
        int e_nxt = nchunks > 1 ? entry(1) : -1;
        for (int ci = 0; ci < nchunks; ++ci) {
            expand();          // the previous chunk's LDS reads ended at the sync below
            wave_lds_sync();
            const int qq = ql_a + ci / nj;
            const unsigned long long vrows = __ballot(lane < KC && e_cur >= 0);
            const bool more = ci + 1 < nchunks;
            if (more) load(max(e_nxt, 0));
            float sc[8];
            gio.scores_at(gk, 0, qf, sc);
            const uint32_t mb = (valid && ql == qq) ? (uint32_t)(vrows >> (8 * q4)) & 0xFFu : 0u;
            softmax_pv<D, 1, false>(S, sc, mb, p.scale_log2,
                                    [&](int, const float* pp, f32x4_t* acc) { gio.pv_at(gv, 0, pp, acc); });
            wave_lds_sync();   // this wave's K and V reads are complete
            if (more) {
                e_cur = e_nxt;
                e_nxt = ci + 2 < nchunks ? entry(ci + 2) : -1;
            }
        }
      }
    };

    // ---- CSA gather (per wave, private LDS tiles aliasing the stream buffers)
    auto gather = [&]() {
        char* gbase = smem + p.lds_gather + wave * p.lds_gather_stride;
        T* gK = reinterpret_cast<T*>(gbase);
        T* gV = gK + KC * TR::KPAD;
        long long* grows = reinterpret_cast<long long*>(gbase + p.lds_gather_stride - KC * 8);
        const T* kc = reinterpret_cast<const T*>(p.k_csa);
        const T* vc = reinterpret_cast<const T*>(p.v_csa);
        const int c_first = wave * 16, c_last = wave * 16 + 15;
        const int ql_a = c_first / p.G;
        int ql_b = c_last / p.G;
        if (ql_b > nq - 1) ql_b = nq - 1;
        long long j_lo = 0, j_hi = p.k;
        if (p.nsplit) {
            j_lo = csa_lo;
            j_hi = csa_hi < p.k ? csa_hi : p.k;
        }
        for (int qq = ql_a; qq <= ql_b; ++qq) {
            const int32_t* sel = p.idx + ((long long)b * p.Tq + i0 + qq) * p.k;
            for (long long j0 = j_lo; j0 < j_hi; j0 += KC) {
                if (lane < KC) {
                    const long long j = j0 + lane;
                    const int e = j < j_hi ? sel[j] : -1;
                    grows[lane] = (e >= 0 && e < p.N_csa) ? ((((long long)b * p.N_csa + e) * p.Hkv + g) * D) : -1;
                }
                wave_lds_sync();
                const bool anyv = lane < KC ? grows[lane] >= 0 : false;
                if (!__any(anyv)) {
                    wave_lds_sync();
                    continue;
                }
                TR::stage(gK, gV, TR::GVST, kc, vc, grows, KC, lane, 64);
                wave_lds_sync();
                float sc[8];
                TR::scores(gK, 0, lane, qf, sc);
                uint32_t mb = 0u;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bool vis = valid && ql == qq && grows[TR::key_of(q4, j)] >= 0;
                    mb |= (vis ? 1u : 0u) << j;
                }
                softmax_pv<D, 1, false>(S, sc, mb, p.scale_log2, [&](int, const float* pp, f32x4_t* acc) {
                    TR::pv(gV, TR::GVST, 0, lane, pp, acc);
                });
                wave_lds_sync();
            }
        }
    };

    // ---- the branch schedule
    if (!p.nsplit) {
        // HCA entries alone first; their raw state parks in oacc.  Then the
        // window once: O_SWA is the window state, and O_HCA merges the window
        // and HCA states, which needs only their maxima and sums:
        //   O_HCA = (e_w A_w + e_h A_h) / (e_w l_w + e_h l_h),  e_x = 2^(m_x - M).
        // Finally the CSA entries continue the window's state (O_CSA).
        // Each stream names the one that follows it (none before a gather:
        // the gather reuses the tile buffers).
        float m_h = -INFINITY, l_h = 0.f;
        if (do_hca) {
            stream(khca, vhca, h_lo, h_hi, ITEM_HCA, kraw, vraw, 0, wlen1, ITEM_WIN);
            m_h = S.m;
            l_h = col_sum(S.l);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) oacc[dt] = S.acc[dt];
            S.init();
        }
        if (do_csa && !GATHER) window(kcsa, vcsa, 0, c_hi, ITEM_CSA);
        else window(nullptr, nullptr, 0, 0, ITEM_WIN);
        {
            const float l_w = col_sum(S.l);
            float c_w = valid ? gate[2] / l_w : 0.f, c_h = 0.f;
            if (do_hca) {
                const float M = fmaxf(S.m, m_h);
                const float e_w = __builtin_amdgcn_exp2f(S.m - M);
                const float e_h = m_h == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_h - M);
                const float den = fmaf(l_w, e_w, l_h * e_h);
                if (valid) {
                    c_w += gate[0] * e_w / den;
                    c_h = gate[0] * e_h / den;
                }
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) oacc[dt][r] = fmaf(c_w, S.acc[dt][r], c_h * oacc[dt][r]);
        }
        if (do_csa) {
            if constexpr (!GATHER) {
                stream(kcsa, vcsa, 0, c_hi, ITEM_CSA, nullptr, nullptr, 0, 0, ITEM_WIN);
            } else {
                __syncthreads();  // the stream buffers become the per-wave gather tiles
                if constexpr (Q4) {
                    if (cq) gather_q4();
                    else gather_dma();
                } else if constexpr (std::is_same<T, bf16_t>::value) {
                    gather_dma();
                } else {
                    gather();
                }
                __syncthreads();
            }
            fold(gate[1]);
        }
    } else {
        // one key range per workgroup; partial states are merged by the combine kernel
        if (do_win) window(nullptr, nullptr, 0, 0, ITEM_WIN);
        if (do_csa) {
            if constexpr (!GATHER) {
                stream(kcsa, vcsa, 0, c_hi, ITEM_CSA, nullptr, nullptr, 0, 0, ITEM_WIN);
            } else {
                __syncthreads();
                if constexpr (Q4) {
                    if (cq) gather_q4();
                    else gather_dma();
                } else if constexpr (std::is_same<T, bf16_t>::value) {
                    gather_dma();
                } else {
                    gather();
                }
                __syncthreads();
            }
        }
        if (do_hca) stream(khca, vhca, h_lo, h_hi, ITEM_HCA, nullptr, nullptr, 0, 0, ITEM_WIN);
    }

    // ------------------------------------------------------------ epilogue
    if (p.nsplit) {
        // partial state of this item: [m, l, -, -, acc[D]] per column at
        // ws[((wg * nsplit + item) * ncol + col) * (D + 4)]
        const float ltot = col_sum(S.l);
        if (!valid) return;   // the combine kernel reads valid columns only
        float* dst = p.ws + (wid * p.ncol + col) * (D + 4);
        if (q4 == 0) {
            dst[0] = S.m;
            dst[1] = ltot;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<float4*>(dst + 4 + 16 * dt + 4 * q4) =
                make_float4(S.acc[dt][0], S.acc[dt][1], S.acc[dt][2], S.acc[dt][3]);
        return;
    }
    if (!valid) return;
    T* orow = reinterpret_cast<T*>(p.out) + (((long long)b * p.Tq + qi) * p.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        float v4[4] = {oacc[dt][0], oacc[dt][1], oacc[dt][2], oacc[dt][3]};
        TR::store_out(orow + 16 * dt + 4 * q4, v4);
    }
}

// Merge the split partial states: one thread per (column, 4 dims).
// Every variant the launcher can select, instantiated explicitly (the host
// compiler otherwise dropped the stubs of some variants).
#define SHATTN_ATTN_INST(T, D, Q)                                               \
    template __global__ void attn_fwd_kernel<T, D, 4, false, Q>(AttnParams);    \
    template __global__ void attn_fwd_kernel<T, D, 4, true, Q>(AttnParams);     \
    template __global__ void attn_fwd_kernel<T, D, 2, false, Q>(AttnParams);    \
    template __global__ void attn_fwd_kernel<T, D, 2, true, Q>(AttnParams);
SHATTN_ATTN_INST(bf16_t, 64, false)
SHATTN_ATTN_INST(bf16_t, 128, false)
SHATTN_ATTN_INST(bf16_t, 64, true)
SHATTN_ATTN_INST(bf16_t, 128, true)
SHATTN_ATTN_INST(float, 64, false)
SHATTN_ATTN_INST(float, 128, false)
#undef SHATTN_ATTN_INST

// Merge of the split partial states.  Eight consecutive threads share one
// (column, 4 dims): each merges every eighth item of a range, then the eight
// partial states combine across the lanes in a fixed order (deterministic).
constexpr int kCombineSub = 8;

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    constexpr int DQ = D / 4;
    const int sub = (int)(gid % kCombineSub);
    const long long rest = gid / kCombineSub;
    const long long ncols_total = (long long)p.B * p.Hkv * p.nqt * p.ncol;
    if (rest >= ncols_total * DQ) return;   // whole groups of eight
    const int dq = (int)(rest % DQ);
    const long long cg = rest / DQ;          // global column
    const int col = (int)(cg % p.ncol);
    const long long wg = cg / p.ncol;
    // the work-id -> query-tile map of the main kernel
    const int qt = p.nqt - 1 - (int)(wg % p.nqt);
    const long long bg = wg / p.nqt;
    const int g = (int)(bg % p.Hkv);
    const int b = (int)(bg / p.Hkv);
    const int i0 = qt * p.QW;
    const int nq = min(p.QW, p.Tq - i0);
    const int ql = col / p.G, hl = col - (col / p.G) * p.G;
    if (ql >= nq) return;                    // uniform over the group of eight
    if (p.q_pos && p.q_pos[b] < 0) return;   // inactive batch slot
    const int h = g * p.G + hl;
    const int qi = i0 + ql;
    float gw[3];
    load_gates(p, b, qi, h, gw);
    const float g0 = gw[0], g1 = gw[1], g2 = gw[2];
    const bool use_hca = p.has_hca && p.n_hca_items > 0;
    const bool use_csa = p.has_csa && p.nsplit > p.n_win_items + p.n_hca_items;
    auto part = [&](int item) -> const float* {
        return p.ws + ((wg * p.nsplit + item) * p.ncol + col) * (D + 4);
    };
    // (m, l, a) <- merge of (m, l, a) and (mi, li, ai)
    auto fold_in = [](float& m, float& l, float* a, float mi, float li, const float* ai) {
        if (mi == -INFINITY) return;
        const float mn = fmaxf(m, mi);
        const float x = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        const float y = __builtin_amdgcn_exp2f(mi - mn);
        l = l * x + li * y;
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = a[r] * x + ai[r] * y;
        m = mn;
    };
    // merge items [it0, it1) into (m, l, a): strided over the group, then across it
    auto merge = [&](int it0, int it1, float& m, float& l, float* a) {
        float pm = -INFINITY, pl = 0.f, pa[4] = {0.f, 0.f, 0.f, 0.f};
        // four of this lane's items per round: their loads go out together,
        // then they fold in item order
        constexpr int U = 4;
        for (int it = it0 + sub; it < it1; it += U * kCombineSub) {
            float2 ml[U];
            float4 ai[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int iu = it + u * kCombineSub;
                if (iu < it1) {
                    const float* s = part(iu);
                    ml[u] = *reinterpret_cast<const float2*>(s);
                    ai[u] = *reinterpret_cast<const float4*>(s + 4 + 4 * dq);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (it + u * kCombineSub < it1) {
                    const float av[4] = {ai[u].x, ai[u].y, ai[u].z, ai[u].w};
                    fold_in(pm, pl, pa, ml[u].x, ml[u].y, av);
                }
            }
        }
#pragma unroll
        for (int off = 1; off < kCombineSub; off <<= 1) {
            const float om = __shfl_xor(pm, off), ol = __shfl_xor(pl, off);
            float oa[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) oa[r] = __shfl_xor(pa[r], off);
            // lower lane's state first on both lanes
            if (sub & off) {
                float tm = om, tl = ol, ta[4] = {oa[0], oa[1], oa[2], oa[3]};
                fold_in(tm, tl, ta, pm, pl, pa);
                pm = tm;
                pl = tl;
#pragma unroll
                for (int r = 0; r < 4; ++r) pa[r] = ta[r];
            } else {
                fold_in(pm, pl, pa, om, ol, oa);
            }
        }
        fold_in(m, l, a, pm, pl, pa);
    };
    float mw = -INFINITY, lw = 0.f, aw[4] = {0.f, 0.f, 0.f, 0.f};
    merge(0, p.n_win_items, mw, lw, aw);
    float o[4];
    for (int r = 0; r < 4; ++r) o[r] = g2 * aw[r] / lw;
    if (use_hca && g0 != 0.f) {
        float m = mw, l = lw, a[4] = {aw[0], aw[1], aw[2], aw[3]};
        merge(p.n_win_items, p.n_win_items + p.n_hca_items, m, l, a);
        for (int r = 0; r < 4; ++r) o[r] += g0 * a[r] / l;
    }
    if (use_csa && g1 != 0.f) {
        float m = mw, l = lw, a[4] = {aw[0], aw[1], aw[2], aw[3]};
        merge(p.n_win_items + p.n_hca_items, p.nsplit, m, l, a);
        for (int r = 0; r < 4; ++r) o[r] += g1 * a[r] / l;
    }
    if (sub == 0) {
        T* orow = reinterpret_cast<T*>(p.out) + (((long long)b * p.Tq + qi) * p.H + h) * D;
        Tr<T, D>::store_out(orow + 4 * dq, o);
    }
}

struct Plan {
    AttnParams p;
    int waves;
    size_t lds;
    long long grid;
    size_t ws_bytes;
    bool launch_main;   // the attention kernel runs (a CSA-items call without CSA items does not)
    bool combine;       // the split partial states are merged after it
};

int make_plan(const shattn_fwd_args* a, Plan& pl) {
    if (!a) return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: null args");
    if (a->struct_size != (int)sizeof(shattn_fwd_args))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: struct_size %d != %d", a->struct_size,
                    (int)sizeof(shattn_fwd_args));
    if (a->gate_mode < 0 || a->gate_mode > 2)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: gate_mode %d (0, 1 or 2)", a->gate_mode);
    if (a->dtype != SHATTN_DTYPE_BF16 && a->dtype != SHATTN_DTYPE_F32)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: unknown dtype %d", a->dtype);
    if (a->B < 0 || a->Tq < 0 || a->H < 1 || a->Hkv < 1 || a->W < 1 || a->Tr < 0)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: bad sizes B=%d Tq=%d H=%d Hkv=%d W=%d Tr=%d",
                    a->B, a->Tq, a->H, a->Hkv, a->W, a->Tr);
    if (a->H % a->Hkv != 0)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: H=%d not a multiple of Hkv=%d", a->H, a->Hkv);
    if (a->d != 64 && a->d != 128)
        return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_fwd: d=%d (supported: 64, 128)", a->d);
    const int G = a->H / a->Hkv;
    if (G > 64) return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_fwd: H/Hkv=%d > 64", G);
    if (!(a->sm_scale >= 0.f) || !std::isfinite(a->sm_scale))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: sm_scale must be finite and >= 0");
    if (a->q_pos0 < 0 || a->raw_pos0 < 0)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: negative position");
    if (a->reserved0 != 0) return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: reserved0 must be 0");
    if (a->raw_ring != 0 && a->raw_ring != 1)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: raw_ring %d (0 or 1)", a->raw_ring);
    if (a->q_pos && !a->raw_ring)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: per-sequence positions (q_pos) need raw_ring = 1");
    if (a->q_pos && (reinterpret_cast<uintptr_t>(a->q_pos) & 7))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: q_pos must be 8-byte aligned");
    // a branch is present iff its ratio (HCA) / row width k (CSA) is positive
    const bool has_hca = a->m_hca > 0;
    const bool has_csa = a->k > 0;
    if (a->m_hca < 0 || a->k < 0 || a->N_hca < 0 || a->N_csa < 0)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: negative m_hca / k / N_hca / N_csa");
    if (has_hca && a->N_hca > 0 && (!a->k_hca || !a->v_hca))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: HCA branch needs k_hca and v_hca");
    if (has_csa && ((a->N_csa > 0 && (!a->k_csa || !a->v_csa)) || (a->B > 0 && a->Tq > 0 && !a->idx)))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: CSA branch needs k_csa, v_csa and idx");
    if (has_csa && a->k > 4096) return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_fwd: k=%d > 4096", a->k);
    if (a->reserved1 != 0) return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: reserved1 must be 0");
    if (a->cache_q4 & ~3)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: cache_q4 = %d (bits 0 and 1 only)", a->cache_q4);
    // 4-bit caches of the branches present
    const int q4 = (has_hca ? (a->cache_q4 & 1) : 0) | (has_csa ? (a->cache_q4 & 2) : 0);
    if (q4 && a->dtype != SHATTN_DTYPE_BF16)
        return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_fwd: 4-bit caches need dtype bf16");
    const float* q4p[4] = {a->q4_k_hca, a->q4_v_hca, a->q4_k_csa, a->q4_v_csa};
    for (int i = 0; i < 4; ++i)
        if ((q4 >> (i >> 1)) & 1) {
            if (!q4p[i]) return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: 4-bit cache without its (min, step)");
            if (reinterpret_cast<uintptr_t>(q4p[i]) & 3)
                return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: (min, step) must be 4-byte aligned");
        }
    if (a->reserved2 != 0 || a->reserved3 != 0)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: reserved2 / reserved3 must be 0");
    if (a->split_part < 0 || a->split_part > 2)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: split_part = %d (0, 1 or 2)", a->split_part);
    if (a->rope_q != 0 && a->rope_q != 1)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: rope_q = %d (0 or 1)", a->rope_q);
    if (a->rope_q &&
        (a->rope_dim < 2 || a->rope_dim % 2 || a->rope_off < 0 || a->rope_off % 2 ||
         (long long)a->rope_off + a->rope_dim > a->d || !(a->rope_base > 0.0) || !std::isfinite(a->rope_base)))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: RoPE of q needs even rope_off / rope_dim inside d and a "
                    "finite base > 0 (got off %d, dim %d, base %g)", a->rope_off, a->rope_dim, a->rope_base);
    AttnParams& p = pl.p;
    p = AttnParams{};
    pl.launch_main = pl.combine = false;
    p.B = a->B;
    p.Tq = a->Tq;
    p.H = a->H;
    p.Hkv = a->Hkv;
    p.G = G;
    p.W = a->W;
    p.Tr = a->Tr;
    pl.ws_bytes = 0;
    pl.grid = 0;
    if (a->B == 0 || a->Tq == 0) return SHATTN_OK;
    if (!a->q || !a->out || !a->k_raw || !a->v_raw || !a->gates)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: null q/out/k_raw/v_raw/gates");
    if (!aligned16(a->q) || !aligned16(a->out) || !aligned16(a->k_raw) || !aligned16(a->v_raw) ||
        (has_hca && (!aligned16(a->k_hca) || !aligned16(a->v_hca))) ||
        (has_csa && (!aligned16(a->k_csa) || !aligned16(a->v_csa) || (reinterpret_cast<uintptr_t>(a->idx) & 3))))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: tensors must be 16-byte aligned");
    // every window row the queries need must be present
    if (a->raw_ring) {
        // a ring of Tr rows holds the last Tr positions: the W + Tq - 1
        // positions the rows' windows span must fit
        if ((long long)a->Tr < (long long)a->W + a->Tq - 1)
            return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: ring of %d rows cannot hold the W + Tq - 1 = %lld "
                        "window positions", a->Tr, (long long)a->W + a->Tq - 1);
    } else {
        const long long lo_need = a->q_pos0 - a->W + 1 > 0 ? a->q_pos0 - a->W + 1 : 0;
        const long long hi_need = a->q_pos0 + a->Tq;  // exclusive
        if (lo_need < a->raw_pos0 || hi_need > a->raw_pos0 + a->Tr)
            return fail(SHATTN_EINVAL,
                        "hybrid_sparse_attn_fwd: window rows [%lld, %lld) not inside raw rows [%lld, %lld)",
                        lo_need, hi_need, (long long)a->raw_pos0, (long long)a->raw_pos0 + a->Tr);
    }
    p.q = a->q;
    p.out = a->out;
    p.k_raw = a->k_raw;
    p.v_raw = a->v_raw;
    p.k_hca = has_hca ? a->k_hca : nullptr;
    p.v_hca = has_hca ? a->v_hca : nullptr;
    p.k_csa = has_csa ? a->k_csa : nullptr;
    p.v_csa = has_csa ? a->v_csa : nullptr;
    p.idx = has_csa ? a->idx : nullptr;
    p.gates = a->gates;
    p.gate_mode = a->gate_mode;
    p.q_pos0 = a->q_pos0;
    p.raw_pos0 = a->raw_pos0;
    p.q_pos = a->q_pos;
    p.ring = a->raw_ring;
    p.has_hca = has_hca;
    p.has_csa = has_csa;
    p.m_hca = has_hca ? a->m_hca : 1;
    p.N_hca = has_hca ? a->N_hca : 0;
    p.N_csa = has_csa ? a->N_csa : 0;
    p.k = has_csa ? a->k : 0;
    p.q4 = q4;
    p.rope_q = a->rope_q;
    p.rope_off = a->rope_q ? a->rope_off : 0;
    p.rope_dim = a->rope_q ? a->rope_dim : 0;
    p.rope_step = a->rope_q ? 2.0 * std::log2(a->rope_base) / a->rope_dim : 0.0;
    for (int i = 0; i < 4; ++i) p.q4p[i] = ((q4 >> (i >> 1)) & 1) ? q4p[i] : nullptr;
    const float scale = a->sm_scale > 0.f ? a->sm_scale : 1.0f / std::sqrt((float)a->d);
    p.scale_log2 = scale * 1.4426950408889634f;
    // 4 waves (64 (query, head) columns) per workgroup, one per SIMD: three
    // workgroups share a CU, so one computes while the others wait at a
    // barrier or on their loads.  (Measured: 8 waves leave one workgroup per
    // CU; 6 waves put two waves of a workgroup on some SIMDs, and every tile
    // barrier then waits for those.)
    // Few columns per (batch, KV head) -- decode: one query times G heads --
    // take two waves, so that no wave attends only padding columns.
    pl.waves = (G <= 32 && (long long)a->Tq * G <= 32) ? 2 : 4;
    p.ncol = pl.waves * 16;
    p.QW = G >= p.ncol ? 1 : p.ncol / G;
    if (G > p.ncol) return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_fwd: H/Hkv=%d too large", G);
    p.nqt = (a->Tq + p.QW - 1) / p.QW;

    const long long nwg = (long long)a->B * a->Hkv * p.nqt;
    // split the key list when there are too few workgroups to fill the chip
    long long keys = (long long)a->W;
    long long nh_max = 0;
    // (per-sequence positions live on the device: every entry may be visible)
    if (has_hca) nh_max = a->q_pos ? a->N_hca : n_visible_host(a->q_pos0 + a->Tq - 1, a->W, a->m_hca, a->N_hca);
    keys += nh_max;
    if (has_csa) keys += a->k;
    p.nsplit = 0;
    if (nwg < 128 && keys > 1024) {
        // one split item per 256 streamed HCA keys and per 64 gathered CSA
        // entries: a gather of 32 rows costs about as much as 4 streamed tiles
        p.split_keys = 256;
        p.split_csa = 64;
        p.n_win_items = 1;
        p.n_hca_items = (int)((nh_max + p.split_keys - 1) / p.split_keys);
        const int n_csa_items = has_csa ? (a->k + p.split_csa - 1) / p.split_csa : 0;
        p.nsplit = p.n_win_items + p.n_hca_items + n_csa_items;
        pl.ws_bytes = (size_t)nwg * p.nsplit * p.ncol * (a->d + 4) * sizeof(float);
        // the items this call runs (split_part): all, the ones that do not
        // read idx (window, HCA), or the CSA ones (then the merge)
        p.item_lo = a->split_part == 2 ? p.n_win_items + p.n_hca_items : 0;
        p.item_n = a->split_part == 0 ? p.nsplit
                 : (a->split_part == 1 ? p.n_win_items + p.n_hca_items : n_csa_items);
        pl.grid = nwg * p.item_n;
        pl.combine = a->split_part != 1;
        pl.launch_main = p.item_n > 0;
    } else {
        // no split: the second call of a two-part call does it all
        pl.grid = a->split_part == 1 ? 0 : nwg;
        pl.combine = false;
        pl.launch_main = true;
    }

    const bool bf = a->dtype == SHATTN_DTYPE_BF16;
    const int esz = bf ? 2 : 4;
    const int kpad = bf ? a->d + 8 : a->d + 4;
    // two staged tiles (double buffer)
    // bf16: K and V [KT][d] unpadded (swizzled); fp32: padded K and V rows
    const size_t tile_b = bf ? (size_t)(2 * KT * a->d) * esz : (size_t)(2 * KT * kpad) * esz;
    const size_t shared_b = 2 * tile_b;
    // per-wave gather tiles: bf16 K and V [KC][d] (DMA-loaded, swizzled); fp32
    // padded K and V rows plus the row list
    // (bf16: then a two-slot ring of 256-byte entry lists)
    const size_t gather_b = bf ? (size_t)(2 * KC * a->d) * esz + 512 : (size_t)(2 * KC * kpad) * esz + KC * 8;
    p.csa_mode = CSA_NONE;
    size_t lds = shared_b;
    if (has_csa) {
        // dense-masked when the union of a tile's selections is likely dense
        const long long span_q = (long long)std::min(p.QW, a->Tq);
        const bool dense = p.nsplit == 0 && G < 8 && a->N_csa <= 4096 &&
                           span_q * a->k >= a->N_csa / 2 && a->k % 4 == 0 && aligned16(a->idx);
        if (dense) {
            p.csa_mode = CSA_DENSE;
            p.bm_words = (a->N_csa + 127) / 128 * 4;   // multiple of 4: rows clear as 16-byte units
            p.lds_bm = (int)shared_b;
            lds = shared_b + (size_t)p.QW * p.bm_words * 4;
        } else {
            p.csa_mode = CSA_GATHER;
            // the bf16 gather addresses a sequence's CSA rows with 32-bit offsets
            if (bf && !(q4 & 2) && (unsigned long long)a->N_csa * a->Hkv * a->d * esz >= (1ull << 32))
                return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_fwd: CSA cache of one sequence >= 4 GiB");
            p.lds_gather = 0;
            p.lds_gather_stride = (int)((gather_b + 15) / 16 * 16);
            lds = std::max(lds, (size_t)p.lds_gather_stride * pl.waves);
        }
    }
    if (q4) {
        // the four 256-entry decode tables (1 KiB each) after everything else
        p.lds_lut = (int)((lds + 15) / 16 * 16);
        lds = (size_t)p.lds_lut + 4 * 1024;
    }
    if (lds > 160 * 1024) return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_fwd: LDS budget exceeded");
    pl.lds = lds;
    return SHATTN_OK;
}

}  // namespace
}  // namespace shattn

using namespace shattn;

extern "C" size_t hybrid_sparse_attn_fwd_workspace_size(const shattn_fwd_args* a) {
    Plan pl;
    if (make_plan(a, pl) != SHATTN_OK) return 0;
    return pl.ws_bytes;
}

template <typename T, int D, int NW, bool GATHER, bool Q4>
static int launch_attn_nw(Plan& pl, hipStream_t s) {
    if (pl.lds > 64 * 1024) {
        // dynamic LDS beyond 64 KiB must be opted into per kernel
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel<T, D, NW, GATHER, Q4>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)pl.lds);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_fwd: %zu bytes of LDS not available: %s",
                        pl.lds, hipGetErrorString(e));
        }
    }
    if (pl.launch_main) {
        hipLaunchKernelGGL((attn_fwd_kernel<T, D, NW, GATHER, Q4>), dim3((unsigned)pl.grid), dim3(NW * 64), pl.lds,
                           s, pl.p);
        hipError_t le = hipGetLastError();
        if (le != hipSuccess)
            return fail(SHATTN_EHIP, "hybrid_sparse_attn_fwd: launch failed (grid %lld, block %d, lds %zu): %s",
                        pl.grid, NW * 64, pl.lds, hipGetErrorString(le));
    }
    if (!pl.p.nsplit || !pl.combine) return SHATTN_OK;
    const long long n = (long long)pl.p.B * pl.p.Hkv * pl.p.nqt * pl.p.ncol * (D / 4) * kCombineSub;
    hipLaunchKernelGGL((attn_combine_kernel<T, D>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       pl.p);
    return check_launch("hybrid_sparse_attn_fwd (combine)");
}

template <typename T, int D, bool Q4>
static int launch_attn_q(Plan& pl, hipStream_t s) {
    const bool gather = pl.p.csa_mode == CSA_GATHER;
    if (pl.waves == 2)
        return gather ? launch_attn_nw<T, D, 2, true, Q4>(pl, s) : launch_attn_nw<T, D, 2, false, Q4>(pl, s);
    return gather ? launch_attn_nw<T, D, 4, true, Q4>(pl, s) : launch_attn_nw<T, D, 4, false, Q4>(pl, s);
}

template <typename T, int D>
static int launch_attn(Plan& pl, hipStream_t s) {
    if constexpr (std::is_same<T, bf16_t>::value)
        if (pl.p.q4) return launch_attn_q<T, D, true>(pl, s);
    return launch_attn_q<T, D, false>(pl, s);
}

extern "C" int hybrid_sparse_attn_fwd(const shattn_fwd_args* a, void* ws, size_t ws_bytes, void* stream) {
    Plan pl;
    int rc = make_plan(a, pl);
    if (rc != SHATTN_OK) return rc;
    if (pl.grid == 0 && !(pl.p.nsplit && pl.combine)) return SHATTN_OK;
    if (pl.ws_bytes > 0) {
        if (!ws || ws_bytes < pl.ws_bytes)
            return fail(SHATTN_EWORKSPACE, "hybrid_sparse_attn_fwd: workspace of %zu bytes needed, %zu given",
                        pl.ws_bytes, ws ? ws_bytes : (size_t)0);
        if (!aligned16(ws)) return fail(SHATTN_EINVAL, "hybrid_sparse_attn_fwd: workspace must be 16-byte aligned");
        pl.p.ws = reinterpret_cast<float*>(ws);
    }
    if (pl.grid > 2147483647LL) return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_fwd: problem too large");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (a->dtype == SHATTN_DTYPE_BF16)
        return a->d == 128 ? launch_attn<bf16_t, 128>(pl, s) : launch_attn<bf16_t, 64>(pl, s);
    return a->d == 128 ? launch_attn<float, 128>(pl, s) : launch_attn<float, 64>(pl, s);
}

// ------------------------------------------------------------ no allocation
// The same launch for callers that cannot allocate a workspace: the split
// decode launch's partial states go to one file-scope device array per GPU
// (each GPU the library runs on holds its own copy until the process ends).
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // the array's device address on each GPU

// Device address of `scratch` on the current device, looked up once per
// device (the array's name is not a device address in host code).
int scratch_on_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(SHATTN_EHIP, "hybrid_sparse_attn_fwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_fwd_noalloc: device %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(SHATTN_EHIP, "hybrid_sparse_attn_fwd_noalloc: hipGetSymbolAddress: %s",
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SHATTN_OK;
}
}  // namespace

extern "C" int hybrid_sparse_attn_fwd_noalloc(const shattn_fwd_args* a, void* stream) {
    Plan pl;
    int rc = make_plan(a, pl);
    if (rc != SHATTN_OK) return rc;
    if (pl.grid == 0 && !(pl.p.nsplit && pl.combine)) return SHATTN_OK;
    if (pl.ws_bytes > kScratchBytes)
        return fail(SHATTN_EUNSUPPORTED,
                    "hybrid_sparse_attn_fwd_noalloc: these arguments need %zu bytes of scratch, the library holds %zu",
                    pl.ws_bytes, kScratchBytes);
    void* ws = nullptr;
    if (pl.ws_bytes > 0 && (rc = scratch_on_current_device(&ws)) != SHATTN_OK) return rc;
    // the split partial states are all written before the combine reads
    // them: nothing in the array needs clearing between calls
    return hybrid_sparse_attn_fwd(a, ws, pl.ws_bytes, stream);
}
