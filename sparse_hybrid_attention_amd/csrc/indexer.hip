// Lightning indexer + exact per-query top-k over the CSA entries on gfx950.
//
// Method ([V4-blog] "CSA": a lightning indexer scores the current query
// against the compressed entries and the Top-K most relevant are kept;
// [Tiny-R2] 3.2 importance_score / topk selection; [CS336] "Attention
// Alternatives": DSA's lightning indexer):
//     score(q, c) = sum_h w[q,h] * max(0, qI[q,h,:] . kI[c,:])
// keep the k_eff = min(k, #visible) visible entries ranked by
// (score descending, entry index ascending), output in ascending index.
//
// Design:
//  * Scores are a dense contraction: MFMA with rows = (query, head) pairs and
//    columns = 16 candidate entries per tile; the head sum (ReLU, w) happens in
//    registers (for Hi = 4 a lane's four accumulator rows are exactly the four
//    heads of one query).  Scores are never written to memory in prefill.
//  * Each wave owns QPW queries and streams their visible entries in index
//    order.  Per query an LDS buffer holds the candidates that can still be
//    in the top-k; a candidate enters when its float32 score is >= tau.  When a
//    buffer fills it is compacted (wave-level): an LDS radix select finds the
//    k-th key, and everything below (k-th score - 2 delta) is dropped, where
//    delta bounds |float32 score - exact score| for that query (MFMA
//    accumulation error bound from the norms of the operands).  Ballot /
//    popcount prefix sums keep every buffer in index order.
//  * Final decision (exact): with T the float32 k-th score, entries above
//    T + 2 delta are certainly selected, entries below T - 2 delta certainly
//    not; the few in between are re-scored in float64 (products of the
//    inputs are exact in float64) and ranked by (score desc, index asc).  The
//    selected set therefore equals the float64 evaluation of the formula.
//  * Decode (few query rows, long N): scoring is split over many workgroups,
//    each writes its float32 scores and a lower bound on the global k-th
//    score (its local ceil(k/chunks)-th score); a collect pass keeps the
//    entries that can reach the top-k into per-chunk lists, and one wave per
//    query runs the same buffer / exact-final logic over those lists.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"

namespace shattn {
namespace {

constexpr int WAVES = 4;
constexpr int TILE = 16;  // candidate entries per MFMA tile
constexpr int MAX_RT = 4; // row tiles per wave

struct IdxParams {
    const void* qI;
    const void* kI;
    const float* w;
    int32_t* idx;
    long long q_pos0;
    const int64_t* q_pos;  // per-sequence position of query row 0 (device [B]), or null: q_pos0 for all
    int B, Tq, N, k, m, W;
    int cap;   // candidate buffer entries per query
    int mcap;  // band list capacity
    int qpw;   // queries per wave
    int nqt;   // query tiles (of WAVES*qpw queries) per sequence
    int wave_stride;  // LDS bytes per wave (prefill), multiple of 16
    float err_c;  // delta = err_c * sum_h |w_h| ||q_h|| * max ||k||
    // split (decode) pipeline workspace
    float* scores;      // [rows, N] float32 scores
    float* chunk_lb;    // [rows, nchunks] chunk_k-th largest score of the chunk
    float* chunk_kmax;  // [rows, nchunks] max ||k||^2 over the chunk
    float* row_qn;      // [rows] sum_h |w_h| ||q_h||
    uint32_t* lists;    // [rows, nchunks, list_cap] keys
    int32_t* list_idx;  // [rows, nchunks, list_cap] entries
    int32_t* list_cnt;  // [rows, nchunks] (may exceed list_cap: then the
                        //  chunk is re-read from `scores`)
    int nchunks, chunk, list_cap, chunk_k;
    int stream_cap;     // split final: candidate buffer of the streaming fallback
    // long prefill pipeline workspace (rows = B * Tq); lists/list_idx/list_cnt
    // then hold one list of list_cap entries per row
    float* kmax_part;   // [B, kblk] max ||k||^2 over blocks of kKmaxBlock entries
    uint32_t* row_thr;  // [rows] entries whose key is >= row_thr enter the row's list
    uint32_t* row_tau;  // [rows] key of the sampled threshold (0: every visible entry is listed)
    float* row_delta;   // [rows] bound of |float32 score - exact score| for the row
    int32_t* row_fail;  // [rows] 1: the list cannot decide the row (the streaming kernel does)
    uint2* row_lists;   // [rows, list_cap] (float32 score bits, entry) pairs in entry order
    int kblk;           // entry blocks per sequence for kmax_part
    int sample_stride;  // sampled entries are 0, S, 2S, ... (S = sample_stride)
    int sample_j;       // the threshold is the sample_j-th largest sampled score
    int list_mcap;      // band list capacity of the list selection pass
    int list_lds_cap;   // list entries the list selection pass holds in LDS (<= list_cap)
};

// ----------------------------------------------------------- key encoding
// order-preserving map float32 -> uint32 (-0.0 and +0.0 share one key)
__device__ __forceinline__ uint32_t fkey(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_f(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ unsigned long long lanemask_lt() {
    const int l = __lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ long long n_visible(long long t, int W, int m, int N) {
    const long long s = t - W + 1;
    if (s <= 0) return 0;
    const long long n = s / m;
    return n < N ? n : N;
}

// Position of query row 0 of sequence b.  A negative per-sequence position
// (an inactive batch slot) gives every row of the sequence no visible entry,
// so its index rows are all -1.
__device__ __forceinline__ long long row_pos0(const IdxParams& p, long long b) {
    if (!p.q_pos) return p.q_pos0;
    const long long t = p.q_pos[b];
    return t < 0 ? -(1ll << 40) : t;
}

// ----------------------------------------------------------- wave selection
struct WaveBuf {
    uint32_t* keys;  // [cap]
    int32_t* ids;    // [cap] (unused when the entries come from an accessor)
    uint32_t* hist;  // [256]
    int32_t* mpos;   // [mcap] buffer positions of the band candidates
    double* mex;     // [mcap] their exact scores
    int32_t* mid;    // [mcap] their entries
};

// Entry of buffer position e: from an LDS array, from a (key, entry) list in
// global memory, or the position itself.  ids4(e0) gives the entries of the
// 4 positions e0 .. e0 + 3 (e0 a multiple of 4 inside the buffer's capacity).
struct LdsIds {
    const int32_t* ids;
    __device__ int operator()(int e) const { return ids[e]; }
    __device__ int4 ids4(int e0) const { return *reinterpret_cast<const int4*>(ids + e0); }
};
struct ListIds {
    const uint2* lst;
    __device__ int operator()(int e) const { return (int)lst[e].y; }
    __device__ int4 ids4(int e0) const {
        const uint4 a = ld16(lst + e0), b = ld16(lst + e0 + 2);
        return make_int4((int)a.y, (int)a.w, (int)b.y, (int)b.w);
    }
};
struct PosIds {
    __device__ int operator()(int e) const { return e; }
    __device__ int4 ids4(int e0) const { return make_int4(e0, e0 + 1, e0 + 2, e0 + 3); }
};
__device__ __forceinline__ int int4_at(const int4& v, int j) {
    return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// Buffers read by the selection passes below are 16-byte aligned and their
// capacity is a multiple of 4 keys: lane l of a pass over 256 keys takes the
// 4 consecutive keys 4l..4l+3 with one 16-byte LDS read (keys past `cnt` are
// read but ignored).
__device__ __forceinline__ uint4 keys4(const uint32_t* keys, int e0) {
    return *reinterpret_cast<const uint4*>(keys + e0);
}
__device__ __forceinline__ uint32_t key_at(const uint4& v, int j) {
    return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

// k-th largest key among keys[0..cnt), 1 <= kk <= cnt.  *n_gt = #keys > result.
// MSD radix select with digits of up to 8 bits taken from the highest bit in
// which the keys differ (the bits above it are common to all keys).  Invariant:
// kk - want keys lie above the current bucket (keys sharing `prefix` on
// `pmask`), and the result is the want-th largest key inside it.  When that is
// the bucket's largest (want == 1) or smallest (want == bucket size) key, one
// min/max scan ends the search.
__device__ __forceinline__ uint32_t radix_kth(const uint32_t* keys, int cnt, int kk, uint32_t* hist, int* n_gt) {
    const int lane = __lane_id();
    uint32_t andv = 0xFFFFFFFFu, orv = 0u;
    for (int base = 0; base < cnt; base += 256) {
        const int e0 = base + 4 * lane;
        if (e0 < cnt) {
            const uint4 v = keys4(keys, e0);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (e0 + j < cnt) {
                    andv &= key_at(v, j);
                    orv |= key_at(v, j);
                }
        }
    }
    andv = wave_allreduce(andv, [](uint32_t a, uint32_t b) { return a & b; });
    orv = wave_allreduce(orv, [](uint32_t a, uint32_t b) { return a | b; });
    const uint32_t diff = andv ^ orv;
    if (diff == 0u) {
        *n_gt = 0;
        return andv;
    }
    int shift = 32 - __clz(diff);   // bits [shift, 32) are common to all keys
    uint32_t pmask = shift >= 32 ? 0u : (0xFFFFFFFFu << shift);
    uint32_t prefix = andv & pmask;
    int want = kk;
    while (shift > 0) {
        const int width = min(8, shift);
        shift -= width;
        const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
        for (int j = 0; j < 4; ++j) hist[lane * 4 + j] = 0u;
        wave_lds_sync();
        for (int base = 0; base < cnt; base += 512) {
            const int e0 = base + 4 * lane, e1 = e0 + 256;
            uint4 v0 = make_uint4(0u, 0u, 0u, 0u), v1 = v0;
            if (e0 < cnt) v0 = keys4(keys, e0);
            if (e1 < cnt) v1 = keys4(keys, e1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = key_at(v0, j);
                if (e0 + j < cnt && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = key_at(v1, j);
                if (e1 + j < cnt && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
            }
        }
        wave_lds_sync();
        const uint32_t c0 = hist[lane * 4 + 0], c1 = hist[lane * 4 + 1];
        const uint32_t c2 = hist[lane * 4 + 2], c3 = hist[lane * 4 + 3];
        const int mine = (int)(c0 + c1 + c2 + c3);
        const int incl = wave_incl_scan(mine);                      // sum over lanes <= this lane
        const int total = __builtin_amdgcn_readlane(incl, 63);
        const int suf = total - incl + mine;                        // sum over lanes >= this lane
        const int above = suf - mine;  // sum over bins of higher lanes
        int bin = -1, cnt_above = 0, cnt_bin = 0;
        if (above < want && want <= suf) {
            int acc = above;
            if (acc + (int)c3 >= want) { bin = lane * 4 + 3; cnt_above = acc; cnt_bin = (int)c3; }
            else {
                acc += c3;
                if (acc + (int)c2 >= want) { bin = lane * 4 + 2; cnt_above = acc; cnt_bin = (int)c2; }
                else {
                    acc += c2;
                    if (acc + (int)c1 >= want) { bin = lane * 4 + 1; cnt_above = acc; cnt_bin = (int)c1; }
                    else { acc += c1; bin = lane * 4 + 0; cnt_above = acc; cnt_bin = (int)c0; }
                }
            }
        }
        const unsigned long long who = __ballot(bin >= 0);
        const int src = __ffsll((long long)who) - 1;
        const int b = __builtin_amdgcn_readlane(bin, src);
        const int ca = __builtin_amdgcn_readlane(cnt_above, src);
        const int cb = __builtin_amdgcn_readlane(cnt_bin, src);
        prefix |= ((uint32_t)b) << shift;
        pmask |= dmask << shift;
        want -= ca;
        wave_lds_sync();
        if (shift > 0 && (want == 1 || want == cb)) {
            const bool top = want == 1;
            uint32_t m = top ? 0u : 0xFFFFFFFFu;
            for (int base = 0; base < cnt; base += 256) {
                const int e0 = base + 4 * lane;
                if (e0 < cnt) {
                    const uint4 v = keys4(keys, e0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t key = key_at(v, j);
                        if (e0 + j < cnt && (key & pmask) == prefix) m = top ? max(m, key) : min(m, key);
                    }
                }
            }
            m = top ? wave_allreduce(m, [](uint32_t x, uint32_t y) { return max(x, y); })
                    : wave_allreduce(m, [](uint32_t x, uint32_t y) { return min(x, y); });
            if (top) {
                *n_gt = kk - 1;
                return m;
            }
            int eq = 0;
            for (int base = 0; base < cnt; base += 256) {
                const int e0 = base + 4 * lane;
                if (e0 < cnt) {
                    const uint4 v = keys4(keys, e0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) eq += (e0 + j < cnt && key_at(v, j) == m) ? 1 : 0;
                }
            }
            *n_gt = kk - (int)wave_allreduce((uint32_t)eq, [](uint32_t x, uint32_t y) { return x + y; });
            return m;
        }
    }
    *n_gt = kk - want;
    return prefix;
}

// k-th largest (1 <= kk <= cnt) of the 16-bit keys keys[0..cnt): two passes of
// 8-bit digits.  keys is 16-byte aligned and readable up to cnt rounded up to
// a multiple of 8.
__device__ __forceinline__ uint32_t radix_kth16(const uint16_t* keys, int cnt, int kk, uint32_t* hist) {
    const int lane = __lane_id();
    uint32_t prefix = 0u;
    int want = kk;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = pass == 0 ? 8 : 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) hist[lane * 4 + j] = 0u;
        wave_lds_sync();
        for (int e0 = 8 * lane; e0 < cnt; e0 += 512) {
            const uint4 v = *reinterpret_cast<const uint4*>(keys + e0);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t key = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
                if (e0 + j < cnt && (pass == 0 || (key >> 8) == prefix)) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
        }
        wave_lds_sync();
        // the bin holding the want-th largest key, bins scanned from the top
        const uint32_t c0 = hist[lane * 4 + 0], c1 = hist[lane * 4 + 1];
        const uint32_t c2 = hist[lane * 4 + 2], c3 = hist[lane * 4 + 3];
        const int mine = (int)(c0 + c1 + c2 + c3);
        const int incl = wave_incl_scan(mine);
        const int total = __builtin_amdgcn_readlane(incl, 63);
        const int suf = total - incl + mine;   // bins of this lane and above
        const int above = suf - mine;
        int bin = -1, cnt_above = 0;
        if (above < want && want <= suf) {
            int acc = above;
            if (acc + (int)c3 >= want) { bin = lane * 4 + 3; cnt_above = acc; }
            else {
                acc += c3;
                if (acc + (int)c2 >= want) { bin = lane * 4 + 2; cnt_above = acc; }
                else {
                    acc += c2;
                    if (acc + (int)c1 >= want) { bin = lane * 4 + 1; cnt_above = acc; }
                    else { acc += c1; bin = lane * 4 + 0; cnt_above = acc; }
                }
            }
        }
        const unsigned long long who = __ballot(bin >= 0);
        const int src = __ffsll((long long)who) - 1;
        prefix = pass == 0 ? (uint32_t)__builtin_amdgcn_readlane(bin, src)
                           : (prefix << 8) | (uint32_t)__builtin_amdgcn_readlane(bin, src);
        want -= __builtin_amdgcn_readlane(cnt_above, src);
        wave_lds_sync();
    }
    return prefix;
}

// Stable in-place compaction: keep entries with key >= lo.  Returns new count.
__device__ __noinline__ int compact_ge(uint32_t* keys, int32_t* ids, int cnt, uint32_t lo) {
    const int lane = __lane_id();
    int out = 0;
    for (int base = 0; base < cnt; base += 64) {
        const int e = base + lane;
        uint32_t key = 0u;
        int32_t id = 0;
        bool keep = false;
        if (e < cnt) {
            key = keys[e];
            id = ids[e];
            keep = key >= lo;
        }
        const unsigned long long msk = __ballot(keep);
        wave_lds_sync();
        if (keep) {
            const int pos = out + __popcll(msk & lanemask_lt());
            keys[pos] = key;
            ids[pos] = id;
        }
        out += __popcll(msk);
        wave_lds_sync();
    }
    return out;
}

// Stable: keep entries with key > kth and the first `need` entries with key == kth.
__device__ __noinline__ int compact_topk(uint32_t* keys, int32_t* ids, int cnt, uint32_t kth, int need) {
    const int lane = __lane_id();
    int out = 0, eq_seen = 0;
    for (int base = 0; base < cnt; base += 64) {
        const int e = base + lane;
        uint32_t key = 0u;
        int32_t id = 0;
        bool gt = false, eq = false;
        if (e < cnt) {
            key = keys[e];
            id = ids[e];
            gt = key > kth;
            eq = key == kth;
        }
        const unsigned long long meq = __ballot(eq);
        const bool keep = gt || (eq && eq_seen + __popcll(meq & lanemask_lt()) < need);
        const unsigned long long msk = __ballot(keep);
        wave_lds_sync();
        if (keep) {
            const int pos = out + __popcll(msk & lanemask_lt());
            keys[pos] = key;
            ids[pos] = id;
        }
        out += __popcll(msk);
        eq_seen += __popcll(meq);
        wave_lds_sync();
    }
    return out;
}

// Streaming compaction of a full buffer.  Returns the new count; *tau_key is the
// new insertion threshold (keys >= tau_key may enter).
__device__ __noinline__ int compact_stream(WaveBuf& wb, int cnt, int kk, float delta, int cap, int slack,
                              uint32_t* tau_key) {
    int n_gt;
    const uint32_t kth = radix_kth(wb.keys, cnt, kk, wb.hist, &n_gt);
    const float T = key_f(kth);
    const uint32_t lo = fkey(T - 2.0f * delta);
    int n = compact_ge(wb.keys, wb.ids, cnt, lo);
    if (n > cap - slack) {
        // more near-ties than the buffer holds: fall back to the float32 order
        n = compact_topk(wb.keys, wb.ids, n, kth, kk - n_gt);
        *tau_key = kth == 0xFFFFFFFFu ? kth : kth + 1u;
        return n;
    }
    *tau_key = lo;
    return n;
}

// Exact (float64) scores of the band candidates, 4 per pass (candidate j is
// entry ids(mpos[j])): 16 lanes per candidate, each holding DI/16 dims of the
// query's HI heads and of the candidate's key; products of the inputs are
// exact in float64 and the 16 partial dot products are combined in a fixed
// order.  mex[j] = exact score, mid[j] = entry (when mid is not null).
template <typename T, int HI, int DI, class Ids>
__device__ void exact_scores(const T* __restrict__ qrow /* [HI][DI] */, const T* __restrict__ kI_b,
                             const float* __restrict__ wrow, Ids ids, const int32_t* mpos, int nM, double* mex,
                             int32_t* mid) {
    constexpr int PER = DI / 16;  // dims per lane (4 or 8)
    const int lane = __lane_id();
    const int slot = lane >> 4, dl = lane & 15;
    float q[HI][PER];
#pragma unroll
    for (int h = 0; h < HI; ++h)
#pragma unroll
        for (int u = 0; u < PER; ++u) q[h][u] = Elem<T>::load1(qrow + h * DI + dl * PER + u);
    for (int j0 = 0; j0 < nM; j0 += 4) {
        const int j = j0 + slot;
        const bool ok = j < nM;
        const int c = ok ? ids(mpos[j]) : 0;
        float kv[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) kv[u] = Elem<T>::load1(kI_b + (long long)c * DI + dl * PER + u);
        double s = 0.0;
#pragma unroll
        for (int h = 0; h < HI; ++h) {
            double d = 0.0;
#pragma unroll
            for (int u = 0; u < PER; ++u) d += (double)q[h][u] * (double)kv[u];
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                const double o = __shfl_xor(d, off);
                d = (dl & off) ? o + d : d + o;
            }
            s += (double)wrow[h] * (d > 0.0 ? d : 0.0);
        }
        if (ok && dl == 0) {
            mex[j] = s;
            if (mid) mid[j] = c;
        }
    }
}

// Final exact selection of one query over its candidate buffer (in ascending
// entry order) and output of its idx row: the kept entries are written in
// buffer order, then -1 up to k.
template <typename T, int HI, int DI, class Ids>
__device__ __forceinline__ void final_select(WaveBuf& wb, Ids ids, int cnt, int k_eff, int k, float delta, int mcap,
                             const T* __restrict__ qrow, const T* __restrict__ kI_b,
                             const float* __restrict__ wrow, int32_t* __restrict__ out_row) {
    const int lane = __lane_id();
    // kept: key >= keep_ge; in the float32 fallback, key > kth plus the first
    // eq_need entries with key == kth
    uint32_t keep_ge = 0u, kth = 0u;
    int eq_need = -1;
    if (cnt > k_eff) {
        int n_gt;
        kth = radix_kth(wb.keys, cnt, k_eff, wb.hist, &n_gt);
        const float Tf = key_f(kth);
        const uint32_t hi = fkey(Tf + 2.0f * delta);
        const uint32_t lo = fkey(Tf - 2.0f * delta);
        // D = key > hi (certain), M = lo <= key <= hi (band); the order of
        // the band list does not matter
        int nD = 0, nM = 0;
        for (int base = 0; base < cnt; base += 256) {
            const int e0 = base + 4 * lane;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (e0 < cnt) v = keys4(wb.keys, e0);
            int cm = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = key_at(v, j);
                nD += e0 + j < cnt && key > hi;
                cm += e0 + j < cnt && key >= lo && key <= hi;
            }
            const int incl = wave_incl_scan(cm);
            int pos = nM + incl - cm;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = key_at(v, j);
                if (e0 + j < cnt && key >= lo && key <= hi) {
                    if (pos < mcap) wb.mpos[pos] = e0 + j;
                    ++pos;
                }
            }
            nM += __builtin_amdgcn_readlane(incl, 63);
        }
        nD = (int)wave_allreduce((uint32_t)nD, [](uint32_t x, uint32_t y) { return x + y; });
        wave_lds_sync();
        const int need = k_eff - nD;
        if (nM <= mcap) {
            // a band of exactly `need` entries is kept whole: no re-scoring
            if (nM > need) {
                exact_scores<T, HI, DI>(qrow, kI_b, wrow, ids, wb.mpos, nM, wb.mex, wb.mid);
                wave_lds_sync();
            }
            // rank within M by (exact desc, index asc); keep the first `need`
            // (with positions as entries, the band list itself holds them)
            const int32_t* rid = std::is_same<Ids, PosIds>::value ? wb.mpos : wb.mid;
            for (int j = lane; j < nM; j += 64) {
                int rank = 0;
                if (nM > need) {
                    const double ex = wb.mex[j];
                    const int id = rid[j];
                    for (int y = 0; y < nM; ++y) {
                        const double ey = wb.mex[y];
                        rank += (ey > ex) || (ey == ex && rid[y] < id);
                    }
                }
                wb.keys[wb.mpos[j]] = rank < need ? 0xFFFFFFFFu : 0u;
            }
            wave_lds_sync();
            keep_ge = hi == 0xFFFFFFFFu ? hi : hi + 1u;
        } else {
            // more entries in the error band than the band list holds: decide
            // on float32 scores (index tie-break)
            eq_need = k_eff - n_gt;
        }
    }
    // kept entries in buffer order: lane l holds 4 consecutive positions, so
    // a prefix sum over lanes orders them; the entries of the next 256
    // positions are fetched while these are placed
    int out = 0, eq_seen = 0;
    int4 idn = make_int4(0, 0, 0, 0);
    if (4 * lane < cnt) idn = ids.ids4(4 * lane);
    for (int base = 0; base < cnt; base += 256) {
        const int e0 = base + 4 * lane;
        const int4 idc = idn;
        if (e0 + 256 < cnt) idn = ids.ids4(e0 + 256);
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (e0 < cnt) v = keys4(wb.keys, e0);
        int keepm = 0;
        if (eq_need < 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) keepm |= (e0 + j < cnt && key_at(v, j) >= keep_ge) << j;
        } else {
            int ce = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) ce += e0 + j < cnt && key_at(v, j) == kth;
            const int ie = wave_incl_scan(ce);
            int eq_rank = eq_seen + ie - ce;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t key = key_at(v, j);
                const bool valid = e0 + j < cnt;
                bool kp = valid && key > kth;
                if (valid && key == kth) kp = eq_rank++ < eq_need;
                keepm |= kp << j;
            }
            eq_seen += __builtin_amdgcn_readlane(ie, 63);
        }
        const int ck = __popc(keepm);
        const int incl = wave_incl_scan(ck);
        int pos = out + incl - ck;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (keepm & (1 << j)) out_row[pos++] = int4_at(idc, j);
        out += __builtin_amdgcn_readlane(incl, 63);
    }
    for (int j = out + lane; j < k; j += 64) out_row[j] = -1;
    wave_lds_sync();
}

// ----------------------------------------------------------- MFMA scoring
template <typename T, int DI> struct IdxMma;
template <int DI> struct IdxMma<bf16_t, DI> {
    static constexpr int KS = DI / 32;
    typedef bf16x8_t F;
    __device__ static void load_a(const bf16_t* row, bool ok, int q4, F* a) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ok) a[ks] = *reinterpret_cast<const bf16x8_t*>(row + 32 * ks + 8 * q4);
            else {
#pragma unroll
                for (int j = 0; j < 8; ++j) a[ks][j] = (__bf16)0.0f;
            }
        }
    }
    // partial squared norm of this lane's slice
    __device__ static float sq(const F* a) {
        float s = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float x = (float)a[ks][j];
                s = fmaf(x, x, s);
            }
        return s;
    }
    __device__ static f32x4_t mma(const F* a, const F* b) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], b[ks], c, 0, 0, 0);
        return c;
    }
};
template <int DI> struct IdxMma<float, DI> {
    static constexpr int KS = DI / 4;
    typedef float F;
    __device__ static void load_a(const float* row, bool ok, int q4, F* a) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = ok ? row[4 * ks + q4] : 0.f;
    }
    __device__ static float sq(const F* a) {
        float s = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = fmaf(a[ks], a[ks], s);
        return s;
    }
    __device__ static f32x4_t mma(const F* a, const F* b) {
        f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[ks], b[ks], c, 0, 0, 0);
        return c;
    }
};

// max(x, 0) as one integer max: every negative float32 (-0.0 included) is a
// negative int32, every other one keeps its bits.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Scores of the lane's query slots from one 16-row accumulator tile.
// Returns the number of slots; s[j], qs[j] = query index within the tile, own[j].
template <int HI>
__device__ __forceinline__ int tile_scores(const f32x4_t& c, const float* wr, int q4, float* s, int* qs,
                                           bool* own) {
    if constexpr (HI == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = wr[r] * relu(c[r]);
            qs[r] = 4 * q4 + r;
            own[r] = true;
        }
        return 4;
    } else if constexpr (HI == 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            s[j] = wr[2 * j] * relu(c[2 * j]) + wr[2 * j + 1] * relu(c[2 * j + 1]);
            qs[j] = 2 * q4 + j;
            own[j] = true;
        }
        return 2;
    } else {
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) part += wr[r] * relu(c[r]);
        if constexpr (HI == 4) {
            s[0] = part;
            qs[0] = q4;
            own[0] = true;
        } else if constexpr (HI == 8) {
            uint32_t lo, hi;
            xor16_pair(__float_as_uint(part), lo, hi);
            s[0] = __uint_as_float(lo) + __uint_as_float(hi);   // (row 2r) + (row 2r+1)
            qs[0] = q4 >> 1;
            own[0] = (q4 & 1) == 0;
        } else {
            const int base = __lane_id() & 15;
            const float p0 = __shfl(part, base), p1 = __shfl(part, base + 16);
            const float p2 = __shfl(part, base + 32), p3 = __shfl(part, base + 48);
            s[0] = (p0 + p1) + (p2 + p3);
            qs[0] = 0;
            own[0] = q4 == 0;
        }
        return 1;
    }
}

// ----------------------------------------------------------- prefill kernel
template <typename T, int HI, int DI>
__global__ __launch_bounds__(WAVES * 64) void index_prefill_kernel(IdxParams p) {
    typedef IdxMma<T, DI> MM;
    constexpr int QPT = 16 / HI;  // queries per row tile
    constexpr int SLOTS = HI == 1 ? 4 : (HI == 2 ? 2 : 1);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q4 = lane >> 4;
    const int qpw = p.qpw, cap = p.cap, mcap = p.mcap;
    const int RT = qpw / QPT;

    // per-wave LDS: keys[qpw][cap] ids[qpw][cap] hist[256] mex[mcap] mpos[mcap] mid[mcap] qn[qpw]
    char* base = smem + (size_t)wave * p.wave_stride;
    uint32_t* keys_all = reinterpret_cast<uint32_t*>(base);
    int32_t* ids_all = reinterpret_cast<int32_t*>(base + 4ull * qpw * cap);
    WaveBuf wb;
    wb.hist = reinterpret_cast<uint32_t*>(base + 8ull * qpw * cap);
    wb.mex = reinterpret_cast<double*>(base + 8ull * qpw * cap + 1024);
    wb.mpos = reinterpret_cast<int32_t*>(base + 8ull * qpw * cap + 1024 + 8ull * mcap);
    wb.mid = reinterpret_cast<int32_t*>(base + 8ull * qpw * cap + 1024 + 12ull * mcap);
    float* qn = reinterpret_cast<float*>(base + 8ull * qpw * cap + 1024 + 16ull * mcap);

    // later queries (more visible entries) first: the light work runs last
    const int qt = p.nqt - 1 - (int)(blockIdx.x % p.nqt);
    const int b = blockIdx.x / p.nqt;
    const int q0 = (qt * WAVES + wave) * qpw;  // first query row of this wave
    const T* qI = reinterpret_cast<const T*>(p.qI);
    const T* kI_b = reinterpret_cast<const T*>(p.kI) + (long long)b * p.N * DI;
    if (p.row_fail) {
        // fallback of the long prefill pipeline: only rows its lists could not
        // decide are (re)computed; a wave without such a row has nothing to do
        bool any = false;
        for (int qw = lane; qw < qpw; qw += 64) {
            const int i = q0 + qw;
            any |= i < p.Tq && p.row_fail[(long long)b * p.Tq + i] != 0;
        }
        if (!__any(any)) return;
    }

    // ---- A fragments (rows = (query, head)), weights, norms
    typename MM::F a[MAX_RT][MM::KS];
    float wr[MAX_RT][4];
    const int rho = lane & 15;
#pragma unroll
    for (int rt = 0; rt < MAX_RT; ++rt) {
        const int qw = rt * QPT + rho / HI, hh = rho % HI;
        const int i = q0 + qw;
        const bool ok = rt < RT && qw < qpw && i < p.Tq;
        MM::load_a(qI + (((long long)b * p.Tq + (ok ? i : 0)) * HI + hh) * DI, ok, q4, a[rt]);
        // weights of this lane's accumulator rows 4*q4 + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * q4 + r;
            const int qr = rt * QPT + row / HI, hr = row % HI;
            const int ir = q0 + qr;
            wr[rt][r] = (rt < RT && qr < qpw && ir < p.Tq) ? p.w[((long long)b * p.Tq + ir) * HI + hr] : 0.f;
        }
        // sum_h |w_h| ||q_h|| per query (row norms combined in fixed head order)
        float n2 = MM::sq(a[rt]);
        n2 = sum_xrows(n2);
        if (rt < RT) {
            // lane rho (q4 == 0) holds ||row rho||^2; gather the HI rows of each query
            const int qsl = lane < QPT ? lane : 0;  // lane j < QPT finishes query slot j
            float acc = 0.f;
            for (int h = 0; h < HI; ++h) {
                const float nr = __shfl(n2, qsl * HI + h);
                const int ir = q0 + rt * QPT + qsl;
                const float wv = (ir < p.Tq && rt * QPT + qsl < qpw)
                                     ? p.w[((long long)b * p.Tq + ir) * HI + h] : 0.f;
                acc += fabsf(wv) * sqrtf(nr);
            }
            if (lane < QPT && rt * QPT + lane < qpw) qn[rt * QPT + lane] = acc;
        }
    }

    // ---- per (row tile, slot) state of the lane's queries
    int cnt[MAX_RT][SLOTS];
    uint32_t tau[MAX_RT][SLOTS];
    int nv[MAX_RT][SLOTS];
    int nv_max = 0;
#pragma unroll
    for (int rt = 0; rt < MAX_RT; ++rt)
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
            cnt[rt][sl] = 0;
            tau[rt][sl] = 0u;
            int qw;
            if (HI == 1) qw = 4 * q4 + sl;
            else if (HI == 2) qw = 2 * q4 + sl;
            else if (HI == 4) qw = q4;
            else if (HI == 8) qw = q4 >> 1;
            else qw = 0;
            qw += rt * QPT;
            const int i = q0 + qw;
            const bool ok = rt < RT && sl < SLOTS && qw < qpw && i < p.Tq;
            nv[rt][sl] = ok ? (int)n_visible(row_pos0(p, b) + i, p.W, p.m, p.N) : 0;
            nv_max = nv[rt][sl] > nv_max ? nv[rt][sl] : nv_max;
        }
    // wave-wide maximum of visible entries
    for (int off = 32; off > 0; off >>= 1) {
        const int o = __shfl_xor(nv_max, off);
        nv_max = o > nv_max ? o : nv_max;
    }
    float kmax2 = 0.f;
    wave_lds_sync();

    // ---- stream the candidates in index order; B fragments of the next PF
    // tiles are loaded while the current PF tiles are scored
    auto load_b = [&](long long c0, typename MM::F* bf) {
        const long long c = c0 + rho;
        MM::load_a(kI_b + (c < p.N ? c : 0) * DI, c < p.N, q4, bf);
    };
    auto process_tile = [&](long long c0, const typename MM::F* bf) {
        const long long c = c0 + rho;
        float n2 = MM::sq(bf);
        n2 = sum_xrows(n2);
        kmax2 = fmaxf(kmax2, n2);
#pragma unroll
        for (int rt = 0; rt < MAX_RT; ++rt) {
            if (rt >= RT) break;
            const f32x4_t acc = MM::mma(a[rt], bf);
            float s[4];
            int qs[4];
            bool own[4];
            const int ns = tile_scores<HI>(acc, wr[rt], q4, s, qs, own);
#pragma unroll
            for (int sl = 0; sl < SLOTS; ++sl) {
                if (sl >= ns) break;
                const uint32_t key = fkey(s[sl]);
                const bool ins = own[sl] && c < nv[rt][sl] && key >= tau[rt][sl];
                const unsigned long long msk = __ballot(ins);
                const unsigned long long gm = msk & (0xFFFFull << (16 * q4));
                const int qw = rt * QPT + qs[sl];
                if (ins) {
                    const int pos = cnt[rt][sl] + __popcll(gm & lanemask_lt());
                    keys_all[qw * cap + pos] = key;
                    ids_all[qw * cap + pos] = (int32_t)c;
                }
                cnt[rt][sl] += __popcll(gm);
            }
        }
        // compaction of full buffers
#pragma unroll
        for (int rt = 0; rt < MAX_RT; ++rt) {
            if (rt >= RT) break;
#pragma unroll
            for (int sl = 0; sl < SLOTS; ++sl) {
                int qw_l;
                if (HI == 1) qw_l = 4 * q4 + sl;
                else if (HI == 2) qw_l = 2 * q4 + sl;
                else if (HI == 4) qw_l = q4;
                else if (HI == 8) qw_l = q4 >> 1;
                else qw_l = 0;
                const bool owner = (HI <= 4) || (HI == 8 ? (q4 & 1) == 0 : q4 == 0);
                const bool full = owner && cnt[rt][sl] > cap - TILE;
                unsigned long long fm = __ballot(full);
                if (fm == 0ull) continue;
                wave_lds_sync();
                const float delta = p.err_c * sqrtf(kmax2);
                for (int g4 = 0; g4 < 4; ++g4) {
                    if (((fm >> (16 * g4)) & 0xFFFFull) == 0ull) continue;
                    const int src = 16 * g4;
                    const int qw = rt * QPT + __builtin_amdgcn_readlane(qw_l, src);
                    const int cq = __builtin_amdgcn_readlane(cnt[rt][sl], src);
                    const int nvq = __builtin_amdgcn_readlane(nv[rt][sl], src);
                    WaveBuf q = wb;
                    q.keys = keys_all + qw * cap;
                    q.ids = ids_all + qw * cap;
                    const int kk = min(p.k, nvq);
                    uint32_t tk;
                    const int nc = compact_stream(q, cq, kk, delta * qn[qw], cap, TILE, &tk);
                    if (q4 == g4) {
                        cnt[rt][sl] = nc;
                        tau[rt][sl] = tk;
                    }
                }
            }
        }
    };
    constexpr int PF = 2;
    typename MM::F bq0[PF][MM::KS], bq1[PF][MM::KS];
    auto group = [&](long long g0, typename MM::F (&cur)[PF][MM::KS], typename MM::F (&nxt)[PF][MM::KS]) {
        const long long g1 = g0 + PF * TILE;
        if (g1 < nv_max) {
#pragma unroll
            for (int t = 0; t < PF; ++t) load_b(g1 + t * TILE, nxt[t]);
        }
#pragma unroll
        for (int t = 0; t < PF; ++t)
            if (g0 + t * TILE < nv_max) process_tile(g0 + t * TILE, cur[t]);
    };
    if (nv_max > 0) {
#pragma unroll
        for (int t = 0; t < PF; ++t) load_b(t * TILE, bq0[t]);
    }
    for (long long g0 = 0; g0 < nv_max; g0 += 2 * PF * TILE) {
        group(g0, bq0, bq1);
        if (g0 + PF * TILE < nv_max) group(g0 + PF * TILE, bq1, bq0);
    }

    // ---- final exact selection per query, output
    const float delta0 = p.err_c * sqrtf(kmax2);
#pragma unroll
    for (int rt = 0; rt < MAX_RT; ++rt) {
        if (rt >= RT) break;
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
            for (int g4 = 0; g4 < 4; ++g4) {
                if (HI == 8 && (g4 & 1)) continue;
                if (HI == 16 && g4 != 0) continue;
                int qw_l;
                if (HI == 1) qw_l = 4 * g4 + sl;
                else if (HI == 2) qw_l = 2 * g4 + sl;
                else if (HI == 4) qw_l = g4;
                else if (HI == 8) qw_l = g4 >> 1;
                else qw_l = 0;
                const int qw = rt * QPT + qw_l;
                const int i = q0 + qw;
                if (qw >= qpw || i >= p.Tq) continue;
                const int src = 16 * g4;
                const int cq = __builtin_amdgcn_readlane(cnt[rt][sl], src);
                const int nvq = __builtin_amdgcn_readlane(nv[rt][sl], src);
                WaveBuf q = wb;
                q.keys = keys_all + qw * cap;
                q.ids = ids_all + qw * cap;
                const int k_eff = min(p.k, nvq);
                const long long row = (long long)b * p.Tq + i;
                if (p.row_fail && p.row_fail[row] == 0) continue;
                final_select<T, HI, DI>(q, LdsIds{q.ids}, cq, k_eff, p.k, delta0 * qn[qw], mcap, qI + row * HI * DI, kI_b,
                                        p.w + row * HI, p.idx + row * p.k);
            }
        }
    }
}

// ----------------------------------------------------------- dense prefill
// Small candidate sets (N <= 2048): every visible score of a query is written
// to LDS once as an order-preserving key, then one exact selection per query
// (no streaming compactions).  Same scoring tiles and the same exact decision
// rule as the streaming kernel.
//
// SAMPLE mode (first pass of the long prefill pipeline): the same scoring over
// the sampled entries 0, S, 2S, ... only; per query the sample_j-th largest
// sampled score becomes the row's threshold estimate (no selection output).
template <typename T, int HI, int DI, bool SAMPLE>
__global__ __launch_bounds__(WAVES * 64, (HI <= 4 && DI == 64) ? 4 : 1) void index_dense_kernel(IdxParams p) {
    typedef IdxMma<T, DI> MM;
    constexpr int QPT = 16 / HI;
    constexpr int SLOTS = HI == 1 ? 4 : (HI == 2 ? 2 : 1);
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q4 = lane >> 4;
    const int qpw = p.qpw, np = p.cap, mcap = p.mcap;   // cap = keys per query (>= N)
    const int RT = qpw / QPT;
    // sampled scores only estimate a threshold (any value is valid there, it
    // only sets the list lengths), so the sampling pass keeps the upper 16
    // bits of each order-preserving key: half the LDS per sample
    constexpr int KB = SAMPLE ? 2 : 4;   // LDS bytes per key
    char* base = smem + (size_t)wave * p.wave_stride;
    uint32_t* keys_all = reinterpret_cast<uint32_t*>(base);
    uint32_t* hist = reinterpret_cast<uint32_t*>(base + (size_t)KB * qpw * np);
    double* mex = reinterpret_cast<double*>(base + (size_t)KB * qpw * np + 1024);
    int32_t* mpos = reinterpret_cast<int32_t*>(base + (size_t)KB * qpw * np + 1024 + 8ull * mcap);
    float* qn = reinterpret_cast<float*>(base + (size_t)KB * qpw * np + 1024 + 12ull * mcap);

    // later queries (more visible entries) first: the light work runs last
    const int qt = p.nqt - 1 - (int)(blockIdx.x % p.nqt);
    const int b = blockIdx.x / p.nqt;
    const int q0 = (qt * WAVES + wave) * qpw;
    const T* qI = reinterpret_cast<const T*>(p.qI);
    const T* kI_b = reinterpret_cast<const T*>(p.kI) + (long long)b * p.N * DI;

    // Cooperative scoring (one row tile per wave): the waves score the queries
    // of the whole workgroup together, wave w taking every WAVES-th entry tile,
    // so that each loaded key tile feeds WAVES row tiles (a quarter of the tile
    // loads on the longest wave's path).  Row tile rt is then wave rt's block
    // of queries and its keys go to that wave's LDS region.
    const bool coop = RT == 1 && WAVES <= MAX_RT;
    const int NRT = coop ? WAVES : RT;   // row tiles this wave scores
    auto rt_q0 = [&](int rt) { return coop ? (qt * WAVES + rt) * qpw : q0 + rt * QPT; };
    auto rt_has = [&](int rt, int ql) { return rt < NRT && (coop ? ql < qpw : rt * QPT + ql < qpw); };
    auto rt_keys = [&](int rt) {   // (in key units of KB bytes)
        return coop ? reinterpret_cast<char*>(smem + (size_t)rt * p.wave_stride)
                    : reinterpret_cast<char*>(base) + (size_t)KB * rt * QPT * np;
    };

    typename MM::F a[MAX_RT][MM::KS];
    float wr[MAX_RT][4];
    const int rho = lane & 15;
#pragma unroll
    for (int rt = 0; rt < MAX_RT; ++rt) {
        const int ql = rho / HI, hh = rho % HI;
        const int i = rt_q0(rt) + ql;
        const bool ok = rt_has(rt, ql) && i < p.Tq;
        MM::load_a(qI + (((long long)b * p.Tq + (ok ? i : 0)) * HI + hh) * DI, ok, q4, a[rt]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * q4 + r;
            const int qr = row / HI, hr = row % HI;
            const int ir = rt_q0(rt) + qr;
            wr[rt][r] = (rt_has(rt, qr) && ir < p.Tq) ? p.w[((long long)b * p.Tq + ir) * HI + hr] : 0.f;
        }
        float n2 = MM::sq(a[rt]);
        n2 = sum_xrows(n2);
        if (coop ? rt == wave : rt < RT) {
            // sum_h |w_h| ||q_h|| of the wave's own queries
            const int qsl = lane < QPT ? lane : 0;
            float acc = 0.f;
            for (int h = 0; h < HI; ++h) {
                const float nr = __shfl(n2, qsl * HI + h);
                const int ir = rt_q0(rt) + qsl;
                const float wv = (ir < p.Tq && rt_has(rt, qsl)) ? p.w[((long long)b * p.Tq + ir) * HI + h] : 0.f;
                acc += fabsf(wv) * sqrtf(nr);
            }
            const int qs = coop ? lane : rt * QPT + lane;
            if (lane < QPT && qs < qpw) qn[qs] = acc;
        }
    }
    // visible entries of the scored queries (SAMPLE: sampled entries)
    const int S = SAMPLE ? p.sample_stride : 1;
    int nv_max = 0;
    for (int rt = 0; rt < (coop ? NRT : 1); ++rt)
        for (int qw = 0; qw < qpw; ++qw) {
            const int i = (coop ? rt_q0(rt) : q0) + qw;
            if (i < p.Tq) nv_max = max(nv_max, (int)n_visible(row_pos0(p, b) + i, p.W, p.m, p.N));
        }
    if (SAMPLE) nv_max = (nv_max + S - 1) / S;
    float kmax2 = 0.f;
    // ---- all scores -> LDS keys
    auto score_tile = [&](int c0, const typename MM::F* bf) {
        const int c = c0 + rho;
        float n2 = MM::sq(bf);
        n2 = sum_xrows(n2);
        kmax2 = fmaxf(kmax2, n2);
#pragma unroll
        for (int rt = 0; rt < MAX_RT; ++rt) {
            if (rt >= NRT) break;
            const f32x4_t acc = MM::mma(a[rt], bf);
            float sc[4];
            int qs[4];
            bool own[4];
            const int ns = tile_scores<HI>(acc, wr[rt], q4, sc, qs, own);
            char* kd = rt_keys(rt);
#pragma unroll
            for (int sl = 0; sl < SLOTS; ++sl) {
                if (sl >= ns) break;
                if (own[sl] && rt_has(rt, qs[sl]) && c < np) {
                    if constexpr (SAMPLE)
                        reinterpret_cast<uint16_t*>(kd)[qs[sl] * np + c] = (uint16_t)(fkey(sc[sl]) >> 16);
                    else
                        reinterpret_cast<uint32_t*>(kd)[qs[sl] * np + c] = fkey(sc[sl]);
                }
            }
        }
    };
    auto load_b = [&](int c0, typename MM::F* bf) {
        const long long e = (long long)(c0 + rho) * S;
        MM::load_a(kI_b + (e < p.N ? e : 0) * DI, e < p.N, q4, bf);
    };
    // the wave's entry tiles j = 0 .. ntl-1 (cooperative: every WAVES-th tile)
    const int ntot = (nv_max + TILE - 1) / TILE;
    const int ntl = coop ? (ntot > wave ? (ntot - wave + WAVES - 1) / WAVES : 0) : ntot;
    auto tile_c0 = [&](int j) { return (coop ? wave + WAVES * j : j) * TILE; };
    constexpr int PF = 2;
    typename MM::F bq0[PF][MM::KS], bq1[PF][MM::KS];
    auto group = [&](int l0, typename MM::F (&cur)[PF][MM::KS], typename MM::F (&nxt)[PF][MM::KS]) {
        const int l1 = l0 + PF;
#pragma unroll
        for (int t = 0; t < PF; ++t)
            if (l1 + t < ntl) load_b(tile_c0(l1 + t), nxt[t]);
#pragma unroll
        for (int t = 0; t < PF; ++t)
            if (l0 + t < ntl) score_tile(tile_c0(l0 + t), cur[t]);
    };
#pragma unroll
    for (int t = 0; t < PF; ++t)
        if (t < ntl) load_b(tile_c0(t), bq0[t]);
    for (int l0 = 0; l0 < ntl; l0 += 2 * PF) {
        group(l0, bq0, bq1);
        if (l0 + PF < ntl) group(l0 + PF, bq1, bq0);
    }
    kmax2 = wave_max_f(kmax2);
    if (coop) {
        // every wave's keys complete; largest ||k||^2 over the workgroup's tiles
        // (each wave's hist slot 0 carries it across; read before any wave
        // reuses its hist)
        if (lane == 0) hist[0] = __float_as_uint(kmax2);
        __syncthreads();
        float km = 0.f;
        for (int w = 0; w < WAVES; ++w)
            km = fmaxf(km, __uint_as_float(*reinterpret_cast<const uint32_t*>(smem + (size_t)w * p.wave_stride +
                                                                             (size_t)KB * qpw * np)));
        kmax2 = km;
        __syncthreads();
    } else {
        wave_lds_sync();
    }

    if constexpr (SAMPLE) {
        // largest ||k||^2 of the sequence (every entry, not only the sampled ones)
        float km2 = 0.f;
        for (int j = lane; j < p.kblk; j += 64) km2 = fmaxf(km2, p.kmax_part[(long long)b * p.kblk + j]);
        const float kmax_all = sqrtf(wave_max_f(km2));
        for (int qw = 0; qw < qpw; ++qw) {
            const int i = q0 + qw;
            if (i >= p.Tq) break;
            const long long row = (long long)b * p.Tq + i;
            const int n = (int)n_visible(row_pos0(p, b) + i, p.W, p.m, p.N);
            const int ns = (n + S - 1) / S;
            const float delta = p.err_c * qn[qw] * kmax_all;
            uint32_t thr = 0u, tau = 0u;   // 0: list every visible entry
            // (a query whose whole visible set fits the list pass's LDS)
            if (n > p.list_lds_cap && ns >= p.sample_j) {
                // the sample_j-th largest truncated key, as a full key with
                // its low 16 bits zero: at most the sampled score itself
                tau = radix_kth16(reinterpret_cast<const uint16_t*>(base) + qw * np, ns, p.sample_j, hist) << 16;
                thr = fkey(key_f(tau) - 2.0f * delta);
            }
            if (lane == 0) {
                p.row_thr[row] = thr;
                p.row_tau[row] = tau;
                p.row_delta[row] = delta;
            }
        }
        return;
    }

    // ---- one exact selection per query
    const float kmax = sqrtf(kmax2);
    for (int qw = 0; qw < qpw; ++qw) {
        const int i = q0 + qw;
        if (i >= p.Tq) break;
        const long long row = (long long)b * p.Tq + i;
        const int n = (int)n_visible(row_pos0(p, b) + i, p.W, p.m, p.N);
        WaveBuf q{keys_all + qw * np, nullptr, hist, mpos, mex, nullptr};
        final_select<T, HI, DI>(q, PosIds{}, n, min(p.k, n), p.k, p.err_c * qn[qw] * kmax, mcap, qI + row * HI * DI,
                                kI_b, p.w + row * HI, p.idx + row * p.k);
    }
}

// ----------------------------------------------------------- long prefill
// Long candidate sets (N > 2048) in prefill, four passes:
//  L0 (index_kmax_kernel): max ||k||^2 per block of entries (for delta);
//  L1 (index_dense_kernel, SAMPLE): per query, a threshold tau from every S-th
//     entry: the sample_j-th largest sampled float32 score;
//  L2 (index_filter_kernel): all float32 scores, entries with
//     score >= tau - 2 delta appended in entry order to the row's list;
//  L3 (index_list_final_kernel): when the list did not overflow and holds at
//     least k_eff entries with score >= tau, the row's float32 k-th score T is
//     >= tau, so the list holds every entry with score >= T - 2 delta: the same
//     exact selection as the other kernels runs over the list.  Any other row
//     is flagged and recomputed by the streaming kernel.
constexpr int kKmaxBlock = 1024;

template <typename T, int DI>
__global__ __launch_bounds__(256) void index_kmax_kernel(IdxParams p) {
    __shared__ float part[4];
    const int tid = threadIdx.x;
    const long long b = blockIdx.x / p.kblk, blk = blockIdx.x % p.kblk;
    const T* kI_b = reinterpret_cast<const T*>(p.kI) + b * (long long)p.N * DI;
    constexpr int V = Elem<T>::kVec;
    float m = 0.f;
    for (int e = tid; e < kKmaxBlock; e += 256) {
        const long long c = blk * kKmaxBlock + e;
        if (c >= p.N) break;
        float s = 0.f;
#pragma unroll
        for (int d0 = 0; d0 < DI; d0 += V) {
            float f[V];
            Elem<T>::unpack(ld16(kI_b + c * DI + d0), f);
#pragma unroll
            for (int j = 0; j < V; ++j) s = fmaf(f[j], f[j], s);
        }
        m = fmaxf(m, s);
    }
    m = wave_max_f(m);
    if ((tid & 63) == 0) part[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) p.kmax_part[blockIdx.x] = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
}

// Row tiles per wave of the filter pass (host and device agree on it): more
// queries per wave read each key tile fewer times; register budget bounds it.
__host__ __device__ constexpr int filter_row_tiles(bool f32, int hi, int di) {
    return f32 ? 1 : 4;
}

// Workgroups per CU the filter pass is compiled for.  Four (a 128-register
// budget) where the kernel fits it without spills in its loop: its MFMAs then
// write ordinary registers (no accumulator-register copies) and four waves
// share each SIMD; elsewhere the compiler's default.
__host__ __device__ constexpr int filter_min_blocks(bool f32, int hi, int di) {
    return (!f32 && di == 64 && (hi == 4 || hi == 8)) ? 4 : 1;
}

// L2: each wave scores FRT row tiles of queries against all their visible
// entries (MFMA tiles as above) and appends the entries that pass the row's
// threshold to the row's list in global memory.  For bf16 keys (64 or 128
// dimensions) the four waves of a workgroup (consecutive queries) share each
// key tile: groups of four tiles are staged in LDS (double-buffered, the next
// group's global loads in flight while the current one is scored), so each
// key row is read from L2 once per 64 queries instead of once per 16.  Other
// forms load their key tiles per wave into registers.
template <typename T, int DI>
__host__ __device__ constexpr bool filter_shared_tiles() {
    return std::is_same<T, bf16_t>::value && (DI == 64 || DI == 128);
}

template <typename T, int HI, int DI>
__global__ __launch_bounds__(WAVES * 64, filter_min_blocks(std::is_same<T, float>::value, HI, DI))
void index_filter_kernel(IdxParams p) {
    typedef IdxMma<T, DI> MM;
    constexpr int QPT = 16 / HI;
    constexpr int SLOTS = HI == 1 ? 4 : (HI == 2 ? 2 : 1);
    constexpr int FRT = filter_row_tiles(std::is_same<T, float>::value, HI, DI);
    constexpr int QPW = FRT * QPT;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q4 = lane >> 4, rho = lane & 15;
    const int qt = p.nqt - 1 - (int)(blockIdx.x % p.nqt);
    const int b = blockIdx.x / p.nqt;
    const int q0 = (qt * WAVES + wave) * QPW;
    constexpr bool SHARED = filter_shared_tiles<T, DI>();
    // with shared key tiles every wave takes part in the loads and barriers
    // (a wave past the last query has no visible entries and scores nothing)
    if (!SHARED && q0 >= p.Tq) return;
    const T* qI = reinterpret_cast<const T*>(p.qI);
    const T* kI_b = reinterpret_cast<const T*>(p.kI) + (long long)b * p.N * DI;
    const int lcap = p.list_cap;

    typename MM::F a[FRT][MM::KS];
    float wr[FRT][4];
#pragma unroll
    for (int rt = 0; rt < FRT; ++rt) {
        const int qw = rt * QPT + rho / HI, hh = rho % HI;
        const int i = q0 + qw;
        const bool ok = i < p.Tq;
        MM::load_a(qI + (((long long)b * p.Tq + (ok ? i : 0)) * HI + hh) * DI, ok, q4, a[rt]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * q4 + r;
            const int ir = q0 + rt * QPT + row / HI;
            wr[rt][r] = ir < p.Tq ? p.w[((long long)b * p.Tq + ir) * HI + row % HI] : 0.f;
        }
    }
    // per (row tile, slot): the lane group's list, visible entries, threshold
    // (as a float: score >= thr_f <=> key >= row_thr), count
    uint2* lst[FRT][SLOTS];
    int nv[FRT][SLOTS], cnt[FRT][SLOTS];
    float thr_f[FRT][SLOTS];
    int nv_max = 0;
#pragma unroll
    for (int rt = 0; rt < FRT; ++rt)
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
            int qw;
            if (HI == 1) qw = 4 * q4 + sl;
            else if (HI == 2) qw = 2 * q4 + sl;
            else if (HI == 4) qw = q4;
            else if (HI == 8) qw = q4 >> 1;
            else qw = 0;
            const int i = q0 + rt * QPT + qw;
            const bool ok = i < p.Tq;
            const long long row = (long long)b * p.Tq + (ok ? i : 0);
            lst[rt][sl] = p.row_lists + row * lcap;
            nv[rt][sl] = ok ? (int)n_visible(row_pos0(p, b) + i, p.W, p.m, p.N) : 0;
            const uint32_t tk = ok ? p.row_thr[row] : 0u;
            thr_f[rt][sl] = tk == 0u ? -INFINITY : key_f(tk);
            cnt[rt][sl] = 0;
            nv_max = max(nv_max, nv[rt][sl]);
        }
    nv_max = (int)wave_allreduce((uint32_t)nv_max, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
    const uint32_t below = (1u << rho) - 1u;   // lanes of this 16-lane group below this one

    auto load_b = [&](int c0, typename MM::F* bf) {
        const int c = c0 + rho;
        MM::load_a(kI_b + (long long)(c < p.N ? c : 0) * DI, c < p.N, q4, bf);
    };
    // every query of the wave sees at least nv_min entries: tiles below it
    // need no visibility test
    int nv_min = 1 << 30;
#pragma unroll
    for (int rt = 0; rt < FRT; ++rt)
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) nv_min = min(nv_min, nv[rt][sl]);
    nv_min = (int)wave_allreduce((uint32_t)nv_min, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
    auto filter_tile = [&](int c0, const typename MM::F* bf) {
        const int c = c0 + rho;
        const bool full = c0 + TILE <= nv_min;
        f32x4_t acc[FRT];
#pragma unroll
        for (int rt = 0; rt < FRT; ++rt) acc[rt] = MM::mma(a[rt], bf);
#pragma unroll
        for (int rt = 0; rt < FRT; ++rt) {
            float sc[4];
            int qs[4];
            bool own[4];
            const int ns = tile_scores<HI>(acc[rt], wr[rt], q4, sc, qs, own);
#pragma unroll
            for (int sl = 0; sl < SLOTS; ++sl) {
                if (sl >= ns) break;
                const bool ins = own[sl] && (full || c < nv[rt][sl]) && sc[sl] >= thr_f[rt][sl];
                const unsigned long long msk = __ballot(ins);
                if (msk == 0ull) continue;
                const uint32_t gb = (uint32_t)(msk >> (16 * q4)) & 0xFFFFu;
                if (ins) {
                    const int pos = cnt[rt][sl] + __popc(gb & below);
                    // the raw float bits: the list pass turns them into keys
                    if (pos < lcap) lst[rt][sl][pos] = make_uint2(__float_as_uint(sc[sl]), (uint32_t)c);
                }
                cnt[rt][sl] += __popc(gb);
            }
        }
    };
    if constexpr (SHARED) {
        // LDS groups of GT key tiles, rows of DI bf16 (DI / 8 pieces of 16
        // bytes); piece j of row r sits at slot j ^ (r & 7), so the 8 lanes of
        // one operand read (rows rho, one piece) hit distinct banks
        constexpr int GT = 4, GROWS = GT * TILE, PIECES = DI / 8;
        constexpr int LPT = GROWS * PIECES / (WAVES * 64);   // 16-byte loads per thread per group
        static_assert(PIECES % 8 == 0 && LPT * WAVES * 64 == GROWS * PIECES,
                      "shared key tiles: bf16, d_idx 64 or 128");
        __shared__ __attribute__((aligned(16))) uint4 kt[2][GROWS * PIECES];
        __shared__ int wg_nv[WAVES];
        if (lane == 0) wg_nv[wave] = nv_max;
        __syncthreads();
        const int nv_wg = max(max(wg_nv[0], wg_nv[1]), max(wg_nv[2], wg_nv[3]));
        const int ngroups = (nv_wg + GROWS - 1) / GROWS;
        uint4 pre[LPT];
        auto load_group = [&](int g) {
#pragma unroll
            for (int u = 0; u < LPT; ++u) {
                const int e = u * WAVES * 64 + tid, r = e / PIECES, j = e % PIECES;
                const int c = g * GROWS + r;
                pre[u] = ld16(kI_b + (long long)(c < p.N ? c : 0) * DI + 8 * j);
            }
        };
        auto store_group = [&](int slot) {
#pragma unroll
            for (int u = 0; u < LPT; ++u) {
                const int e = u * WAVES * 64 + tid, r = e / PIECES, j = e % PIECES;
                kt[slot][r * PIECES + (j ^ (r & 7))] = pre[u];
            }
        };
        if (ngroups > 0) {
            load_group(0);
            store_group(0);
        }
        __syncthreads();
        for (int g = 0; g < ngroups; ++g) {
            if (g + 1 < ngroups) load_group(g + 1);
            const uint4* buf = kt[g & 1];
#pragma unroll
            for (int t = 0; t < GT; ++t) {
                const int c0 = g * GROWS + t * TILE;
                if (c0 < nv_max) {
                    const int r = t * TILE + rho;
                    typename MM::F bf[MM::KS];
#pragma unroll
                    for (int ks = 0; ks < MM::KS; ++ks) {
                        const int j = 4 * ks + q4;
                        bf[ks] = *reinterpret_cast<const bf16x8_t*>(&buf[r * PIECES + (j ^ (r & 7))]);
                    }
                    filter_tile(c0, bf);
                }
            }
            // the other slot was last read before the previous barrier
            if (g + 1 < ngroups) store_group((g + 1) & 1);
            __syncthreads();
        }
    } else {
        constexpr int PF = 2;
        typename MM::F bq0[PF][MM::KS], bq1[PF][MM::KS];
        auto group = [&](int g0, typename MM::F (&cur)[PF][MM::KS], typename MM::F (&nxt)[PF][MM::KS]) {
            const int g1 = g0 + PF * TILE;
            if (g1 < nv_max) {
#pragma unroll
                for (int t = 0; t < PF; ++t) load_b(g1 + t * TILE, nxt[t]);
            }
#pragma unroll
            for (int t = 0; t < PF; ++t)
                if (g0 + t * TILE < nv_max) filter_tile(g0 + t * TILE, cur[t]);
        };
        if (nv_max > 0) {
#pragma unroll
            for (int t = 0; t < PF; ++t) load_b(t * TILE, bq0[t]);
        }
        for (int g0 = 0; g0 < nv_max; g0 += 2 * PF * TILE) {
            group(g0, bq0, bq1);
            if (g0 + PF * TILE < nv_max) group(g0 + PF * TILE, bq1, bq0);
        }
    }
    // counts (a count above list_cap marks an overflowed list)
    const bool owner = (HI <= 4) || (HI == 8 ? (q4 & 1) == 0 : q4 == 0);
#pragma unroll
    for (int rt = 0; rt < FRT; ++rt)
#pragma unroll
        for (int sl = 0; sl < SLOTS; ++sl) {
            int qw;
            if (HI == 1) qw = 4 * q4 + sl;
            else if (HI == 2) qw = 2 * q4 + sl;
            else if (HI == 4) qw = q4;
            else if (HI == 8) qw = q4 >> 1;
            else qw = 0;
            const int i = q0 + rt * QPT + qw;
            if (owner && rho == 0 && i < p.Tq) p.list_cnt[(long long)b * p.Tq + i] = cnt[rt][sl];
        }
}

// L3: one wave per row: exact selection over the row's list, or a failure flag.
template <typename T, int HI, int DI>
__global__ __launch_bounds__(64) void index_list_final_kernel(IdxParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x;
    const long long row = blockIdx.x;
    const long long b = row / p.Tq, i = row % p.Tq;
    const int lcap = p.list_cap;
    const int kcap = p.list_lds_cap;   // <= lcap: longer lists fail over to the streaming kernel
    // LDS: keys[kcap] hist[256] mex[list_mcap] mpos[list_mcap] mid[list_mcap]; entries stay in the list
    WaveBuf wb;
    wb.keys = reinterpret_cast<uint32_t*>(smem);
    wb.ids = nullptr;
    wb.hist = reinterpret_cast<uint32_t*>(smem + 4ull * kcap);
    wb.mex = reinterpret_cast<double*>(smem + 4ull * kcap + 1024);
    wb.mpos = reinterpret_cast<int32_t*>(smem + 4ull * kcap + 1024 + 8ull * p.list_mcap);
    wb.mid = reinterpret_cast<int32_t*>(smem + 4ull * kcap + 1024 + 12ull * p.list_mcap);
    const long long nvq = n_visible(row_pos0(p, b) + i, p.W, p.m, p.N);
    const int k_eff = (int)std::min<long long>(p.k, nvq);
    const int cnt = p.list_cnt[row];
    bool ok = cnt <= kcap;
    if (ok) {
        // two (key, entry) pairs per lane and 16-byte load, eight loads in flight
        const uint32_t tau = p.row_tau[row];
        const uint2* lst = p.row_lists + row * lcap;
        int n_ge = 0;
        for (int base = 0; base < cnt; base += 1024) {
            uint4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = base + 128 * u + 2 * lane;
                if (e < cnt) v[u] = ld16(lst + e);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int e = base + 128 * u + 2 * lane;
                if (e < cnt) {
                    const uint32_t k0 = fkey(__uint_as_float(v[u].x)), k1 = fkey(__uint_as_float(v[u].z));
                    *reinterpret_cast<uint2*>(wb.keys + e) = make_uint2(k0, k1);
                    n_ge += (k0 >= tau) + (e + 1 < cnt && k1 >= tau);
                }
            }
        }
        n_ge = (int)wave_allreduce((uint32_t)n_ge, [](uint32_t x, uint32_t y) { return x + y; });
        ok = n_ge >= k_eff;
    }
    if (lane == 0) p.row_fail[row] = ok ? 0 : 1;
    if (!ok) return;
    wave_lds_sync();
    const T* qI = reinterpret_cast<const T*>(p.qI);
    const T* kI_b = reinterpret_cast<const T*>(p.kI) + b * (long long)p.N * DI;
    final_select<T, HI, DI>(wb, ListIds{p.row_lists + row * lcap}, cnt, k_eff, p.k, p.row_delta[row], p.list_mcap,
                            qI + row * HI * DI, kI_b,
                            p.w + row * HI, p.idx + row * p.k);
}

// ----------------------------------------------------------- split pipeline
// S1: one wave per (query row, chunk of entries): float32 scores of the row
// against the chunk (written to the workspace), the chunk's chunk_k-th largest
// score and the chunk's max ||k||^2.  If every chunk holds >= chunk_k visible
// entries and nchunks * chunk_k >= k, the minimum over chunks of those scores
// is a lower bound of the row's float32 k-th score.
template <typename T, int HI, int DI>
__global__ __launch_bounds__(64) void index_split_score_kernel(IdxParams p) {
    typedef IdxMma<T, DI> MM;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint32_t* skeys = reinterpret_cast<uint32_t*>(smem);          // [chunk]
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + 4ull * p.chunk);
    const int lane = threadIdx.x, q4 = lane >> 4, rho = lane & 15;
    const int chunk_id = blockIdx.x % p.nchunks;
    const long long row = blockIdx.x / p.nchunks;
    const long long b = row / p.Tq, i = row % p.Tq;
    const long long nvq = n_visible(row_pos0(p, b) + i, p.W, p.m, p.N);
    const long long c_lo = (long long)chunk_id * p.chunk;
    const long long c_hi = std::min<long long>(c_lo + p.chunk, nvq);
    const T* qI = reinterpret_cast<const T*>(p.qI);
    const T* kI_b = reinterpret_cast<const T*>(p.kI) + b * (long long)p.N * DI;

    // A rows: the HI heads of this query (rows >= HI are zero)
    typename MM::F a[MM::KS];
    MM::load_a(qI + (row * HI + (rho < HI ? rho : 0)) * DI, rho < HI, q4, a);
    float wr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int rr = 4 * q4 + r;
        wr[r] = rr < HI ? p.w[row * HI + rr] : 0.f;
    }
    if (chunk_id == 0) {
        float n2 = MM::sq(a);
        n2 = sum_xrows(n2);
        float acc = 0.f;
        for (int h = 0; h < HI; ++h) acc += fabsf(p.w[row * HI + h]) * sqrtf(__uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(n2), h)));
        if (lane == 0) p.row_qn[row] = acc;
    }
    float kmax2 = 0.f;
    auto load_b = [&](long long c0, typename MM::F* bf) {
        const long long c = c0 + rho;
        const bool cok = c < c_hi;
        MM::load_a(kI_b + (cok ? c : 0) * DI, cok, q4, bf);
    };
    auto score_tile = [&](long long c0, const typename MM::F* bf) {
        const long long c = c0 + rho;
        const bool cok = c < c_hi;
        float n2 = MM::sq(bf);
        n2 = sum_xrows(n2);
        kmax2 = fmaxf(kmax2, n2);
        const f32x4_t acc = MM::mma(a, bf);
        float s[4];
        int qs[4];
        bool own[4];
        tile_scores<HI>(acc, wr, q4, s, qs, own);
        // the row is query 0 of the tile; its owning lanes hold s[0]
        if (own[0] && qs[0] == 0 && cok) {
            p.scores[row * p.N + c] = s[0];
            skeys[c - c_lo] = fkey(s[0]);
        }
    };
    // the chunk streams through registers PF tiles at a time: the next group's
    // loads are in flight while a group is scored (two alternating buffers, so
    // rows in flight are never copied)
    constexpr int PF = 4;
    typename MM::F bq0[PF][MM::KS], bq1[PF][MM::KS];
    auto group = [&](long long g0, typename MM::F (&cur)[PF][MM::KS], typename MM::F (&nxt)[PF][MM::KS]) {
        const long long g1 = g0 + PF * TILE;
        if (g1 < c_hi) {
#pragma unroll
            for (int t = 0; t < PF; ++t) load_b(g1 + t * TILE, nxt[t]);
        }
#pragma unroll
        for (int t = 0; t < PF; ++t)
            if (g0 + t * TILE < c_hi) score_tile(g0 + t * TILE, cur[t]);
    };
    if (c_lo < c_hi) {
#pragma unroll
        for (int t = 0; t < PF; ++t) load_b(c_lo + t * TILE, bq0[t]);
    }
    for (long long g0 = c_lo; g0 < c_hi; g0 += 2 * PF * TILE) {
        group(g0, bq0, bq1);
        if (g0 + PF * TILE < c_hi) group(g0 + PF * TILE, bq1, bq0);
    }
    kmax2 = wave_max_f(kmax2);
    wave_lds_sync();
    const int n = c_hi > c_lo ? (int)(c_hi - c_lo) : 0;
    float lb = -INFINITY;
    if (n >= p.chunk_k) {
        int n_gt;
        lb = key_f(radix_kth(skeys, n, p.chunk_k, hist, &n_gt));
    }
    if (lane == 0) {
        p.chunk_lb[row * p.nchunks + chunk_id] = lb;
        p.chunk_kmax[row * p.nchunks + chunk_id] = kmax2;
    }
}

__device__ __forceinline__ void row_bound(const IdxParams& p, long long row, float* lb_out, float* delta_out) {
    const int lane = __lane_id();
    float lb = INFINITY, km = 0.f;
    for (int j = lane; j < p.nchunks; j += 64) {
        lb = fminf(lb, p.chunk_lb[row * p.nchunks + j]);
        km = fmaxf(km, p.chunk_kmax[row * p.nchunks + j]);
    }
    for (int off = 32; off > 0; off >>= 1) {
        lb = fminf(lb, __shfl_xor(lb, off));
        km = fmaxf(km, __shfl_xor(km, off));
    }
    *lb_out = lb;
    *delta_out = p.err_c * p.row_qn[row] * sqrtf(km);
}

// S2: one wave per (row, chunk): keep, in index order, the chunk's entries whose
// float32 score can still reach the row's top-k (>= lower bound - 2 delta).
__global__ __launch_bounds__(64) void index_split_collect_kernel(IdxParams p) {
    const int lane = threadIdx.x;
    const int chunk_id = blockIdx.x % p.nchunks;
    const long long row = blockIdx.x / p.nchunks;
    const long long b = row / p.Tq, i = row % p.Tq;
    const long long nvq = n_visible(row_pos0(p, b) + i, p.W, p.m, p.N);
    float lb, delta;
    row_bound(p, row, &lb, &delta);
    const uint32_t lo = lb == -INFINITY ? 0u : fkey(lb - 2.0f * delta);
    const long long c_lo = (long long)chunk_id * p.chunk;
    const long long c_hi = std::min<long long>(c_lo + p.chunk, nvq);
    uint32_t* lk = p.lists + (row * p.nchunks + chunk_id) * (long long)p.list_cap;
    int32_t* li = p.list_idx + (row * p.nchunks + chunk_id) * (long long)p.list_cap;
    int out = 0;
    for (long long base = c_lo; base < c_hi; base += 64) {
        const long long c = base + lane;
        uint32_t key = 0u;
        bool keep = false;
        if (c < c_hi) {
            key = fkey(p.scores[row * p.N + c]);
            keep = key >= lo;
        }
        const unsigned long long msk = __ballot(keep);
        const int pos = out + __popcll(msk & lanemask_lt());
        if (keep && pos < p.list_cap) {
            lk[pos] = key;
            li[pos] = (int32_t)c;
        }
        out += __popcll(msk);
    }
    if (lane == 0) p.list_cnt[row * p.nchunks + chunk_id] = out;
}

// S3: one workgroup (kFinalThreads) per row.  When no chunk list overflowed
// and the lists fit in LDS, all their entries are gathered in parallel, in
// entry order, and one wave makes the exact final selection over them;
// otherwise one wave streams the lists (and overflowed chunks' scores)
// through the candidate buffer as before.
constexpr int kFinalThreads = 256;

template <typename T, int HI, int DI>
__global__ __launch_bounds__(kFinalThreads) void index_split_final_kernel(IdxParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const long long row = blockIdx.x;
    const long long b = row / p.Tq, i = row % p.Tq;
    const int cap = p.cap;   // LDS candidate slots (>= the streaming buffer)
    WaveBuf wb;
    wb.keys = reinterpret_cast<uint32_t*>(smem);
    wb.ids = reinterpret_cast<int32_t*>(smem + 4ull * cap);
    wb.hist = reinterpret_cast<uint32_t*>(smem + 8ull * cap);
    wb.mex = reinterpret_cast<double*>(smem + 8ull * cap + 1024);
    wb.mpos = reinterpret_cast<int32_t*>(smem + 8ull * cap + 1024 + 8ull * p.mcap);
    wb.mid = reinterpret_cast<int32_t*>(smem + 8ull * cap + 1024 + 12ull * p.mcap);
    int32_t* offs = reinterpret_cast<int32_t*>(smem + 8ull * cap + 1024 + 16ull * p.mcap);  // [nchunks + 1]
    __shared__ int s_total, s_over;
    const long long nvq = n_visible(row_pos0(p, b) + i, p.W, p.m, p.N);
    const int k_eff = (int)std::min<long long>(p.k, nvq);
    float lb, delta;
    row_bound(p, row, &lb, &delta);
    const T* qI = reinterpret_cast<const T*>(p.qI);
    const T* kI_b = reinterpret_cast<const T*>(p.kI) + b * (long long)p.N * DI;

    // ---- list sizes -> entry offsets (exclusive prefix in chunk order)
    if (wave == 0) {
        int base = 0, over = 0;
        for (int j0 = 0; j0 < p.nchunks; j0 += 64) {
            const int j = j0 + lane;
            const int lc = j < p.nchunks ? p.list_cnt[row * p.nchunks + j] : 0;
            over |= lc > p.list_cap;
            const int incl = wave_incl_scan(lc);
            if (j < p.nchunks) offs[j] = base + incl - lc;
            base += __builtin_amdgcn_readlane(incl, 63);
        }
        over = __any(over);
        if (lane == 0) {
            offs[p.nchunks] = base;
            s_total = base;
            s_over = over;
        }
    }
    __syncthreads();
    const int total = s_total;
    if (!s_over && total <= cap) {
        // ---- parallel gather: entry t belongs to the chunk whose offset range
        // holds it; each thread places four entries per round, their eight
        // loads in flight together
        constexpr int GU = 4;
        for (int t0 = tid; t0 < total; t0 += GU * kFinalThreads) {
            long long src[GU];
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int t = t0 + u * kFinalThreads;
                int lo = 0, hi = p.nchunks - 1;   // last chunk with offs[j] <= t
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (offs[mid] <= t) lo = mid;
                    else hi = mid - 1;
                }
                src[u] = t < total ? (row * p.nchunks + lo) * (long long)p.list_cap + (t - offs[lo]) : -1;
            }
            uint32_t kv[GU];
            int32_t iv[GU];
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                if (src[u] >= 0) {
                    kv[u] = p.lists[src[u]];
                    iv[u] = p.list_idx[src[u]];
                }
            }
#pragma unroll
            for (int u = 0; u < GU; ++u) {
                const int t = t0 + u * kFinalThreads;
                if (src[u] >= 0) {
                    wb.keys[t] = kv[u];
                    wb.ids[t] = iv[u];
                }
            }
        }
        __syncthreads();
        if (wave == 0)
            final_select<T, HI, DI>(wb, LdsIds{wb.ids}, total, k_eff, p.k, delta, p.mcap, qI + row * HI * DI, kI_b,
                                    p.w + row * HI, p.idx + row * p.k);
        return;
    }
    if (wave != 0) return;
    // ---- fallback: stream the chunk lists (or whole chunks) through the buffer
    uint32_t tau = lb == -INFINITY ? 0u : fkey(lb - 2.0f * delta);
    int cnt = 0;
    for (int j = 0; j < p.nchunks; ++j) {
        const int lc = p.list_cnt[row * p.nchunks + j];
        const bool from_list = lc <= p.list_cap;
        const long long c_lo = (long long)j * p.chunk;
        const long long c_hi = std::min<long long>(c_lo + p.chunk, nvq);
        const long long n = from_list ? lc : (c_hi > c_lo ? c_hi - c_lo : 0);
        const uint32_t* lk = p.lists + (row * p.nchunks + j) * (long long)p.list_cap;
        const int32_t* li = p.list_idx + (row * p.nchunks + j) * (long long)p.list_cap;
        for (long long base = 0; base < n; base += 64) {
            const long long e = base + lane;
            uint32_t key = 0u;
            int32_t id = 0;
            bool ins = false;
            if (e < n) {
                if (from_list) {
                    key = lk[e];
                    id = li[e];
                } else {
                    id = (int32_t)(c_lo + e);
                    key = fkey(p.scores[row * p.N + id]);
                }
                ins = key >= tau;
            }
            const unsigned long long msk = __ballot(ins);
            if (ins) {
                const int pos = cnt + __popcll(msk & lanemask_lt());
                wb.keys[pos] = key;
                wb.ids[pos] = id;
            }
            cnt += __popcll(msk);
            if (cnt > p.stream_cap - 64) {
                wave_lds_sync();
                cnt = compact_stream(wb, cnt, k_eff, delta, p.stream_cap, 64, &tau);
            }
        }
    }
    wave_lds_sync();
    final_select<T, HI, DI>(wb, LdsIds{wb.ids}, cnt, k_eff, p.k, delta, p.mcap, qI + row * HI * DI, kI_b,
                            p.w + row * HI,
                            p.idx + row * p.k);
}

// No candidate entries (N = 0): every index row is -1.
__global__ __launch_bounds__(256) void index_fill_empty_kernel(IdxParams p) {
    const long long n = (long long)p.B * p.Tq * p.k;
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p.idx[i] = -1;
}

// ----------------------------------------------------------- host planning
// launch shape of a kernel that tiles queries over waves (dense / prefill kernels)
struct IdxLaunch {
    int qpw, nqt, wave_stride, cap;
    long long grid;
    size_t lds;
};

struct IdxPlan {
    IdxParams p;
    bool split;
    bool dense;  // small N: all scores of a query in LDS, one exact select
    bool longp;  // long prefill pipeline (sample, filter, list final, fallback)
    bool empty;  // no candidates (N = 0): every row is -1
    size_t lds;  // dense: per workgroup; split: final kernel; long: list final kernel
    size_t lds_score;
    long long grid;
    size_t ws_bytes;
    IdxLaunch ls, lf;  // long: sampling pass (dense kernel) and streaming fallback
    long long grid_kmax, grid_filter;
};

constexpr int kMaxLds = 160 * 1024;
constexpr int kDenseMaxN = 2048;
constexpr int kSampleMax = 1024;  // long prefill: sampled entries per query at most

int make_idx_plan(int B, int Tq, int N, int Hi, int d_idx, int64_t q_pos0, int m, int W, int k,
                  int dtype, IdxPlan& pl) {
    if (dtype != SHATTN_DTYPE_BF16 && dtype != SHATTN_DTYPE_F32)
        return fail(SHATTN_EINVAL, "csa_index_topk: unknown dtype %d", dtype);
    if (B < 0 || Tq < 0 || N < 0 || Hi < 1 || d_idx < 1 || m < 1 || W < 1 || k < 1 || q_pos0 < 0)
        return fail(SHATTN_EINVAL, "csa_index_topk: bad sizes B=%d Tq=%d N=%d Hi=%d d_idx=%d m=%d W=%d k=%d",
                    B, Tq, N, Hi, d_idx, m, W, k);
    if (Hi != 1 && Hi != 2 && Hi != 4 && Hi != 8 && Hi != 16)
        return fail(SHATTN_EUNSUPPORTED, "csa_index_topk: Hi=%d (supported: 1, 2, 4, 8, 16)", Hi);
    if (d_idx != 64 && d_idx != 128)
        return fail(SHATTN_EUNSUPPORTED, "csa_index_topk: d_idx=%d (supported: 64, 128)", d_idx);
    if (k > 2048) return fail(SHATTN_EUNSUPPORTED, "csa_index_topk: k=%d > 2048", k);
    IdxParams& p = pl.p;
    p = IdxParams{};
    p.B = B;
    p.Tq = Tq;
    p.N = N;
    p.k = k;
    p.m = m;
    p.W = W;
    p.q_pos0 = q_pos0;
    p.cap = ((k + std::max(64, k / 2)) + 63) / 64 * 64;
    p.mcap = std::min(p.cap, 256);
    // |float32 score - exact| <= err_c * sum_h |w_h| ||q_h|| * max ||k||:
    // 2*d_idx*u for the dot products (any summation order, rounding or
    // truncation inside the MFMA), Hi + 2 roundings of the weighted head sum,
    // and a factor 2 of margin.
    p.err_c = 2.0f * (2.0f * d_idx + Hi + 4.0f) * 5.9604645e-8f;
    pl.ws_bytes = 0;
    pl.grid = 0;
    pl.dense = false;
    pl.longp = false;
    pl.empty = false;
    pl.ls = IdxLaunch{};
    pl.lf = IdxLaunch{};
    pl.grid_kmax = pl.grid_filter = 0;
    const long long rows = (long long)B * Tq;
    pl.split = rows > 0 && rows <= 64 && N >= 8192;
    if (pl.split) {
        p.chunk = 2048;   // 2 waves per SIMD at 1M context x 16 rows
        p.nchunks = (N + p.chunk - 1) / p.chunk;
        p.chunk_k = (k + p.nchunks - 1) / p.nchunks;
        p.list_cap = 256;
        size_t off = 0;
        auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
        const size_t o_scores = take((size_t)rows * N * 4);
        const size_t o_lb = take((size_t)rows * p.nchunks * 4);
        const size_t o_km = take((size_t)rows * p.nchunks * 4);
        const size_t o_qn = take((size_t)rows * 4);
        const size_t o_lk = take((size_t)rows * p.nchunks * p.list_cap * 4);
        const size_t o_li = take((size_t)rows * p.nchunks * p.list_cap * 4);
        const size_t o_lc = take((size_t)rows * p.nchunks * 4);
        pl.ws_bytes = off;
        // offsets are stored in the pointers until the workspace is known
        p.scores = reinterpret_cast<float*>(o_scores);
        p.chunk_lb = reinterpret_cast<float*>(o_lb);
        p.chunk_kmax = reinterpret_cast<float*>(o_km);
        p.row_qn = reinterpret_cast<float*>(o_qn);
        p.lists = reinterpret_cast<uint32_t*>(o_lk);
        p.list_idx = reinterpret_cast<int32_t*>(o_li);
        p.list_cnt = reinterpret_cast<int32_t*>(o_lc);
        pl.lds_score = 4ull * p.chunk + 1024;
        // final kernel: LDS slots for every listed candidate of a row (parallel
        // path); the streaming fallback uses the first stream_cap of them
        p.stream_cap = p.cap;
        const long long fixed = 1024 + 16ll * p.mcap + 4ll * (p.nchunks + 1) + 16;
        const long long cap_fit = (kMaxLds - fixed) / 8;
        if (cap_fit < p.stream_cap)
            return fail(SHATTN_EUNSUPPORTED, "csa_index_topk: N=%d needs more LDS than available", N);
        p.cap = (int)std::min<long long>(12288, cap_fit / 64 * 64);
        if (p.cap < p.stream_cap) p.cap = p.stream_cap;
        pl.lds = (8ull * p.cap + (size_t)fixed + 15) / 16 * 16;
        pl.grid = rows;
        return SHATTN_OK;
    }
    const int qpt = 16 / Hi;
    if (N == 0) {
        // no candidates: every row is -1
        pl.empty = true;
        pl.grid = (rows * k + 255) / 256;
        return SHATTN_OK;
    }
    // Hi = 16 never takes the dense kernel (selection from LDS, N <= 2048):
    // that form at Hi = 16 is not covered by a passing GPU test (one build of
    // it took a memory fault whose cause was not found), so Hi = 16 always
    // takes the long pipeline below, whose kernels pass at Hi = 16.
    pl.dense = N <= kDenseMaxN && Hi != 16;
    if (pl.dense) {
        // p.cap = per-query key slots (N rounded up to a tile).  The band list is
        // short (an overflowing band falls back to the float32 order): the
        // workgroup's LDS stays small enough for four workgroups per CU.
        p.cap = (N + TILE - 1) / TILE * TILE;
        p.mcap = std::min(p.mcap, 64);
        auto dense_wave = [&](int q) { return (4ull * q * p.cap + 1024 + 12ull * p.mcap + 4ull * q + 15) / 16 * 16; };
        int qpw = 4 * qpt;
        while (qpw > qpt && WAVES * dense_wave(qpw) > (size_t)kMaxLds) qpw -= qpt;
        while (qpw > qpt && rows > 0 && (rows + (long long)WAVES * qpw - 1) / (WAVES * qpw) < 1024) qpw -= qpt;
        if (WAVES * dense_wave(qpw) > (size_t)kMaxLds) pl.dense = false;
        else {
            p.qpw = qpw;
            p.wave_stride = (int)dense_wave(qpw);
            p.nqt = (Tq + WAVES * qpw - 1) / (WAVES * qpw);
            pl.lds = WAVES * dense_wave(qpw);
            pl.grid = (long long)B * p.nqt;
            return SHATTN_OK;
        }
        p.cap = ((k + std::max(64, k / 2)) + 63) / 64 * 64;
    }
    // ---- long prefill pipeline
    pl.longp = true;
    // streaming fallback: queries per wave so that 4 waves fit the LDS budget
    {
        int qpw = std::max(16, qpt);
        if (qpw > 4 * qpt) qpw = 4 * qpt;
        auto per_wave = [&](int q) { return (8ull * q * p.cap + 1024 + 16ull * p.mcap + 4ull * q + 31) / 16 * 16; };
        while (qpw > qpt && WAVES * per_wave(qpw) > (size_t)kMaxLds) qpw -= qpt;
        if (WAVES * per_wave(qpw) > (size_t)kMaxLds)
            return fail(SHATTN_EUNSUPPORTED, "csa_index_topk: k=%d needs more LDS than available", k);
        while (qpw > qpt && rows > 0 && (rows + (long long)WAVES * qpw - 1) / (WAVES * qpw) < 512) qpw -= qpt;
        pl.lf.qpw = qpw;
        pl.lf.cap = p.cap;
        pl.lf.wave_stride = (int)per_wave(qpw);
        pl.lf.nqt = (Tq + WAVES * qpw - 1) / (WAVES * qpw);
        pl.lf.lds = WAVES * per_wave(qpw);
        pl.lf.grid = (long long)B * pl.lf.nqt;
    }
    // sampling pass: stride S (a power of two) with at most kSampleMax sampled
    // entries per query whose keys fit the dense kernel's LDS
    // (the sampling pass keeps no band list: its LDS is 16-bit keys,
    // histogram and query norms, and its launch runs with mcap = 0)
    auto sample_wave = [&](int q, int np) { return (2ull * q * np + 1024 + 4ull * q + 15) / 16 * 16; };
    int S = 1, np = 0;
    for (;; S *= 2) {
        np = ((N + S - 1) / S + TILE - 1) / TILE * TILE;
        if (np <= kSampleMax && WAVES * sample_wave(qpt, np) <= (size_t)kMaxLds) break;
    }
    {
        // one row tile per wave (the cooperative form: each key tile feeds the
        // four waves' row tiles) keeps the most workgroups per CU: at the 128K
        // CSA prefill two instead of one.  Hi = 16 keeps four row tiles per
        // wave (the form its tests cover).
        int qpw = Hi == 16 ? 4 * qpt : qpt;
        while (qpw > qpt && WAVES * sample_wave(qpw, np) > (size_t)kMaxLds) qpw -= qpt;
        pl.ls.qpw = qpw;
        pl.ls.cap = np;
        pl.ls.wave_stride = (int)sample_wave(qpw, np);
        pl.ls.nqt = (Tq + WAVES * qpw - 1) / (WAVES * qpw);
        pl.ls.lds = WAVES * sample_wave(qpw, np);
        pl.ls.grid = (long long)B * pl.ls.nqt;
    }
    // threshold rank j among the samples and list capacity: with r = k / S the
    // expected number of entries above the j-th sampled score is about j * S
    // (standard deviation about sqrt(j) * S); j = r + 5 sqrt(r) + 2 keeps it
    // above k, the capacity j * S + 7 sqrt(j) * S keeps the list from
    // overflowing, except on inputs with structure at the sampling period (those
    // rows fail over to the streaming kernel).
    const double r = (double)k / S;
    const int j = (int)std::ceil(r) + (int)std::ceil(5.0 * std::sqrt(r)) + 2;
    long long lcap = (long long)std::ceil(j * (double)S + 7.0 * std::sqrt((double)j) * S) + 64;
    // the list pass keeps a short band list (an overflowing band is decided
    // on float32 scores), so more of its one-wave workgroups share a CU
    p.list_mcap = std::min(p.mcap, 64);
    const long long lcap_fit = (kMaxLds - 1024 - 16ll * p.list_mcap - 16) / 4 / 64 * 64;
    lcap = std::min((lcap + 63) / 64 * 64, lcap_fit);
    p.sample_stride = S;
    p.sample_j = j;
    p.list_cap = (int)lcap;
    p.kblk = (N + kKmaxBlock - 1) / kKmaxBlock;
    const int frt = filter_row_tiles(dtype == SHATTN_DTYPE_F32, Hi, d_idx);
    const int qpw_f = frt * qpt;
    p.nqt = (Tq + WAVES * qpw_f - 1) / (WAVES * qpw_f);
    pl.grid_filter = (long long)B * p.nqt;
    pl.grid_kmax = (long long)B * p.kblk;
    pl.grid = rows;
    // the list pass holds lists of up to j S + 5.5 sqrt(j) S + 64 entries (the
    // mean length plus 5.5 standard deviations) in LDS; a longer list takes the
    // streaming kernel, whose one wave per such query then costs about a
    // millisecond, so the margin keeps that out of unstructured inputs.  At
    // the 128K CSA prefill (k 512, S 32, j 38) that is 2368 instead of 2688
    // entries, and 14 instead of 12 of the pass's one-wave workgroups fit a CU.
    long long kcap = (long long)std::ceil(j * (double)S + 5.5 * std::sqrt((double)j) * S) + 64;
    kcap = std::min((kcap + 63) / 64 * 64, lcap);
    p.list_lds_cap = (int)kcap;
    pl.lds = (4ull * kcap + 1024 + 16ull * p.list_mcap + 15) / 16 * 16;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
    const size_t o_km = take((size_t)B * p.kblk * 4);
    const size_t o_thr = take((size_t)rows * 4);
    const size_t o_tau = take((size_t)rows * 4);
    const size_t o_del = take((size_t)rows * 4);
    const size_t o_fail = take((size_t)rows * 4);
    const size_t o_cnt = take((size_t)rows * 4);
    const size_t o_lst = take((size_t)rows * lcap * 8);
    pl.ws_bytes = off;
    p.kmax_part = reinterpret_cast<float*>(o_km);
    p.row_thr = reinterpret_cast<uint32_t*>(o_thr);
    p.row_tau = reinterpret_cast<uint32_t*>(o_tau);
    p.row_delta = reinterpret_cast<float*>(o_del);
    p.row_fail = reinterpret_cast<int32_t*>(o_fail);
    p.list_cnt = reinterpret_cast<int32_t*>(o_cnt);
    p.row_lists = reinterpret_cast<uint2*>(o_lst);
    return SHATTN_OK;
}

int allow_lds(const void* kernel, size_t lds) {
    if (lds <= 64 * 1024) return SHATTN_OK;
    hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SHATTN_EUNSUPPORTED, "csa_index_topk: %zu bytes of LDS unavailable", lds);
    }
    return SHATTN_OK;
}

IdxParams with_launch(const IdxParams& p, const IdxLaunch& l) {
    IdxParams q = p;
    q.qpw = l.qpw;
    q.nqt = l.nqt;
    q.wave_stride = l.wave_stride;
    q.cap = l.cap;
    return q;
}

template <typename T, int HI, int DI>
int launch_idx(IdxPlan& pl, hipStream_t s) {
    int rc;
    if (pl.empty) {
        hipLaunchKernelGGL(index_fill_empty_kernel, dim3((unsigned)pl.grid), dim3(256), 0, s, pl.p);
        return check_launch("csa_index_topk (empty)");
    }
    if (pl.dense) {
        // the plan never gives Hi = 16 the dense form, and it is not compiled
        // for it (no passing GPU test covers it)
        if constexpr (HI == 16) {
            return fail(SHATTN_EUNSUPPORTED, "csa_index_topk: no dense selection form at Hi=16");
        } else {
            if ((rc = allow_lds(reinterpret_cast<const void*>(&index_dense_kernel<T, HI, DI, false>), pl.lds)))
                return rc;
            hipLaunchKernelGGL((index_dense_kernel<T, HI, DI, false>), dim3((unsigned)pl.grid), dim3(WAVES * 64),
                               pl.lds, s, pl.p);
            return check_launch("csa_index_topk");
        }
    }
    if (pl.longp) {
        hipLaunchKernelGGL((index_kmax_kernel<T, DI>), dim3((unsigned)pl.grid_kmax), dim3(256), 0, s, pl.p);
        if ((rc = check_launch("csa_index_topk (kmax)"))) return rc;
        if ((rc = allow_lds(reinterpret_cast<const void*>(&index_dense_kernel<T, HI, DI, true>), pl.ls.lds)))
            return rc;
        IdxParams ps = with_launch(pl.p, pl.ls);
        ps.mcap = 0;   // no band list in the sampling pass's LDS
        hipLaunchKernelGGL((index_dense_kernel<T, HI, DI, true>), dim3((unsigned)pl.ls.grid), dim3(WAVES * 64),
                           pl.ls.lds, s, ps);
        if ((rc = check_launch("csa_index_topk (sample)"))) return rc;
        hipLaunchKernelGGL((index_filter_kernel<T, HI, DI>), dim3((unsigned)pl.grid_filter), dim3(WAVES * 64), 0, s,
                           pl.p);
        if ((rc = check_launch("csa_index_topk (filter)"))) return rc;
        if ((rc = allow_lds(reinterpret_cast<const void*>(&index_list_final_kernel<T, HI, DI>), pl.lds))) return rc;
        hipLaunchKernelGGL((index_list_final_kernel<T, HI, DI>), dim3((unsigned)pl.grid), dim3(64), pl.lds, s, pl.p);
        if ((rc = check_launch("csa_index_topk (list final)"))) return rc;
        if ((rc = allow_lds(reinterpret_cast<const void*>(&index_prefill_kernel<T, HI, DI>), pl.lf.lds))) return rc;
        hipLaunchKernelGGL((index_prefill_kernel<T, HI, DI>), dim3((unsigned)pl.lf.grid), dim3(WAVES * 64),
                           pl.lf.lds, s, with_launch(pl.p, pl.lf));
        return check_launch("csa_index_topk (fallback)");
    }
    const long long rows = pl.grid;
    hipLaunchKernelGGL((index_split_score_kernel<T, HI, DI>), dim3((unsigned)(rows * pl.p.nchunks)), dim3(64),
                       pl.lds_score, s, pl.p);
    rc = check_launch("csa_index_topk (score)");
    if (rc) return rc;
    hipLaunchKernelGGL(index_split_collect_kernel, dim3((unsigned)(rows * pl.p.nchunks)), dim3(64), 0, s, pl.p);
    rc = check_launch("csa_index_topk (collect)");
    if (rc) return rc;
    if ((rc = allow_lds(reinterpret_cast<const void*>(&index_split_final_kernel<T, HI, DI>), pl.lds))) return rc;
    hipLaunchKernelGGL((index_split_final_kernel<T, HI, DI>), dim3((unsigned)rows), dim3(kFinalThreads), pl.lds, s,
                       pl.p);
    return check_launch("csa_index_topk (final)");
}

template <typename T, int HI>
int launch_idx_di(IdxPlan& pl, int d_idx, hipStream_t s) {
    return d_idx == 128 ? launch_idx<T, HI, 128>(pl, s) : launch_idx<T, HI, 64>(pl, s);
}
template <typename T>
int launch_idx_hi(IdxPlan& pl, int Hi, int d_idx, hipStream_t s) {
    switch (Hi) {
        case 1: return launch_idx_di<T, 1>(pl, d_idx, s);
        case 2: return launch_idx_di<T, 2>(pl, d_idx, s);
        case 4: return launch_idx_di<T, 4>(pl, d_idx, s);
        case 8: return launch_idx_di<T, 8>(pl, d_idx, s);
        default: return launch_idx_di<T, 16>(pl, d_idx, s);
    }
}

}  // namespace
}  // namespace shattn

using namespace shattn;

extern "C" size_t csa_index_topk_workspace_size(int B, int Tq, int N, int Hi, int d_idx, int k) {
    IdxPlan pl;
    // positions and ratio do not change the workspace size
    if (make_idx_plan(B, Tq, N, Hi, d_idx, 0, 1, 1, k, SHATTN_DTYPE_BF16, pl) != SHATTN_OK) return 0;
    return pl.ws_bytes;
}

static int index_topk_impl(const void* qI, const void* kI, const float* w, int32_t* idx, int B, int Tq, int N,
                           int Hi, int d_idx, int64_t q_pos0, const int64_t* q_pos, int m, int W, int k,
                           int dtype, void* ws, size_t ws_bytes, void* stream) {
    IdxPlan pl;
    int rc = make_idx_plan(B, Tq, N, Hi, d_idx, q_pos0, m, W, k, dtype, pl);
    if (rc != SHATTN_OK) return rc;
    if (B == 0 || Tq == 0) return SHATTN_OK;
    if (!qI || !w || !idx || (N > 0 && !kI)) return fail(SHATTN_EINVAL, "csa_index_topk: null pointer");
    if (q_pos && (reinterpret_cast<uintptr_t>(q_pos) & 7))
        return fail(SHATTN_EINVAL, "csa_index_topk_varlen: q_pos must be 8-byte aligned");
    pl.p.q_pos = q_pos;
    if (!aligned16(qI) || (N > 0 && !aligned16(kI)) || (reinterpret_cast<uintptr_t>(w) & 3) ||
        (reinterpret_cast<uintptr_t>(idx) & 3))
        return fail(SHATTN_EINVAL, "csa_index_topk: qI/kI must be 16-byte aligned, w/idx 4-byte aligned");
    if (pl.ws_bytes > 0) {
        if (!ws || ws_bytes < pl.ws_bytes)
            return fail(SHATTN_EWORKSPACE, "csa_index_topk: workspace of %zu bytes needed, %zu given", pl.ws_bytes,
                        ws ? ws_bytes : (size_t)0);
        if (reinterpret_cast<uintptr_t>(ws) & 255)
            return fail(SHATTN_EINVAL, "csa_index_topk: workspace must be 256-byte aligned");
        char* base = reinterpret_cast<char*>(ws);
        IdxParams& p = pl.p;
        auto at = [&](auto* off) { return reinterpret_cast<decltype(off)>(base + reinterpret_cast<size_t>(off)); };
        if (pl.split) {
            p.scores = at(p.scores);
            p.chunk_lb = at(p.chunk_lb);
            p.chunk_kmax = at(p.chunk_kmax);
            p.row_qn = at(p.row_qn);
        } else {
            p.kmax_part = at(p.kmax_part);
            p.row_thr = at(p.row_thr);
            p.row_tau = at(p.row_tau);
            p.row_delta = at(p.row_delta);
            p.row_fail = at(p.row_fail);
            p.row_lists = at(p.row_lists);
        }
        if (pl.split) {
            p.lists = at(p.lists);
            p.list_idx = at(p.list_idx);
        }
        p.list_cnt = at(p.list_cnt);
    }
    pl.p.qI = qI;
    pl.p.kI = kI;
    pl.p.w = w;
    pl.p.idx = idx;
    if (pl.grid > 2147483647LL / 64 || pl.ls.grid > 2147483647LL / 64 || pl.lf.grid > 2147483647LL / 64 ||
        pl.grid_kmax > 2147483647LL)
        return fail(SHATTN_EUNSUPPORTED, "csa_index_topk: problem too large");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return dtype == SHATTN_DTYPE_BF16 ? launch_idx_hi<bf16_t>(pl, Hi, d_idx, s)
                                      : launch_idx_hi<float>(pl, Hi, d_idx, s);
}

extern "C" int csa_index_topk(const void* qI, const void* kI, const float* w, int32_t* idx, int B, int Tq,
                              int N, int Hi, int d_idx, int64_t q_pos0, int m, int W, int k, int dtype,
                              void* ws, size_t ws_bytes, void* stream) {
    return index_topk_impl(qI, kI, w, idx, B, Tq, N, Hi, d_idx, q_pos0, nullptr, m, W, k, dtype, ws, ws_bytes,
                           stream);
}

extern "C" int csa_index_topk_varlen(const void* qI, const void* kI, const float* w, int32_t* idx, int B, int Tq,
                                     int N, int Hi, int d_idx, const int64_t* q_pos, int m, int W, int k,
                                     int dtype, void* ws, size_t ws_bytes, void* stream) {
    if (!q_pos && B > 0 && Tq > 0) return fail(SHATTN_EINVAL, "csa_index_topk_varlen: null q_pos");
    return index_topk_impl(qI, kI, w, idx, B, Tq, N, Hi, d_idx, 0, q_pos, m, W, k, dtype, ws, ws_bytes, stream);
}
