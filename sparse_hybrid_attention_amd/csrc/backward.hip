// Backward pass of the hybrid (HCA / CSA / SWA) attention path over a prefill
// on gfx950: gradients of the gated attention output with respect to Q, the
// raw K/V rows, the compression logits of both ratios and the gates.
//
// Method: the derivative of the forward definitions (the block merge of
// [V4-code] section 1; one softmax per branch over {window} and {HCA entries
// or selected CSA entries}, [V4-blog] "1. hybrid attn"; the per-head / per-
// token branch gate of [Tiny-R2] 3.1.2 / 3.2).  The CSA selection is a fixed
// input (a top-k has no derivative) and the storage rounding of the
// compressed caches is taken as the identity.
//
// With O_b the output of branch b, w_b its gate weight and dOut the incoming
// gradient, branch b sees dO_b = w_b dOut.  For a query row and key j of a
// branch's set, with s_j the scaled logit, P_bj = exp(s_j - LSE_b),
// dpo_j = dOut . v_j and D_b = dOut . O_b (which is also dL/dw_b):
//   dS_j = sum over the branches holding j of w_b P_bj (dpo_j - D_b)
//   dq  += scale dS_j k_j,  dk_j += scale dS_j q,  dv_j += (sum_b w_b P_bj) dOut.
// Window keys belong to every branch present; HCA entries to the HCA branch;
// selected CSA entries to the CSA branch.
//
// Kernels (float32 arithmetic; four lanes per row, each holding a quarter of
// the head dim, so a dot product is four partial sums and two in-register
// exchanges; a wave holds 16 rows and walks the union of their key or query
// sets in lockstep, masking per row):
//   1. query side: per (row, head) one pass for LSE_b and D_b (an online
//      softmax carrying a scalar accumulator of dpo), a second for dq;
//   2. block weights P = softmax(z) of every compression logit tensor;
//   3. key side, compressed entries: HCA entries over the query rows that see
//      them, CSA entries over the rows whose selection holds them (found with
//      one coalesced read of the row's selection and a wave-wide OR);
//   4. key side, raw rows over their window band, plus the compressed-cache
//      gradients routed back through the block merge (dx = P_i dxc);
//   5. logit gradients: dP_i = sum over blocks of dxc . x_i as per-chunk
//      partials, then dz_i = P_i (dP_i - sum_l P_l dP_l) summing the partials
//      in a fixed order;
//   6. gate gradients (per head: a fixed-order sum over rows).
// No floating-point atomics: every output element is written by one thread
// in a fixed order, so results are deterministic.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/hybrid_attn.h"
#include "common.h"

namespace shattn {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 16;                 // four lanes per row
constexpr int kRowsPerGroup = kRowsPerWave * 4;  // four waves
constexpr int kDpChunk = 32;                     // blocks per dP partial sum

// one compression whose logits get a gradient: x are the raw rows (K or V),
// dxc the cache gradient, z the logits, pz the block weights, dz the result
struct ZJob {
    const void* x;
    const float* dxc;
    const float* z;
    float* pz;
    float* dp;
    float* dz;
    int m, N, nchunk;
};

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const void* k_hca;
    const void* v_hca;
    const void* k_csa;
    const void* v_csa;
    const int32_t* idx;
    const float* gates;
    float* dq;
    float* dk;
    float* dv;
    float* dgates;
    float* stats;      // [B, T, H, 6]: LSE_b (log2 domain) for b = HCA, CSA, SWA, then D_b
    float* dkc_hca;    // [B, N_hca, Hkv, d] cache gradients
    float* dvc_hca;
    float* dkc_csa;    // [B, N_csa, Hkv, d]
    float* dvc_csa;
    ZJob z[4];         // zk_hca, zv_hca (HCA present), then zk_csa, zv_csa (CSA present)
    int nz;
    int B, T, H, Hkv, G, W, gate_mode;
    int m_hca, N_hca, m_csa, N_csa, ksel;
    int has_hca, has_csa;
    float scale;       // softmax scale
    float scale_log2;  // scale * log2(e)
};

// this lane's quarter of a row (D / 4 elements, from element part * D / 4)
template <typename T, int D> __device__ __forceinline__ void load_part(const T* row, int part, float* out) {
    constexpr int NP = D / 4;
    constexpr int V = Elem<T>::kVec;
    const T* p = row + part * NP;
#pragma unroll
    for (int u = 0; u < NP / V; ++u) Elem<T>::unpack(ld16(p + u * V), out + u * V);
}

// sum over the four lanes of a row, the same value on all four: (l0 + l1) + (l2 + l3)
__device__ __forceinline__ float quad_sum(float v) {
    v += __uint_as_float(dpp_mov<0xB1>(__float_as_uint(v)));   // lane ^ 1
    v += __uint_as_float(dpp_mov<0x4E>(__float_as_uint(v)));   // lane ^ 2
    return v;
}

template <int NP> __device__ __forceinline__ float dot_part(const float* a, const float* b) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < NP; ++e) s = fmaf(a[e], b[e], s);
    return s;
}

// entries of ratio m wholly before the window of the query at t
__device__ __forceinline__ int n_visible(int t, int W, int m, int N) {
    const int s = t - W + 1;
    if (s <= 0) return 0;
    const int n = s / m;
    return n < N ? n : N;
}

// gate weights [HCA, CSA, SWA] of (b, t, h)
__device__ __forceinline__ void gate_w(const BwdParams& p, int b, int t, int h, float* g) {
    const float* src = p.gate_mode == 0 ? p.gates + h * 3 : p.gates + (((long long)b * p.T + t) * p.H + h) * 3;
    g[0] = src[0];
    g[1] = src[1];
    g[2] = src[2];
    if (p.gate_mode == 2) {
        const float mx = fmaxf(g[0], fmaxf(g[1], g[2]));
        const float e0 = expf(g[0] - mx), e1 = expf(g[1] - mx), e2 = expf(g[2] - mx);
        const float inv = 1.0f / (e0 + e1 + e2);
        g[0] = e0 * inv;
        g[1] = e1 * inv;
        g[2] = e2 * inv;
    }
}

__device__ __forceinline__ uint32_t branch_mask_window(const BwdParams& p) {
    return 4u | (p.has_hca ? 1u : 0u) | (p.has_csa ? 2u : 0u);
}

// ------------------------------------------------------------ 1. query side
// Workgroup: 64 consecutive rows of one (sequence, head); a wave takes 16.
// The wave walks the union of its rows' windows, the HCA entries visible to
// its last row and the CSA selections column by column, every key masked per
// row.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_query_kernel(BwdParams p) {
    constexpr int NP = D / 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int part = lane & 3, ri = lane >> 2;
    const int ntile = (p.T + kRowsPerGroup - 1) / kRowsPerGroup;
    const int work = (int)xcd_work_id(blockIdx.x, gridDim.x);
    const int tile = work % ntile;
    const int h = (work / ntile) % p.H;
    const int b = work / (ntile * p.H);
    const int g = h / p.G;
    const int ta = tile * kRowsPerGroup + wave * kRowsPerWave;
    if (ta >= p.T) return;
    const int tb = min(ta + kRowsPerWave - 1, p.T - 1);
    const int t = min(ta + ri, tb);
    const bool valid = ta + ri <= tb;
    const int rs = p.Hkv * D;
    const long long qoff = (((long long)b * p.T + t) * p.H + h) * D;
    float qv[NP], ov[NP];
    load_part<T, D>(reinterpret_cast<const T*>(p.q) + qoff, part, qv);
    load_part<T, D>(reinterpret_cast<const T*>(p.dout) + qoff, part, ov);
    float gw[3];
    gate_w(p, b, t, h, gw);
    const T* kraw = reinterpret_cast<const T*>(p.k) + (long long)b * p.T * rs + g * D;
    const T* vraw = reinterpret_cast<const T*>(p.v) + (long long)b * p.T * rs + g * D;
    const T* khca = reinterpret_cast<const T*>(p.k_hca) + (long long)b * p.N_hca * rs + g * D;
    const T* vhca = reinterpret_cast<const T*>(p.v_hca) + (long long)b * p.N_hca * rs + g * D;
    const T* kcsa = reinterpret_cast<const T*>(p.k_csa) + (long long)b * p.N_csa * rs + g * D;
    const T* vcsa = reinterpret_cast<const T*>(p.v_csa) + (long long)b * p.N_csa * rs + g * D;
    const int32_t* sel = p.idx + ((long long)b * p.T + t) * p.ksel;
    const int w_lo = max(0, ta - p.W + 1);
    const int my_lo = t - p.W + 1;
    const int nh_max = p.has_hca ? n_visible(tb, p.W, p.m_hca, p.N_hca) : 0;
    const int nh = p.has_hca ? n_visible(t, p.W, p.m_hca, p.N_hca) : 0;
    const int nc = p.has_csa ? n_visible(t, p.W, p.m_csa, p.N_csa) : 0;
    const int nsel = p.has_csa ? p.ksel : 0;
    const uint32_t win_mask = branch_mask_window(p);
    // every key of the wave's sets: f(this row's branch bits, k row, v row)
    auto visit = [&](auto&& f) {
        for (int j = w_lo; j <= tb; ++j) {
            const uint32_t mb = (valid && j >= my_lo && j <= t) ? win_mask : 0u;
            f(mb, kraw + (long long)j * rs, vraw + (long long)j * rs);
        }
        for (int c = 0; c < nh_max; ++c) {
            const uint32_t mb = (valid && c < nh) ? 1u : 0u;
            f(mb, khca + (long long)c * rs, vhca + (long long)c * rs);
        }
        for (int jj = 0; jj < nsel; ++jj) {
            const int e = sel[jj];
            const bool ok = valid && e >= 0 && e < nc;
            // a column no row of the wave can use reads nothing (the cache may
            // be empty); otherwise row 0 exists and stands in for unused lanes
            if (!__any(ok)) continue;
            const long long r = (long long)(ok ? e : 0) * rs;
            f(ok ? 2u : 0u, kcsa + r, vcsa + r);
        }
    };
    // pass 1: per branch LSE (log2 domain) and D_b = sum_j P_bj dpo_j, online
    float mx[3] = {-INFINITY, -INFINITY, -INFINITY}, sm[3] = {0.f, 0.f, 0.f}, ac[3] = {0.f, 0.f, 0.f};
    visit([&](uint32_t mb, const T* kr, const T* vr) {
        float kv[NP], vv[NP];
        load_part<T, D>(kr, part, kv);
        load_part<T, D>(vr, part, vv);
        const float s2 = quad_sum(dot_part<NP>(qv, kv)) * p.scale_log2;
        const float dpo = quad_sum(dot_part<NP>(ov, vv));
#pragma unroll
        for (int br = 0; br < 3; ++br) {
            if (!(mb & (1u << br))) continue;
            const float mn = fmaxf(mx[br], s2);
            const float a = exp2f(mx[br] - mn), e = exp2f(s2 - mn);
            sm[br] = fmaf(sm[br], a, e);
            ac[br] = fmaf(ac[br], a, e * dpo);
            mx[br] = mn;
        }
    });
    float lse[3], Db[3];
#pragma unroll
    for (int br = 0; br < 3; ++br) {
        const bool any = sm[br] > 0.f;
        lse[br] = any ? mx[br] + log2f(sm[br]) : 0.f;
        Db[br] = any ? ac[br] / sm[br] : 0.f;
    }
    if (valid && part == 0) {
        float* st = p.stats + (((long long)b * p.T + t) * p.H + h) * 6;
#pragma unroll
        for (int br = 0; br < 3; ++br) {
            st[br] = lse[br];
            st[3 + br] = Db[br];
        }
    }
    // pass 2: dS_j and dq
    float dqv[NP];
#pragma unroll
    for (int e = 0; e < NP; ++e) dqv[e] = 0.f;
    visit([&](uint32_t mb, const T* kr, const T* vr) {
        float kv[NP], vv[NP];
        load_part<T, D>(kr, part, kv);
        load_part<T, D>(vr, part, vv);
        const float s2 = quad_sum(dot_part<NP>(qv, kv)) * p.scale_log2;
        const float dpo = quad_sum(dot_part<NP>(ov, vv));
        float ds = 0.f;
#pragma unroll
        for (int br = 0; br < 3; ++br)
            if (mb & (1u << br)) ds = fmaf(gw[br] * exp2f(s2 - lse[br]), dpo - Db[br], ds);
#pragma unroll
        for (int e = 0; e < NP; ++e) dqv[e] = fmaf(ds, kv[e], dqv[e]);
    });
    if (!valid) return;
    float* dst = p.dq + qoff + part * NP;
#pragma unroll
    for (int e = 0; e < NP; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            make_float4(p.scale * dqv[e], p.scale * dqv[e + 1], p.scale * dqv[e + 2], p.scale * dqv[e + 3]);
}

// ------------------------------------------------------------ 2. block weights
// pz[i, ch] = softmax over i < m of z[i, ch] (one thread per channel; blockIdx.y = job)
__global__ __launch_bounds__(kThreads) void bwd_weights_kernel(BwdParams p, int nch) {
    const ZJob& J = p.z[blockIdx.y];
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= nch) return;
    float mx = -INFINITY;
    for (int i = 0; i < J.m; ++i) mx = fmaxf(mx, J.z[(long long)i * nch + c]);
    float s = 0.f;
    for (int i = 0; i < J.m; ++i) s += expf(J.z[(long long)i * nch + c] - mx);
    const float inv = 1.0f / s;
    for (int i = 0; i < J.m; ++i) J.pz[(long long)i * nch + c] = expf(J.z[(long long)i * nch + c] - mx) * inv;
}

// ------------------------------------------------------------ 3./4. key side
// KIND 0: raw rows (window keys of every present branch; queries t in
// [j, j + W - 1]), then the cache gradients routed through the block merge;
// 1: HCA entries (HCA branch; queries t >= (c+1) m + W - 1);
// 2: CSA entries (CSA branch; the visible queries whose selection holds c).
// Workgroup: 64 consecutive keys of one (sequence, KV head); a wave takes 16,
// walking the union of their query ranges in lockstep, G heads per row.
template <typename T, int D, int KIND>
__global__ __launch_bounds__(kThreads) void bwd_key_kernel(BwdParams p) {
    constexpr int NP = D / 4;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int part = lane & 3, ri = lane >> 2;
    const int nkeys = KIND == 0 ? p.T : (KIND == 1 ? p.N_hca : p.N_csa);
    const int ntile = (nkeys + kRowsPerGroup - 1) / kRowsPerGroup;
    const int work = (int)xcd_work_id(blockIdx.x, gridDim.x);
    const int tile = work % ntile;
    const int g = (work / ntile) % p.Hkv;
    const int b = work / (ntile * p.Hkv);
    const int ja = tile * kRowsPerGroup + wave * kRowsPerWave;
    if (ja >= nkeys) return;
    const int jb = min(ja + kRowsPerWave - 1, nkeys - 1);
    const int j = min(ja + ri, jb);
    const bool valid = ja + ri <= jb;
    const int rs = p.Hkv * D;
    const T* kbase = reinterpret_cast<const T*>(KIND == 0 ? p.k : (KIND == 1 ? p.k_hca : p.k_csa));
    const T* vbase = reinterpret_cast<const T*>(KIND == 0 ? p.v : (KIND == 1 ? p.v_hca : p.v_csa));
    const long long krow = ((long long)b * nkeys + j) * rs + g * D;
    float kv[NP], vv[NP];
    load_part<T, D>(kbase + krow, part, kv);
    load_part<T, D>(vbase + krow, part, vv);
    const int m = KIND == 1 ? p.m_hca : p.m_csa;
    auto first_t = [&](int key) { return KIND == 0 ? key : (key + 1) * m + p.W - 1; };
    const int t_lo = first_t(ja);
    const int t_hi = KIND == 0 ? min(jb + p.W - 1, p.T - 1) : p.T - 1;
    const int my_first = first_t(j);
    const int my_last = KIND == 0 ? j + p.W - 1 : p.T - 1;
    const uint32_t bmask = KIND == 0 ? branch_mask_window(p) : (KIND == 1 ? 1u : 2u);
    float dkv[NP], dvv[NP];
#pragma unroll
    for (int e = 0; e < NP; ++e) {
        dkv[e] = 0.f;
        dvv[e] = 0.f;
    }
    for (int t = t_lo; t <= t_hi; ++t) {
        bool in = valid && t >= my_first && t <= my_last;
        if (KIND == 2) {
            // which of the wave's 16 entries row t selects: one selection
            // element per lane, OR over the wave
            const int32_t* sel = p.idx + ((long long)b * p.T + t) * p.ksel;
            uint32_t bits = 0u;
            for (int c0 = 0; c0 < p.ksel; c0 += 64) {
                const int e = c0 + lane < p.ksel ? sel[c0 + lane] : -1;
                if (e >= ja && e <= jb) bits |= 1u << (e - ja);
            }
            bits = wave_allreduce(bits, [](uint32_t a, uint32_t c) { return a | c; });
            in = in && ((bits >> ri) & 1u);
        }
        if (!__any(in)) continue;
        for (int hh = 0; hh < p.G; ++hh) {
            const int h = g * p.G + hh;
            const long long qoff = (((long long)b * p.T + t) * p.H + h) * D;
            float qv[NP], ov[NP];
            load_part<T, D>(reinterpret_cast<const T*>(p.q) + qoff, part, qv);
            load_part<T, D>(reinterpret_cast<const T*>(p.dout) + qoff, part, ov);
            const float* st = p.stats + (((long long)b * p.T + t) * p.H + h) * 6;
            float gw[3];
            gate_w(p, b, t, h, gw);
            const float s2 = quad_sum(dot_part<NP>(qv, kv)) * p.scale_log2;
            const float dpo = quad_sum(dot_part<NP>(ov, vv));
            float wsum = 0.f, ds = 0.f;
#pragma unroll
            for (int br = 0; br < 3; ++br) {
                if (!(bmask & (1u << br))) continue;
                const float pw = gw[br] * exp2f(s2 - st[br]);
                wsum += pw;
                ds = fmaf(pw, dpo - st[3 + br], ds);
            }
            if (!in) {
                wsum = 0.f;
                ds = 0.f;
            }
#pragma unroll
            for (int e = 0; e < NP; ++e) {
                dkv[e] = fmaf(ds, qv[e], dkv[e]);
                dvv[e] = fmaf(wsum, ov[e], dvv[e]);
            }
        }
    }
    if (!valid) return;
#pragma unroll
    for (int e = 0; e < NP; ++e) dkv[e] *= p.scale;
    if (KIND == 0) {
        // raw row j also feeds block j / m of each compression (full blocks only)
        const int nch = p.Hkv * D;
        const int ch0 = g * D + part * NP;
#pragma unroll
        for (int which = 0; which < 2; ++which) {
            const bool present = which == 0 ? p.has_hca : p.has_csa;
            if (!present) continue;
            const int mm = which == 0 ? p.m_hca : p.m_csa;
            const int N = which == 0 ? p.N_hca : p.N_csa;
            const int blk = j / mm;
            if (blk >= N) continue;
            const int i = j - blk * mm;
            const int zk = which == 0 ? 0 : (p.has_hca ? 2 : 0);
            const ZJob& Jk = p.z[zk];
            const ZJob& Jv = p.z[zk + 1];
            const long long co = ((long long)b * N + blk) * nch + ch0;
            const float* pk = Jk.pz + (long long)i * nch + ch0;
            const float* pv = Jv.pz + (long long)i * nch + ch0;
#pragma unroll
            for (int e = 0; e < NP; ++e) {
                dkv[e] = fmaf(pk[e], Jk.dxc[co + e], dkv[e]);
                dvv[e] = fmaf(pv[e], Jv.dxc[co + e], dvv[e]);
            }
        }
    }
    float* dk = KIND == 0 ? p.dk : (KIND == 1 ? p.dkc_hca : p.dkc_csa);
    float* dv = KIND == 0 ? p.dv : (KIND == 1 ? p.dvc_hca : p.dvc_csa);
    const long long o = krow + part * NP;
#pragma unroll
    for (int e = 0; e < NP; e += 4) {
        *reinterpret_cast<float4*>(dk + o + e) = make_float4(dkv[e], dkv[e + 1], dkv[e + 2], dkv[e + 3]);
        *reinterpret_cast<float4*>(dv + o + e) = make_float4(dvv[e], dvv[e + 1], dvv[e + 2], dvv[e + 3]);
    }
}

// ------------------------------------------------------------ 5. logit gradients
// dp[b, chunk, i, ch] = sum over the chunk's blocks c of dxc[b, c, ch] x[b, c m + i, ch]
// (one thread per (b, chunk, i, ch); blockIdx.y = job)
template <typename T>
__global__ __launch_bounds__(kThreads) void bwd_dp_kernel(BwdParams p, int nch) {
    const ZJob& J = p.z[blockIdx.y];
    const long long per_chunk = (long long)J.m * nch;
    const long long total = (long long)p.B * J.nchunk * per_chunk;
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    if (gid >= total) return;
    const long long bc = gid / per_chunk;
    const long long r = gid - bc * per_chunk;
    const int b = (int)(bc / J.nchunk), chunk = (int)(bc - (long long)b * J.nchunk);
    const int i = (int)(r / nch), c = (int)(r - (long long)i * nch);
    const T* x = reinterpret_cast<const T*>(J.x);
    const int c_end = min(J.N, (chunk + 1) * kDpChunk);
    float s = 0.f;
    for (int blk = chunk * kDpChunk; blk < c_end; ++blk)
        s = fmaf(J.dxc[((long long)b * J.N + blk) * nch + c],
                 Elem<T>::load1(x + ((long long)b * p.T + (long long)blk * J.m + i) * nch + c), s);
    J.dp[gid] = s;
}

// dz[i, ch] = P_i (dP_i - sum_l P_l dP_l); dP_i = sum over (b, chunk) in
// order (one thread per channel; blockIdx.y = job).  dz holds dP_i between
// the two loops.
__global__ __launch_bounds__(kThreads) void bwd_dz_kernel(BwdParams p, int nch) {
    const ZJob& J = p.z[blockIdx.y];
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= nch) return;
    const long long per_chunk = (long long)J.m * nch;
    const int nbc = p.B * J.nchunk;
    float cen = 0.f;
    for (int i = 0; i < J.m; ++i) {
        float dp = 0.f;
        for (int bc = 0; bc < nbc; ++bc) dp += J.dp[bc * per_chunk + (long long)i * nch + c];
        J.dz[(long long)i * nch + c] = dp;
        cen = fmaf(J.pz[(long long)i * nch + c], dp, cen);
    }
    for (int i = 0; i < J.m; ++i) {
        const long long o = (long long)i * nch + c;
        J.dz[o] = J.pz[o] * (J.dz[o] - cen);
    }
}

// ------------------------------------------------------------ 6. gates
// per head (mode 0): dgates[h, br] = sum over rows of D_br, a strided sum per
// thread then a fixed tree over the workgroup (one workgroup per (h, br))
__global__ __launch_bounds__(kThreads) void bwd_gate_head_kernel(BwdParams p) {
    __shared__ float red[kThreads];
    const int h = blockIdx.x / 3, br = blockIdx.x % 3;
    const long long rows = (long long)p.B * p.T;
    float s = 0.f;
    for (long long r = threadIdx.x; r < rows; r += kThreads) s += p.stats[(r * p.H + h) * 6 + 3 + br];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) p.dgates[h * 3 + br] = red[0];
}

// per token: weights (mode 1) take D_br; logits (mode 2) go through the
// branch softmax, dlogit = w (D - sum w D)
__global__ __launch_bounds__(kThreads) void bwd_gate_token_kernel(BwdParams p) {
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long n = (long long)p.B * p.T * p.H;
    if (gid >= n) return;
    const float* st = p.stats + gid * 6 + 3;
    float* dst = p.dgates + gid * 3;
    if (p.gate_mode == 1) {
        dst[0] = st[0];
        dst[1] = st[1];
        dst[2] = st[2];
        return;
    }
    const int h = (int)(gid % p.H);
    const long long bt = gid / p.H;
    float w[3];
    gate_w(p, (int)(bt / p.T), (int)(bt % p.T), h, w);
    const float c = fmaf(w[0], st[0], fmaf(w[1], st[1], w[2] * st[2]));
    dst[0] = w[0] * (st[0] - c);
    dst[1] = w[1] * (st[1] - c);
    dst[2] = w[2] * (st[2] - c);
}

// ------------------------------------------------------------ host side
struct BwdPlan {
    size_t off_stats, off_dkc_hca, off_dvc_hca, off_dkc_csa, off_dvc_csa, off_pz[4], off_dp[4];
    size_t bytes;
    int N_hca, N_csa;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int bwd_validate(const shattn_bwd_args* a) {
    if (!a) return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: null argument struct");
    if (a->struct_size != (int)sizeof(shattn_bwd_args))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: struct_size %d != %d", a->struct_size,
                    (int)sizeof(shattn_bwd_args));
    if (a->dtype != SHATTN_DTYPE_BF16 && a->dtype != SHATTN_DTYPE_F32)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: unknown dtype %d", a->dtype);
    if (a->B < 0 || a->T < 0 || a->H < 1 || a->Hkv < 1 || a->W < 1 || a->H % a->Hkv || a->m_hca < 0 ||
        a->m_csa < 0 || a->k < 0 || a->reserved0 != 0)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: bad sizes B=%d T=%d H=%d Hkv=%d W=%d m_hca=%d "
                    "m_csa=%d k=%d", a->B, a->T, a->H, a->Hkv, a->W, a->m_hca, a->m_csa, a->k);
    if (a->d != 64 && a->d != 128)
        return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_bwd: d=%d (supported: 64, 128)", a->d);
    if (a->gate_mode < 0 || a->gate_mode > 2)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: gate_mode %d", a->gate_mode);
    if (a->k > 0 && a->m_csa < 1)
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: CSA branch (k=%d) needs m_csa >= 1", a->k);
    if (a->m_hca > 1024 || a->m_csa > 1024)
        return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_bwd: ratio above 1024");
    if (!(a->sm_scale >= 0.f) || !std::isfinite(a->sm_scale))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: sm_scale must be finite and >= 0");
    if ((long long)a->B * a->T * a->H > (1LL << 31) - 1 || (long long)a->T + a->W > (1LL << 30))
        return fail(SHATTN_EUNSUPPORTED, "hybrid_sparse_attn_bwd: problem too large");
    const bool hca = a->m_hca > 0, csa = a->k > 0;
    const bool rows = (long long)a->B * a->T > 0;
    if (!a->gates || !a->dgates || (rows && (!a->q || !a->k_raw || !a->v_raw || !a->dout || !a->dq || !a->dk ||
                                             !a->dv)))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: null pointer");
    if (hca && (!a->zk_hca || !a->zv_hca || !a->dzk_hca || !a->dzv_hca ||
                ((long long)a->B * (a->T / a->m_hca) > 0 && (!a->k_hca || !a->v_hca))))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: null HCA pointer");
    if (csa && (!a->zk_csa || !a->zv_csa || !a->dzk_csa || !a->dzv_csa ||
                ((long long)a->B * (a->T / a->m_csa) > 0 && (!a->k_csa || !a->v_csa)) || (rows && !a->idx)))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: null CSA pointer");
    const void* al[] = {a->q, a->k_raw, a->v_raw, a->dout, a->dq, a->dk, a->dv,
                        hca ? a->k_hca : nullptr, hca ? a->v_hca : nullptr, csa ? a->k_csa : nullptr,
                        csa ? a->v_csa : nullptr, a->dk_hca, a->dv_hca, a->dk_csa, a->dv_csa};
    for (const void* ptr : al)
        if (!aligned16(ptr)) return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: tensors must be 16-byte aligned");
    const uintptr_t small = reinterpret_cast<uintptr_t>(a->gates) | reinterpret_cast<uintptr_t>(a->dgates) |
                            reinterpret_cast<uintptr_t>(csa ? a->idx : nullptr) |
                            reinterpret_cast<uintptr_t>(hca ? a->zk_hca : nullptr) |
                            reinterpret_cast<uintptr_t>(hca ? a->zv_hca : nullptr) |
                            reinterpret_cast<uintptr_t>(hca ? a->dzk_hca : nullptr) |
                            reinterpret_cast<uintptr_t>(hca ? a->dzv_hca : nullptr) |
                            reinterpret_cast<uintptr_t>(csa ? a->zk_csa : nullptr) |
                            reinterpret_cast<uintptr_t>(csa ? a->zv_csa : nullptr) |
                            reinterpret_cast<uintptr_t>(csa ? a->dzk_csa : nullptr) |
                            reinterpret_cast<uintptr_t>(csa ? a->dzv_csa : nullptr);
    if (small & 3u) return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: float32 / int32 operands must be 4-byte aligned");
    return SHATTN_OK;
}

BwdPlan bwd_plan(const shattn_bwd_args* a) {
    BwdPlan pl{};
    const bool hca = a->m_hca > 0, csa = a->k > 0;
    pl.N_hca = hca ? a->T / a->m_hca : 0;
    pl.N_csa = csa ? a->T / a->m_csa : 0;
    const size_t nch = (size_t)a->Hkv * a->d;
    size_t off = 0;
    auto take = [&](size_t floats) {
        const size_t o = off;
        off += align256(floats * sizeof(float));
        return o;
    };
    pl.off_stats = take((size_t)a->B * a->T * a->H * 6);
    pl.off_dkc_hca = take(a->dk_hca ? 0 : (size_t)a->B * pl.N_hca * nch);
    pl.off_dvc_hca = take(a->dv_hca ? 0 : (size_t)a->B * pl.N_hca * nch);
    pl.off_dkc_csa = take(a->dk_csa ? 0 : (size_t)a->B * pl.N_csa * nch);
    pl.off_dvc_csa = take(a->dv_csa ? 0 : (size_t)a->B * pl.N_csa * nch);
    for (int jb = 0; jb < 4; ++jb) {
        const bool present = jb < 2 ? hca : csa;
        const int m = jb < 2 ? a->m_hca : a->m_csa;
        const int N = jb < 2 ? pl.N_hca : pl.N_csa;
        const int nchunk = N > 0 ? (N + kDpChunk - 1) / kDpChunk : 1;
        pl.off_pz[jb] = take(present ? (size_t)m * nch : 0);
        pl.off_dp[jb] = take(present ? (size_t)a->B * nchunk * m * nch : 0);
    }
    pl.bytes = off;
    return pl;
}

template <typename T, int D> int bwd_launch(const shattn_bwd_args* a, const BwdPlan& pl, char* ws, hipStream_t s) {
    BwdParams p{};
    const bool hca = a->m_hca > 0, csa = a->k > 0;
    p.q = a->q;
    p.k = a->k_raw;
    p.v = a->v_raw;
    p.dout = a->dout;
    p.k_hca = a->k_hca;
    p.v_hca = a->v_hca;
    p.k_csa = a->k_csa;
    p.v_csa = a->v_csa;
    p.idx = a->idx;
    p.gates = a->gates;
    p.dq = a->dq;
    p.dk = a->dk;
    p.dv = a->dv;
    p.dgates = a->dgates;
    p.stats = reinterpret_cast<float*>(ws + pl.off_stats);
    p.dkc_hca = a->dk_hca ? a->dk_hca : reinterpret_cast<float*>(ws + pl.off_dkc_hca);
    p.dvc_hca = a->dv_hca ? a->dv_hca : reinterpret_cast<float*>(ws + pl.off_dvc_hca);
    p.dkc_csa = a->dk_csa ? a->dk_csa : reinterpret_cast<float*>(ws + pl.off_dkc_csa);
    p.dvc_csa = a->dv_csa ? a->dv_csa : reinterpret_cast<float*>(ws + pl.off_dvc_csa);
    p.B = a->B;
    p.T = a->T;
    p.H = a->H;
    p.Hkv = a->Hkv;
    p.G = a->H / a->Hkv;
    p.W = a->W;
    p.gate_mode = a->gate_mode;
    p.m_hca = a->m_hca;
    p.N_hca = pl.N_hca;
    p.m_csa = a->m_csa;
    p.N_csa = pl.N_csa;
    p.ksel = a->k;
    p.has_hca = hca;
    p.has_csa = csa;
    p.scale = a->sm_scale > 0.f ? a->sm_scale : (float)(1.0 / std::sqrt((double)D));
    p.scale_log2 = (float)((double)p.scale * 1.4426950408889634);
    const int nch = a->Hkv * D;
    for (int jb = 0; jb < 4; ++jb) {
        const bool present = jb < 2 ? hca : csa;
        if (!present) continue;
        ZJob& J = p.z[p.nz++];
        J.x = (jb & 1) == 0 ? a->k_raw : a->v_raw;
        J.dxc = jb == 0 ? p.dkc_hca : jb == 1 ? p.dvc_hca : jb == 2 ? p.dkc_csa : p.dvc_csa;
        J.z = jb == 0 ? a->zk_hca : jb == 1 ? a->zv_hca : jb == 2 ? a->zk_csa : a->zv_csa;
        J.dz = jb == 0 ? a->dzk_hca : jb == 1 ? a->dzv_hca : jb == 2 ? a->dzk_csa : a->dzv_csa;
        J.m = jb < 2 ? a->m_hca : a->m_csa;
        J.N = jb < 2 ? pl.N_hca : pl.N_csa;
        J.nchunk = J.N > 0 ? (J.N + kDpChunk - 1) / kDpChunk : 1;
        J.pz = reinterpret_cast<float*>(ws + pl.off_pz[jb]);
        J.dp = reinterpret_cast<float*>(ws + pl.off_dp[jb]);
    }
    const dim3 blk(kThreads);
    auto tiles = [](int n) { return (long long)((n + kRowsPerGroup - 1) / kRowsPerGroup); };
    const long long qgrid = (long long)a->B * a->H * tiles(a->T);
    if (qgrid > 0) hipLaunchKernelGGL((bwd_query_kernel<T, D>), dim3((unsigned)qgrid), blk, 0, s, p);
    if (p.nz > 0)
        hipLaunchKernelGGL(bwd_weights_kernel, dim3((nch + kThreads - 1) / kThreads, p.nz), blk, 0, s, p, nch);
    const long long hgrid = (long long)a->B * a->Hkv * tiles(pl.N_hca);
    if (hca && hgrid > 0) hipLaunchKernelGGL((bwd_key_kernel<T, D, 1>), dim3((unsigned)hgrid), blk, 0, s, p);
    const long long cgrid = (long long)a->B * a->Hkv * tiles(pl.N_csa);
    if (csa && cgrid > 0) hipLaunchKernelGGL((bwd_key_kernel<T, D, 2>), dim3((unsigned)cgrid), blk, 0, s, p);
    const long long rgrid = (long long)a->B * a->Hkv * tiles(a->T);
    if (rgrid > 0) hipLaunchKernelGGL((bwd_key_kernel<T, D, 0>), dim3((unsigned)rgrid), blk, 0, s, p);
    if (p.nz > 0) {
        long long most = 0;
        for (int z = 0; z < p.nz; ++z) {
            const long long n = (long long)a->B * p.z[z].nchunk * p.z[z].m * nch;
            most = n > most ? n : most;
        }
        if (most > 0)
            hipLaunchKernelGGL((bwd_dp_kernel<T>), dim3((unsigned)((most + kThreads - 1) / kThreads), p.nz), blk, 0,
                               s, p, nch);
        hipLaunchKernelGGL(bwd_dz_kernel, dim3((nch + kThreads - 1) / kThreads, p.nz), blk, 0, s, p, nch);
    }
    if (a->gate_mode == 0) {
        hipLaunchKernelGGL(bwd_gate_head_kernel, dim3(a->H * 3), blk, 0, s, p);
    } else {
        const long long n = (long long)a->B * a->T * a->H;
        if (n > 0)
            hipLaunchKernelGGL(bwd_gate_token_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), blk, 0, s, p);
    }
    return check_launch("hybrid_sparse_attn_bwd");
}

}  // namespace
}  // namespace shattn

using namespace shattn;

extern "C" size_t hybrid_sparse_attn_bwd_workspace_size(const shattn_bwd_args* a) {
    if (bwd_validate(a) != SHATTN_OK) return 0;
    return bwd_plan(a).bytes;
}

extern "C" int hybrid_sparse_attn_bwd(const shattn_bwd_args* a, void* ws, size_t ws_bytes, void* stream) {
    const int rc = bwd_validate(a);
    if (rc != SHATTN_OK) return rc;
    const BwdPlan pl = bwd_plan(a);
    if (pl.bytes > 0 && (!ws || ws_bytes < pl.bytes))
        return fail(SHATTN_EWORKSPACE, "hybrid_sparse_attn_bwd: workspace of %zu bytes needed, %zu given", pl.bytes,
                    ws ? ws_bytes : (size_t)0);
    if (pl.bytes > 0 && !aligned16(ws))
        return fail(SHATTN_EINVAL, "hybrid_sparse_attn_bwd: workspace must be 16-byte aligned");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* w = reinterpret_cast<char*>(ws);
    if (a->dtype == SHATTN_DTYPE_BF16)
        return a->d == 128 ? bwd_launch<bf16_t, 128>(a, pl, w, s) : bwd_launch<bf16_t, 64>(a, pl, w, s);
    return a->d == 128 ? bwd_launch<float, 128>(a, pl, w, s) : bwd_launch<float, 64>(a, pl, w, s);
}
