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
// Two forms of the query and key sides.
//
// Coefficient form (bf16 inputs, CSA caches up to 4096 entries, workspace for
// 8 bytes per (row, head, key) pair): the contractions run on MFMA.
//   1'. selection bitmaps of every row with per-word prefix counts (the rank
//       of an entry in its row's selection);
//   1'. query side: per 64 rows of a (sequence, head), K / V chunks of every
//       key source staged in LDS; pass 1 takes each branch's LSE and D_b,
//       pass 2 computes S, dP and dS^T on MFMA, accumulates dQ^T += K^T dS^T
//       (dS split into two bf16 parts) and writes (dS, sum_b w_b P_b) of every
//       (row, head, key) as the key sides' coefficients;
//   3'./4'. key sides: dK^T = Q^T dS and dV^T = dO^T (w P) on MFMA from LDS-
//       staged Q / dO chunks, per raw row, HCA entry (row ranges with fixed-
//       order partial sums) and CSA entry.
// VALU form (every other case; also the reference the coefficient form is
// checked against): four lanes per row, each holding a quarter of the head
// dim, a dot product being four partial sums and two in-register exchanges;
// a wave holds 16 rows and walks the union of their key or query sets in
// lockstep, masking per row:
//   1. query side: per (row, head) one pass for LSE_b and D_b (an online
//      softmax carrying a scalar accumulator of dpo), a second for dq;
//   3. key side, compressed entries: HCA entries over the query rows that see
//      them, CSA entries over the rows whose selection holds them (found with
//      one coalesced read of the row's selection and a wave-wide OR);
//   4. key side, raw rows over their window band.
// Both forms share:
//   2. block weights P = softmax(z) of every compression logit tensor;
//   the compressed-cache gradients routed back through the block merge
//      (dx = P_i dxc) in the raw-row key side's epilogue;
//   5. logit gradients: dP_i = sum over blocks of dxc . x_i as per-chunk
//      partials, then dz_i = P_i (dP_i - sum_l P_l dP_l) summing the partials
//      in a fixed order;
//   6. gate gradients (per head: a fixed-order sum over rows).
// No floating-point atomics: every output element is written by one thread
// in a fixed order, so results are deterministic.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

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
    // coefficient form (bf16, small N_csa): the query side writes, per
    // (row, head, key of its sets), (dS, sum_b w_b P_b) and the key sides
    // read them instead of recomputing scores
    float2* coef_w;    // [B, H, T, W]: window key at slot pos - (t - W + 1)
    float2* coef_h;    // [B, H, T, N_hca]
    float2* coef_c;    // [B, H, T, k]: the r-th visible selected entry of row t (ascending)
    uint32_t* bm;      // [B, T, bmw] selection bitmap of each row (visible entries only)
    int32_t* bmpre;    // [B, T, bmw] selected entries of the row in the words before
    int bmw;
    float* hpart;      // [B, Hkv, nrange, N_hca, 2, d] HCA cache-gradient partial sums per row range
    int nrange;        // row ranges of kKeyRange rows (HCA key side)
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


// ------------------------------------------------------------ 1'. query side on MFMA
// (bf16, N_csa small enough for a per-row selection bitmap)
// Selection bitmap of every row (visible entries only) and, per word, the
// number of selected entries in the words before it: the rank of an entry in
// its row's ascending selection is pre[w] + popcount(word & bits below).
constexpr int kMaxBmw = 128;   // bitmap words of a row (entries up to 4096)

__global__ __launch_bounds__(kThreads) void bwd_bitmap_kernel(BwdParams p) {
    // one wave per row: the row's words are built in LDS (selections OR their
    // bits in, one entry per lane per step), then written out with a
    // wave-wide prefix count
    __shared__ uint32_t words[kThreads / 64][kMaxBmw];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * (kThreads / 64) + wv;
    if (row >= (long long)p.B * p.T) return;
    const int t = (int)(row % p.T);
    uint32_t* wd = words[wv];
    for (int w = lane; w < p.bmw; w += 64) wd[w] = 0u;
    wave_lds_sync();
    const int nc = n_visible(t, p.W, p.m_csa, p.N_csa);
    const int32_t* sel = p.idx + row * p.ksel;
    for (int j = lane; j < p.ksel; j += 64) {
        const int e = sel[j];
        if (e >= 0 && e < nc) atomicOr(&wd[e >> 5], 1u << (e & 31));
    }
    wave_lds_sync();
    int run = 0;   // selected entries in the earlier 64-word groups
    for (int w0 = 0; w0 < p.bmw; w0 += 64) {
        const int w = w0 + lane;
        const uint32_t x = w < p.bmw ? wd[w] : 0u;
        const int c = __popc(x);
        const int incl = wave_incl_scan(c);
        if (w < p.bmw) {
            p.bm[row * p.bmw + w] = x;
            p.bmpre[row * p.bmw + w] = run + incl - c;
        }
        run += __shfl(incl, 63);
    }
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kKC = 32;   // keys per MFMA chunk

// Workgroup: 64 query rows of one (sequence, head), 16 per wave as the
// columns of the transposed products S^T = K Q^T and dP^T = V dO^T (32 keys
// x 16 columns per chunk, v_mfma_f32_16x16x32_bf16) and dQ^T += K^T dS^T.
// K and V chunks of every key source (the union of the tile's windows, the
// HCA entries its last row sees, every CSA entry it could select, masked per
// row through the bitmap) are staged once per workgroup in LDS by direct
// global->LDS loads, row-major with 16-byte pieces XOR-swizzled per row,
// double-buffered.  Pass 1: per column and branch an online log-sum-exp and
// D_b = sum_j P_bj dpo_j (per-lane partial states merged across the column's
// four lanes at the end).  Pass 2: P, dS and sum_b w_b P_b per (row, key)
// are written as coefficients for the key sides; dQ accumulates K^T dS^T on
// MFMA with dS split into two bf16 parts (hi + lo, about 16 significant
// bits) so that the float32 gradient keeps its precision.
template <int D>
__global__ __launch_bounds__(kThreads, 3) void bwd_query_mfma_kernel(BwdParams p) {
    constexpr int PIECES = D / 8, ROWB = D * 2, RPI = 1024 / ROWB, KS = D / 32, DT = D / 16;
    constexpr int MAT = kKC * ROWB, NL = kKC / RPI;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    auto swz = [](int row) { return ((row & 3) | (((row >> 3) & 3) << 2)) & (PIECES - 1); };
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, q4 = lane >> 4;
    const int ntile = (p.T + 63) / 64;
    const int work = (int)xcd_work_id(blockIdx.x, gridDim.x);
    const int tile = work % ntile;
    const int h = (work / ntile) % p.H;
    const int b = work / (ntile * p.H);
    const int g = h / p.G;
    const int t0 = tile * 64;
    const int t_last = min(t0 + 63, p.T - 1);
    const int t = t0 + wave * 16 + n;
    const bool valid = t < p.T;
    const int rs = p.Hkv * D;
    // B operands: this column's query and incoming gradient, dims 32 ks + 8 q4 .. +7
    bf16x8_t qf[KS], of[KS];
    {
        const long long off = (((long long)b * p.T + (valid ? t : t_last)) * p.H + h) * D;
        const bf16_t* qr = reinterpret_cast<const bf16_t*>(p.q) + off;
        const bf16_t* orw = reinterpret_cast<const bf16_t*>(p.dout) + off;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = *reinterpret_cast<const bf16x8_t*>(qr + 32 * ks + 8 * q4);
            of[ks] = *reinterpret_cast<const bf16x8_t*>(orw + 32 * ks + 8 * q4);
        }
    }
    float gw[3];
    gate_w(p, b, valid ? t : t_last, h, gw);
    // A-operand reads of a 32-row matrix: S^T rows (keys 8 (r >> 2) + (r & 3)
    // and +4) and the transposing reads of K^T (rows 8 (lane >> 4) + (sl >> 2)
    // and +4, dims 16 dt + 4 (sl & 3) .. +3)
    int kro[KS], tro[DT];
    {
        const int key0 = 8 * (n >> 2) + (n & 3);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kro[ks] = key0 * ROWB + (((4 * ks + q4) ^ swz(key0)) * 16);
        const int sl = n, trow = 8 * q4 + (sl >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            tro[dt] = trow * ROWB + (((2 * dt + ((sl & 3) >> 1)) ^ swz(trow)) * 16) + 8 * (sl & 1);
    }
    // key sources of the workgroup: window rows [w_lo, t_last], HCA entries
    // [0, nh_max), CSA entries [0, nc_max)
    const int w_lo = max(0, t0 - p.W + 1);
    const int wn = t_last - w_lo + 1;
    const int nh_max = p.has_hca ? n_visible(t_last, p.W, p.m_hca, p.N_hca) : 0;
    const int nc_max = p.has_csa ? n_visible(t_last, p.W, p.m_csa, p.N_csa) : 0;
    const int cw = (wn + kKC - 1) / kKC, ch = (nh_max + kKC - 1) / kKC, cc = (nc_max + kKC - 1) / kKC;
    const int nchunks = cw + ch + cc;
    const bf16_t* kraw = reinterpret_cast<const bf16_t*>(p.k) + (long long)b * p.T * rs + g * D;
    const bf16_t* vraw = reinterpret_cast<const bf16_t*>(p.v) + (long long)b * p.T * rs + g * D;
    const bf16_t* khca = reinterpret_cast<const bf16_t*>(p.k_hca) + (long long)b * p.N_hca * rs + g * D;
    const bf16_t* vhca = reinterpret_cast<const bf16_t*>(p.v_hca) + (long long)b * p.N_hca * rs + g * D;
    const bf16_t* kcsa = reinterpret_cast<const bf16_t*>(p.k_csa) + (long long)b * p.N_csa * rs + g * D;
    const bf16_t* vcsa = reinterpret_cast<const bf16_t*>(p.v_csa) + (long long)b * p.N_csa * rs + g * D;
    // chunk ci: its type (0 window, 1 HCA, 2 CSA), first key (position or entry), valid rows
    auto chunk = [&](int ci, int& type, int& base, int& nv) {
        if (ci < cw) {
            type = 0;
            base = w_lo + ci * kKC;
            nv = min(kKC, wn - ci * kKC);
        } else if (ci < cw + ch) {
            type = 1;
            base = (ci - cw) * kKC;
            nv = min(kKC, nh_max - base);
        } else {
            type = 2;
            base = (ci - cw - ch) * kKC;
            nv = min(kKC, nc_max - base);
        }
    };
    auto tbuf = [&](int par) { return smem + par * 2 * MAT; };
    auto stage = [&](int ci, char* buf) {
        int type, base, nv;
        chunk(ci, type, base, nv);
        const bf16_t* kb = type == 0 ? kraw : (type == 1 ? khca : kcsa);
        const bf16_t* vb = type == 0 ? vraw : (type == 1 ? vhca : vcsa);
        kb += (long long)base * rs;
        vb += (long long)base * rs;
#pragma unroll
        for (int L = wave; L < 2 * NL; L += 4) {
            const int mat = L / NL, li = L - mat * NL;
            const int row = li * RPI + lane / PIECES, slot = lane % PIECES;
            const bf16_t* src = (mat ? vb : kb) + (long long)(row < nv ? row : 0) * rs + ((slot ^ swz(row)) * 8);
            __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(buf + mat * MAT + li * 1024), 16, 0, 0);
        }
    };
    auto mfma_scores = [&](const char* mb, const bf16x8_t* bop, float* s) {
        f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(mb + kro[ks]);
            const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(mb + kro[ks] + 4 * ROWB);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bop[ks], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bop[ks], s1, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[r] = s0[r];
            s[4 + r] = s1[r];
        }
    };
    // membership of this column's keys 8 q4 + j of chunk (type, base): branch
    // bits, and for CSA entries the word of the row's bitmap
    const uint32_t win_mask = branch_mask_window(p);
    const int nh_t = p.has_hca && valid ? n_visible(t, p.W, p.m_hca, p.N_hca) : 0;
    const uint32_t* bmrow = p.bm + ((long long)b * p.T + (valid ? t : 0)) * p.bmw;
    const int32_t* prerow = p.bmpre + ((long long)b * p.T + (valid ? t : 0)) * p.bmw;
    auto members = [&](int type, int base, int nv, uint32_t* mbits, uint32_t& word) {
        word = 0u;
        if (type == 2 && valid) word = bmrow[base >> 5];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kk = 8 * q4 + j;
            uint32_t m = 0u;
            if (valid && kk < nv) {
                const int key = base + kk;
                if (type == 0) m = (key >= t - p.W + 1 && key <= t) ? win_mask : 0u;
                else if (type == 1) m = key < nh_t ? 1u : 0u;
                else m = ((word >> (kk & 31)) & 1u) ? 2u : 0u;
            }
            mbits[j] = m;
        }
    };

    // ---- pass 1: per-lane partial (max, sum, sum P dpo) per branch
    float mx[3] = {-INFINITY, -INFINITY, -INFINITY}, sm[3] = {0.f, 0.f, 0.f}, ac[3] = {0.f, 0.f, 0.f};
    float lse[3], Db[3];
    f32x4_t acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // the two passes as one loop body compiled twice (pass a constant in each)
    auto run_pass = [&](auto pass_c) {
        constexpr int pass = decltype(pass_c)::value;
        if (nchunks > 0) stage(0, tbuf(0));
        for (int ci = 0; ci < nchunks; ++ci) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();                       // chunk ci in tbuf(ci & 1); tbuf(ci + 1 & 1) free
            if (ci + 1 < nchunks) stage(ci + 1, tbuf((ci + 1) & 1));
            const char* kb = tbuf(ci & 1);
            const char* vb = kb + MAT;
            int type, base, nv;
            chunk(ci, type, base, nv);
            float s[8], dpo[8];
            mfma_scores(kb, qf, s);
            mfma_scores(vb, of, dpo);
            uint32_t mbits[8], word;
            members(type, base, nv, mbits, word);
            if constexpr (pass == 0) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float s2 = s[j] * p.scale_log2;
#pragma unroll
                    for (int br = 0; br < 3; ++br) {
                        if (!(mbits[j] & (1u << br))) continue;
                        const float mn = fmaxf(mx[br], s2);
                        const float a = exp2f(mx[br] - mn), e = exp2f(s2 - mn);
                        sm[br] = fmaf(sm[br], a, e);
                        ac[br] = fmaf(ac[br], a, e * dpo[j]);
                        mx[br] = mn;
                    }
                }
            } else {
                float ds[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float s2 = s[j] * p.scale_log2;
                    float d_ = 0.f, wp = 0.f;
#pragma unroll
                    for (int br = 0; br < 3; ++br) {
                        if (!(mbits[j] & (1u << br))) continue;
                        const float pw = gw[br] * exp2f(s2 - lse[br]);
                        wp += pw;
                        d_ = fmaf(pw, dpo[j] - Db[br], d_);
                    }
                    ds[j] = d_;
                    if (mbits[j]) {
                        const int key = base + 8 * q4 + j;
                        const long long rowc = ((long long)b * p.H + h) * p.T + t;
                        const float2 c2 = make_float2(d_, wp);
                        if (type == 0) p.coef_w[rowc * p.W + (key - (t - p.W + 1))] = c2;
                        else if (type == 1) p.coef_h[rowc * p.N_hca + key] = c2;
                        else {
                            const int bit = (8 * q4 + j) & 31;
                            const int r = prerow[base >> 5] + __popc(word & ((1u << bit) - 1u));
                            p.coef_c[rowc * p.ksel + r] = c2;
                        }
                    }
                }
                // dQ^T += K^T dS^T, dS = hi + lo in bf16
                bf16x8_t bhi, blo;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const __bf16 hi = (__bf16)ds[j];
                    bhi[j] = hi;
                    blo[j] = (__bf16)(ds[j] - (float)hi);
                }
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const char* a = kb + tro[dt];
                    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a));
                    const i16x4_t hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a + 4 * ROWB));
                    const i16x4_t lohi[2] = {lo, hi4};
                    bf16x8_t aop;
                    __builtin_memcpy(&aop, lohi, 16);
                    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, bhi, acc[dt], 0, 0, 0);
                    acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, blo, acc[dt], 0, 0, 0);
                }
            }
        }
        __syncthreads();   // every wave is done with both tiles before they are restaged
        if constexpr (pass == 0) {
            // merge the column's four lanes (n, n + 16, n + 32, n + 48) in a fixed order
#pragma unroll
            for (int br = 0; br < 3; ++br) {
                uint32_t lo, hi;
                xor16_pair(__float_as_uint(mx[br]), lo, hi);
                float M = fmaxf(__uint_as_float(lo), __uint_as_float(hi));
                xor32_pair(__float_as_uint(M), lo, hi);
                M = fmaxf(__uint_as_float(lo), __uint_as_float(hi));
                const float f = M == -INFINITY ? 0.f : exp2f(mx[br] - M);
                const float l = sum_xrows(sm[br] * f), a = sum_xrows(ac[br] * f);
                lse[br] = l > 0.f ? M + log2f(l) : 0.f;
                Db[br] = l > 0.f ? a / l : 0.f;
            }
            if (valid && q4 == 0) {
                float* st = p.stats + (((long long)b * p.T + t) * p.H + h) * 6;
#pragma unroll
                for (int br = 0; br < 3; ++br) {
                    st[br] = lse[br];
                    st[3 + br] = Db[br];
                }
            }
        }
    };
    run_pass(std::integral_constant<int, 0>());
    run_pass(std::integral_constant<int, 1>());
    if (!valid) return;
    float* dst = p.dq + (((long long)b * p.T + t) * p.H + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<float4*>(dst + 16 * dt + 4 * q4) =
            make_float4(p.scale * acc[dt][0], p.scale * acc[dt][1], p.scale * acc[dt][2], p.scale * acc[dt][3]);
}

// ------------------------------------------------------------ 2. block weights
// pz[i, ch] = softmax over i < m of z[i, ch] (one thread per channel; blockIdx.y = job)
__global__ __launch_bounds__(kThreads) void bwd_weights_kernel(BwdParams p, int nch) {
    const ZJob& J = p.z[blockIdx.y];
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= nch) return;
    float mx = -INFINITY;
#pragma unroll 16
    for (int i = 0; i < J.m; ++i) mx = fmaxf(mx, J.z[(long long)i * nch + c]);
    float s = 0.f;
#pragma unroll 16
    for (int i = 0; i < J.m; ++i) s += expf(J.z[(long long)i * nch + c] - mx);
    const float inv = 1.0f / s;
#pragma unroll 16
    for (int i = 0; i < J.m; ++i) J.pz[(long long)i * nch + c] = expf(J.z[(long long)i * nch + c] - mx) * inv;
}

// ------------------------------------------------------------ 3./4. key side
// KIND 0: raw rows (window keys of every present branch; queries t in
// [j, j + W - 1]), then the cache gradients routed through the block merge;
// 1: HCA entries (HCA branch; queries t >= (c+1) m + W - 1);
// 2: CSA entries (CSA branch; the visible queries whose selection holds c).
// Workgroup: 64 consecutive keys of one (sequence, KV head); a wave takes 16,
// walking the union of their query ranges in lockstep, G heads per row.
// COEF: (dS, sum_b w_b P_b) of each (row, head, key) come from the query
// side's coefficients (and CSA membership from the row bitmaps) instead of
// being recomputed from the scores.
template <typename T, int D, int KIND, bool COEF>
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
        uint32_t word = 0u;
        if (KIND == 2 && COEF) {
            word = p.bm[((long long)b * p.T + t) * p.bmw + (j >> 5)];
            in = in && ((word >> (j & 31)) & 1u);
        } else if (KIND == 2) {
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
            float wsum = 0.f, ds = 0.f;
            if constexpr (COEF) {
                if (in) {
                    const long long rowc = ((long long)b * p.H + h) * p.T + t;
                    float2 c2;
                    if (KIND == 0) c2 = p.coef_w[rowc * p.W + (j - t + p.W - 1)];
                    else if (KIND == 1) c2 = p.coef_h[rowc * p.N_hca + j];
                    else c2 = p.coef_c[rowc * p.ksel + p.bmpre[((long long)b * p.T + t) * p.bmw + (j >> 5)] +
                                       __popc(word & ((1u << (j & 31)) - 1u))];
                    ds = c2.x;
                    wsum = c2.y;
                }
            } else {
                const float* st = p.stats + (((long long)b * p.T + t) * p.H + h) * 6;
                float gw[3];
                gate_w(p, b, t, h, gw);
                const float s2 = quad_sum(dot_part<NP>(qv, kv)) * p.scale_log2;
                const float dpo = quad_sum(dot_part<NP>(ov, vv));
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


// ------------------------------------------------------------ 3'./4'. key sides on MFMA
// dK^T (d x keys) = Q^T (d x rows) dS (rows x keys) and dV^T = dO^T (w P),
// 32 rows per chunk (v_mfma_f32_16x16x32_bf16; the coefficient operand split
// into two bf16 parts, hi + lo).  Q and dO rows of the chunk are staged in
// LDS (row-major, swizzled, direct global->LDS loads, double-buffered) and
// read transposed; the coefficient operand of a lane is its key's
// coefficients at the chunk's rows 8 (lane >> 4) .. +7 (zero outside the
// key's row set).
//   KIND 0: raw rows; workgroup = 64 consecutive keys (16 per wave), rows
//           [j0, j0 + 63 + W - 1]; epilogue: the cache gradients routed
//           through the block merge.
//   KIND 1: HCA entries; workgroup = a range of kKeyRange rows, its four
//           waves one 32-row chunk each, every entry tile of 16; partial sums
//           per range (combined in a fixed order by bwd_hca_reduce_kernel).
//   KIND 2: CSA entries; workgroup = 64 consecutive entries, rows from the
//           first one that sees its first entry.
constexpr int kKeyRange = 128;

template <int D> struct QTile {
    static constexpr int PIECES = D / 8, ROWB = D * 2, RPI = 1024 / ROWB, DT = D / 16;
    static constexpr int MAT = 32 * ROWB, NL = 32 / RPI;
    __device__ static int swz(int row) { return ((row & 3) | (((row >> 3) & 3) << 2)) & (PIECES - 1); }
};

template <int D, int KIND>
__global__ __launch_bounds__(kThreads, 2) void bwd_key_mfma_kernel(BwdParams p) {
    typedef QTile<D> QT;
    constexpr int ROWB = QT::ROWB, DT = QT::DT, MAT = QT::MAT, NL = QT::NL, RPI = QT::RPI, PIECES = QT::PIECES;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, q4 = lane >> 4;
    const int rs = p.Hkv * D;            // K/V row stride
    const int qs = p.H * D;              // Q / dO row stride
    const int work = (int)xcd_work_id(blockIdx.x, gridDim.x);
    int b, g, j0 = 0, r_lo, r_hi;       // rows [r_lo, r_hi] of the workgroup
    if (KIND == 1) {
        const int rg = work % p.nrange;
        g = (work / p.nrange) % p.Hkv;
        b = work / (p.nrange * p.Hkv);
        r_lo = rg * kKeyRange + wave * 32;            // this wave's chunk
        r_hi = min(r_lo + 31, p.T - 1);
    } else {
        const int nkeys = KIND == 0 ? p.T : p.N_csa;
        const int ntile = (nkeys + 63) / 64;
        const int tile = work % ntile;
        g = (work / ntile) % p.Hkv;
        b = work / (ntile * p.Hkv);
        j0 = tile * 64;
        r_lo = KIND == 0 ? j0 : (j0 + 1) * p.m_csa + p.W - 1;
        r_hi = KIND == 0 ? min(j0 + 63 + p.W - 1, p.T - 1) : p.T - 1;
    }
    const int j = j0 + wave * 16 + n;    // this lane's key (KIND 0, 2)
    const int nkeys = KIND == 0 ? p.T : (KIND == 1 ? p.N_hca : p.N_csa);
    // transposing-read offsets of a 32-row matrix (rows 8 q4 + (n >> 2) and +4)
    int tro[DT];
    {
        const int trow = 8 * q4 + (n >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            tro[dt] = trow * ROWB + (((2 * dt + ((n & 3) >> 1)) ^ QT::swz(trow)) * 16) + 8 * (n & 1);
    }
    // KIND 1: one buffer per wave; else two shared by the workgroup
    auto tbuf = [&](int par) { return smem + (KIND == 1 ? wave * 2 * MAT : par * 2 * MAT); };
    // stage rows [r0, r0 + 32) of head h's Q and dO (rows past r_hi repeat r0)
    auto stage = [&](int h, int r0, char* buf, int nw, int w0) {
        const bf16_t* qb = reinterpret_cast<const bf16_t*>(p.q) + ((long long)b * p.T * p.H + h) * D;
        const bf16_t* ob = reinterpret_cast<const bf16_t*>(p.dout) + ((long long)b * p.T * p.H + h) * D;
#pragma unroll
        for (int L = w0; L < 2 * NL; L += nw) {
            const int mat = L / NL, li = L - mat * NL;
            const int row = li * RPI + lane / PIECES, slot = lane % PIECES;
            const int t = r0 + row <= r_hi ? r0 + row : r0;
            const bf16_t* src = (mat ? ob : qb) + (long long)t * qs + ((slot ^ QT::swz(row)) * 8);
            __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(buf + mat * MAT + li * 1024), 16, 0, 0);
        }
    };
    auto aop_at = [&](const char* mb, int dt) {
        const char* a = mb + tro[dt];
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(a + 4 * ROWB));
        const i16x4_t lohi[2] = {lo, hi};
        bf16x8_t aop;
        __builtin_memcpy(&aop, lohi, 16);
        return aop;
    };
    // coefficient of key `key` (or entry) at row t of head h: (dS, w P), zero outside its row set
    auto coef = [&](int h, int t, int key) -> float2 {
        if (t > r_hi || key >= nkeys) return make_float2(0.f, 0.f);
        const long long rowc = ((long long)b * p.H + h) * p.T + t;
        if (KIND == 0) {
            if (t < key || t > key + p.W - 1) return make_float2(0.f, 0.f);
            return p.coef_w[rowc * p.W + (key - t + p.W - 1)];
        } else if (KIND == 1) {
            if (key >= n_visible(t, p.W, p.m_hca, p.N_hca)) return make_float2(0.f, 0.f);
            return p.coef_h[rowc * p.N_hca + key];
        } else {
            const long long bw = ((long long)b * p.T + t) * p.bmw + (key >> 5);
            const uint32_t word = p.bm[bw];
            if (!((word >> (key & 31)) & 1u)) return make_float2(0.f, 0.f);
            return p.coef_c[rowc * p.ksel + p.bmpre[bw] + __popc(word & ((1u << (key & 31)) - 1u))];
        }
    };
    // pipelined form (KIND 0, 2): the bitmap words and prefix counts of this
    // lane's rows (KIND 2) and then its coefficients, loaded ahead of use
    auto load_w = [&](int r0, int key, uint32_t* word, int* pre) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = r0 + 8 * q4 + i;
            word[i] = 0u;
            pre[i] = 0;
            if (KIND == 2 && t <= r_hi && key < nkeys) {
                const long long bw = ((long long)b * p.T + t) * p.bmw + (key >> 5);
                word[i] = p.bm[bw];
                pre[i] = p.bmpre[bw];
            }
        }
    };
    auto load_c = [&](int h, int r0, int key, const uint32_t* word, const int* pre, float2* c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = r0 + 8 * q4 + i;
            c[i] = make_float2(0.f, 0.f);
            if (t > r_hi || key >= nkeys) continue;
            const long long rowc = ((long long)b * p.H + h) * p.T + t;
            if (KIND == 0) {
                if (t >= key && t <= key + p.W - 1) c[i] = p.coef_w[rowc * p.W + (key - t + p.W - 1)];
            } else if (KIND == 2) {
                if ((word[i] >> (key & 31)) & 1u)
                    c[i] = p.coef_c[rowc * p.ksel + pre[i] + __popc(word[i] & ((1u << (key & 31)) - 1u))];
            }
        }
    };
    auto split = [](const float* v, bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const __bf16 h_ = (__bf16)v[i];
            hi[i] = h_;
            lo[i] = (__bf16)(v[i] - (float)h_);
        }
    };
    // accumulate one staged chunk given this lane's coefficients c[0..7]
    auto mfma_chunk = [&](const char* buf, const float2* c, f32x4_t* ak, f32x4_t* av) {
        float ds[8], wp[8];
        bool any = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ds[i] = c[i].x;
            wp[i] = c[i].y;
            any |= c[i].x != 0.f || c[i].y != 0.f;
        }
        if (!__any(any)) return;
        bf16x8_t dh, dl, wh, wl;
        split(ds, dh, dl);
        split(wp, wh, wl);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16x8_t aq = aop_at(buf, dt), ao = aop_at(buf + MAT, dt);
            ak[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, dh, ak[dt], 0, 0, 0);
            ak[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, dl, ak[dt], 0, 0, 0);
            av[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, wh, av[dt], 0, 0, 0);
            av[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, wl, av[dt], 0, 0, 0);
        }
    };
    // one staged chunk (rows r0 ..) for key `key`, coefficients loaded on the spot
    auto chunk = [&](const char* buf, int h, int r0, int key, f32x4_t* ak, f32x4_t* av) {
        float2 c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = coef(h, r0 + 8 * q4 + i, key);
        mfma_chunk(buf, c, ak, av);
    };
    const int ch0 = g * D + 4 * q4;   // channel of acc[dt][0] within a K/V row: + 16 dt
    if (KIND == 1) {
        // this wave: one chunk of 32 rows, every entry tile of 16 (a chunk
        // past the end still writes its zero partials)
        const bool active = r_lo < p.T;
        char* buf = tbuf(0);
        const int rg = work % p.nrange;
        for (int ct = 0; ct * 16 < p.N_hca; ++ct) {
            f32x4_t ak[DT], av[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) ak[dt] = av[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            for (int hh = 0; hh < p.G && active; ++hh) {
                const int h = g * p.G + hh;
                stage(h, r_lo, buf, 1, 0);
                __builtin_amdgcn_s_waitcnt(0);
                wave_lds_sync();
                chunk(buf, h, r_lo, ct * 16 + n, ak, av);
                wave_lds_sync();
            }
            // partial of this wave's chunk; the four waves' partials of a range
            // are added in wave order by the reduce kernel
            const int c = ct * 16 + n;
            if (c < p.N_hca) {
                float* dst = p.hpart + ((((long long)b * p.Hkv + g) * p.nrange + rg) * 4 + wave) * (long long)p.N_hca * 2 * D;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    *reinterpret_cast<float4*>(dst + ((long long)c * 2) * D + 16 * dt + 4 * q4) =
                        make_float4(ak[dt][0], ak[dt][1], ak[dt][2], ak[dt][3]);
                    *reinterpret_cast<float4*>(dst + ((long long)c * 2 + 1) * D + 16 * dt + 4 * q4) =
                        make_float4(av[dt][0], av[dt][1], av[dt][2], av[dt][3]);
                }
            }
        }
        return;
    }
    if (j0 >= nkeys) return;
    f32x4_t ak[DT], av[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) ak[dt] = av[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int nch = r_hi >= r_lo ? (r_hi - r_lo + 32) / 32 : 0;
    for (int hh = 0; hh < p.G && KIND == 0; ++hh) {
        // raw rows: coefficients loaded on the spot (the window's single load
        // per row; holding the next chunk's would cost a wave per SIMD)
        const int h = g * p.G + hh;
        if (nch > 0) stage(h, r_lo, tbuf(0), 4, wave);
        for (int ci = 0; ci < nch; ++ci) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (ci + 1 < nch) stage(h, r_lo + 32 * (ci + 1), tbuf((ci + 1) & 1), 4, wave);
            chunk(tbuf(ci & 1), h, r_lo + 32 * ci, j, ak, av);
        }
        __syncthreads();
    }
    for (int hh = 0; hh < p.G && KIND == 2; ++hh) {
        const int h = g * p.G + hh;
        // chunk ci + 1's coefficients (and chunk ci + 2's bitmap words) load
        // while chunk ci is computed
        uint32_t w1[8], w2[8];
        int p1[8], p2[8];
        float2 c0[8];
        if (nch > 0) {
            stage(h, r_lo, tbuf(0), 4, wave);
            load_w(r_lo, j, w1, p1);
            load_c(h, r_lo, j, w1, p1, c0);
            load_w(r_lo + 32, j, w1, p1);
        }
        for (int ci = 0; ci < nch; ++ci) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            const int r1 = r_lo + 32 * (ci + 1);
            float2 c1[8];
            if (ci + 1 < nch) {
                stage(h, r1, tbuf((ci + 1) & 1), 4, wave);
                load_c(h, r1, j, w1, p1, c1);
                load_w(r1 + 32, j, w2, p2);
            }
            mfma_chunk(tbuf(ci & 1), c0, ak, av);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                c0[i] = c1[i];
                w1[i] = w2[i];
                p1[i] = p2[i];
            }
        }
        __syncthreads();
    }
    if (j >= nkeys) return;
    float dk[DT][4], dv[DT][4];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dk[dt][r] = p.scale * ak[dt][r];
            dv[dt][r] = av[dt][r];
        }
    if (KIND == 0) {
        // raw row j also feeds block j / m of each compression (full blocks only)
        const int nchn = p.Hkv * D;
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
            const long long co = ((long long)b * N + blk) * nchn;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int chn = ch0 + 16 * dt + r;
                    dk[dt][r] = fmaf(Jk.pz[(long long)i * nchn + chn], Jk.dxc[co + chn], dk[dt][r]);
                    dv[dt][r] = fmaf(Jv.pz[(long long)i * nchn + chn], Jv.dxc[co + chn], dv[dt][r]);
                }
        }
    }
    float* dko = KIND == 0 ? p.dk : p.dkc_csa;
    float* dvo = KIND == 0 ? p.dv : p.dvc_csa;
    const long long o = ((long long)b * nkeys + j) * rs + ch0;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        *reinterpret_cast<float4*>(dko + o + 16 * dt) = make_float4(dk[dt][0], dk[dt][1], dk[dt][2], dk[dt][3]);
        *reinterpret_cast<float4*>(dvo + o + 16 * dt) = make_float4(dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]);
    }
}

// HCA cache gradients: the partial sums of every (range, wave) chunk added in
// order (one thread per (b, entry, channel))
__global__ __launch_bounds__(kThreads) void bwd_hca_reduce_kernel(BwdParams p, int D) {
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long nchn = (long long)p.Hkv * D;
    if (gid >= (long long)p.B * p.N_hca * nchn) return;
    const int b = (int)(gid / (p.N_hca * nchn));
    const long long r = gid - (long long)b * p.N_hca * nchn;
    const int c = (int)(r / nchn), chn = (int)(r - (long long)c * nchn);
    const int g = chn / D, e = chn - g * D;
    float sk = 0.f, sv = 0.f;
    for (int rc = 0; rc < p.nrange * 4; ++rc) {
        const float* src = p.hpart + ((((long long)b * p.Hkv + g) * p.nrange) * 4 + rc) * (long long)p.N_hca * 2 * D;
        sk += src[((long long)c * 2) * D + e];
        sv += src[((long long)c * 2 + 1) * D + e];
    }
    p.dkc_hca[gid] = p.scale * sk;
    p.dvc_hca[gid] = sv;
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
#pragma unroll 8
    for (int blk = chunk * kDpChunk; blk < c_end; ++blk)
        s = fmaf(J.dxc[((long long)b * J.N + blk) * nch + c],
                 Elem<T>::load1(x + ((long long)b * p.T + (long long)blk * J.m + i) * nch + c), s);
    J.dp[gid] = s;
}

// dP_i = sum over (b, chunk) of the partials, in order, stored in dz (one
// thread per (i, ch); blockIdx.y = job)
__global__ __launch_bounds__(kThreads) void bwd_dpsum_kernel(BwdParams p, int nch) {
    const ZJob& J = p.z[blockIdx.y];
    const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
    const long long per_chunk = (long long)J.m * nch;
    if (gid >= per_chunk) return;
    const int nbc = p.B * J.nchunk;
    float dp = 0.f;
#pragma unroll 8
    for (int bc = 0; bc < nbc; ++bc) dp += J.dp[bc * per_chunk + gid];
    J.dz[gid] = dp;
}

// dz[i, ch] = P_i (dP_i - sum_l P_l dP_l) (one thread per channel; blockIdx.y = job)
__global__ __launch_bounds__(kThreads) void bwd_dz_kernel(BwdParams p, int nch) {
    const ZJob& J = p.z[blockIdx.y];
    const int c = blockIdx.x * kThreads + threadIdx.x;
    if (c >= nch) return;
    float cen = 0.f;
#pragma unroll 16
    for (int i = 0; i < J.m; ++i) cen = fmaf(J.pz[(long long)i * nch + c], J.dz[(long long)i * nch + c], cen);
#pragma unroll 16
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
    size_t off_coef_w, off_coef_h, off_coef_c, off_bm, off_bmpre, off_hpart;
    int nrange;
    size_t bytes;
    int N_hca, N_csa;
    bool coef;   // MFMA query side and coefficient key sides
    int bmw;
};

// The coefficient form holds (dS, sum w P) of every (row, head, key of its
// sets): 8 bytes per pair, at most this much workspace for them.
constexpr size_t kCoefMaxBytes = (size_t)8 << 30;
// largest CSA entry count attended through the row bitmaps (masked chunks)
constexpr int kCoefMaxNcsa = 4096;   // = 32 * kMaxBmw

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
    // coefficient form: bf16, CSA entries few enough to attend masked
    const size_t rows = (size_t)a->B * a->T;
    const size_t coef_b = rows * a->H * 8 * ((size_t)a->W + pl.N_hca + (csa ? a->k : 0));
    pl.coef = a->dtype == SHATTN_DTYPE_BF16 && pl.N_csa <= kCoefMaxNcsa && coef_b <= kCoefMaxBytes;
    if (pl.coef) {
        pl.bmw = csa ? (pl.N_csa + 31) / 32 : 0;
        auto takeb = [&](size_t bytes) {
            const size_t o = off;
            off += align256(bytes);
            return o;
        };
        pl.off_coef_w = takeb(rows * a->H * (size_t)a->W * 8);
        pl.off_coef_h = takeb(rows * a->H * (size_t)pl.N_hca * 8);
        pl.off_coef_c = takeb(csa ? rows * a->H * (size_t)a->k * 8 : 0);
        pl.off_bm = takeb(rows * (size_t)pl.bmw * 4);
        pl.off_bmpre = takeb(rows * (size_t)pl.bmw * 4);
        pl.nrange = (a->T + kKeyRange - 1) / kKeyRange;
        pl.off_hpart = takeb((size_t)a->B * a->Hkv * pl.nrange * 4 * pl.N_hca * 2 * a->d * 4);
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
    const long long hgrid = (long long)a->B * a->Hkv * tiles(pl.N_hca);
    const long long cgrid = (long long)a->B * a->Hkv * tiles(pl.N_csa);
    const long long rgrid = (long long)a->B * a->Hkv * tiles(a->T);
    bool coef = false;
    if constexpr (std::is_same<T, bf16_t>::value) coef = pl.coef;
    if (coef) {
        if constexpr (std::is_same<T, bf16_t>::value) {
            p.coef_w = reinterpret_cast<float2*>(ws + pl.off_coef_w);
            p.coef_h = reinterpret_cast<float2*>(ws + pl.off_coef_h);
            p.coef_c = reinterpret_cast<float2*>(ws + pl.off_coef_c);
            p.bm = reinterpret_cast<uint32_t*>(ws + pl.off_bm);
            p.bmpre = reinterpret_cast<int32_t*>(ws + pl.off_bmpre);
            p.bmw = pl.bmw;
            p.hpart = reinterpret_cast<float*>(ws + pl.off_hpart);
            p.nrange = pl.nrange;
            const long long rows = (long long)a->B * a->T;
            if (csa && rows > 0)
                hipLaunchKernelGGL(bwd_bitmap_kernel, dim3((unsigned)((rows + 3) / 4)), blk, 0, s, p);
            const size_t lds = 4 * (size_t)32 * D * 2;   // K and V chunks, double-buffered
            if (qgrid > 0) hipLaunchKernelGGL((bwd_query_mfma_kernel<D>), dim3((unsigned)qgrid), blk, lds, s, p);
            if (p.nz > 0)
                hipLaunchKernelGGL(bwd_weights_kernel, dim3((nch + kThreads - 1) / kThreads, p.nz), blk, 0, s, p, nch);
            const size_t mat = (size_t)32 * D * 2;
            if (hca && pl.N_hca > 0 && rows > 0) {
                hipLaunchKernelGGL((bwd_key_mfma_kernel<D, 1>), dim3((unsigned)((long long)a->B * a->Hkv * pl.nrange)),
                                   blk, 8 * mat, s, p);
                const long long n = (long long)a->B * pl.N_hca * nch;
                hipLaunchKernelGGL(bwd_hca_reduce_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), blk, 0, s,
                                   p, D);
            }
            if (csa && cgrid > 0)
                hipLaunchKernelGGL((bwd_key_mfma_kernel<D, 2>), dim3((unsigned)cgrid), blk, 4 * mat, s, p);
            if (rgrid > 0) hipLaunchKernelGGL((bwd_key_mfma_kernel<D, 0>), dim3((unsigned)rgrid), blk, 4 * mat, s, p);
        }
    } else {
        if (qgrid > 0) hipLaunchKernelGGL((bwd_query_kernel<T, D>), dim3((unsigned)qgrid), blk, 0, s, p);
        if (p.nz > 0)
            hipLaunchKernelGGL(bwd_weights_kernel, dim3((nch + kThreads - 1) / kThreads, p.nz), blk, 0, s, p, nch);
        if (hca && hgrid > 0)
            hipLaunchKernelGGL((bwd_key_kernel<T, D, 1, false>), dim3((unsigned)hgrid), blk, 0, s, p);
        if (csa && cgrid > 0)
            hipLaunchKernelGGL((bwd_key_kernel<T, D, 2, false>), dim3((unsigned)cgrid), blk, 0, s, p);
        if (rgrid > 0) hipLaunchKernelGGL((bwd_key_kernel<T, D, 0, false>), dim3((unsigned)rgrid), blk, 0, s, p);
    }
    if (p.nz > 0) {
        long long most = 0;
        for (int z = 0; z < p.nz; ++z) {
            const long long n = (long long)a->B * p.z[z].nchunk * p.z[z].m * nch;
            most = n > most ? n : most;
        }
        if (most > 0)
            hipLaunchKernelGGL((bwd_dp_kernel<T>), dim3((unsigned)((most + kThreads - 1) / kThreads), p.nz), blk, 0,
                               s, p, nch);
        int mmax = 0;
        for (int z = 0; z < p.nz; ++z) mmax = p.z[z].m > mmax ? p.z[z].m : mmax;
        const long long nsum = (long long)mmax * nch;
        hipLaunchKernelGGL(bwd_dpsum_kernel, dim3((unsigned)((nsum + kThreads - 1) / kThreads), p.nz), blk, 0, s, p,
                           nch);
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
