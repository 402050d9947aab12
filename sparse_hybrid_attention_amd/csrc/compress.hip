// Block compression of K and V on gfx950.
//
// Method ([V4-code] section 1, block merge; [V4-blog] "CSA" 4:1 diagram):
// every m consecutive raw rows become one entry, a per-channel weighted sum
// whose weights are the softmax, over the m block positions, of a learned
// [m, Hkv, d] logit tensor.
//
// Design (HBM-bound streaming, write = read / m):
//  * A block of m rows of one sequence is one contiguous [m, C] slab
//    (C = Hkv*d channels), so each thread owns one 16-byte channel group
//    (8 bf16 / 4 fp32 channels) and PPT consecutive block positions; it keeps
//    those PPT x 8 softmax weights in registers for every block it visits.
//  * R = ceil(m / PPT) threads share a channel group; their float32 partial
//    sums are combined through LDS in a fixed order (deterministic).  For
//    m <= 8 a thread covers the whole block and writes its 16 bytes directly.
//  * The softmax of the logits is computed once per workgroup: each thread
//    reduces its own positions, partial max / sum are combined in LDS.
//  * K and V are two slices of the same launch (blockIdx.z).
//  * Each wave issues PPT independent 128-bit loads per block; consecutive
//    lanes read consecutive 16-byte groups of a row (coalesced).
#include "common.h"

namespace shattn {

namespace {

constexpr int kThreads = 256;
constexpr int kPPT = 8;  // block positions per thread

template <typename T>
__global__ __launch_bounds__(kThreads) void compress_kernel(
    const T* __restrict__ x0, const T* __restrict__ x1, const float* __restrict__ z0,
    const float* __restrict__ z1, T* __restrict__ y0, T* __restrict__ y1, int T_len, int C,
    int m, int N, int R, int NGt, long long total_blocks, int blocks_per_wg) {
    constexpr int VW = Elem<T>::kVec;
    const T* __restrict__ x = blockIdx.z ? x1 : x0;
    const float* __restrict__ z = blockIdx.z ? z1 : z0;
    T* __restrict__ y = blockIdx.z ? y1 : y0;

    __shared__ float red[kThreads * VW];

    const int NG = C / VW;
    const int tid = threadIdx.x;
    const int s = tid / NGt;          // position subset (R > 1) or block lane (R == 1)
    const int jl = tid - s * NGt;     // channel group within the tile
    const int j = blockIdx.x * NGt + jl;
    const int nsub = kThreads / NGt;  // threads per channel group in the workgroup
    const bool active = (R == 1 ? s < nsub : s < R) && (j < NG);
    const int ppt = (m < kPPT) ? m : kPPT;
    const int spos = R == 1 ? 0 : s;  // which positions of the block this thread owns

    const long long bc0 = (long long)blockIdx.y * blocks_per_wg;
    long long bc1 = bc0 + blocks_per_wg;
    if (bc1 > total_blocks) bc1 = total_blocks;
    // rows of block bc owned by this thread (R > 1: positions s*ppt .. +ppt)
    auto load_rows = [&](long long bc, uint4* raw) {
        const long long b = bc / N;
        const long long c = bc - b * N;
        const T* __restrict__ src = x + ((size_t)b * T_len + (size_t)c * m + (size_t)s * ppt) * C + (size_t)j * VW;
#pragma unroll
        for (int q = 0; q < kPPT; ++q)
            raw[q] = (q < ppt && s * ppt + q < m) ? ld16_stream(src + (size_t)q * C) : make_uint4(0, 0, 0, 0);
    };
    uint4 rowsA[kPPT];
    if (R > 1 && active && bc0 < bc1) load_rows(bc0, rowsA);   // first block in flight during the set-up

    // ---- softmax weights of this thread's positions and channels (16-byte
    // logit loads; the partials of the R threads of a channel group combine
    // in LDS in a fixed order)
    float p[kPPT][VW];
    float mx[VW];
#pragma unroll
    for (int v = 0; v < VW; ++v) mx[v] = -INFINITY;
#pragma unroll
    for (int q = 0; q < kPPT; ++q) {
        const int i = spos * ppt + q;
        if (active && q < ppt && i < m) {
            const float4* zs = reinterpret_cast<const float4*>(z + (size_t)i * C + (size_t)j * VW);
#pragma unroll
            for (int u = 0; u < VW / 4; ++u) {
                const float4 f = zs[u];
                p[q][4 * u + 0] = f.x;
                p[q][4 * u + 1] = f.y;
                p[q][4 * u + 2] = f.z;
                p[q][4 * u + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int v = 0; v < VW; ++v) p[q][v] = -INFINITY;
        }
#pragma unroll
        for (int v = 0; v < VW; ++v) mx[v] = fmaxf(mx[v], p[q][v]);
    }
    auto combine = [&](float* vals, bool is_max) {
#pragma unroll
        for (int u = 0; u < VW / 4; ++u)
            reinterpret_cast<float4*>(red + tid * VW)[u] =
                make_float4(vals[4 * u], vals[4 * u + 1], vals[4 * u + 2], vals[4 * u + 3]);
        __syncthreads();
        if (active) {
#pragma unroll
            for (int v = 0; v < VW; ++v) vals[v] = is_max ? -INFINITY : 0.f;
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int u = 0; u < VW / 4; ++u) {
                    const float4 f = reinterpret_cast<const float4*>(red + (r * NGt + jl) * VW)[u];
                    const float g[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        vals[4 * u + e] = is_max ? fmaxf(vals[4 * u + e], g[e]) : vals[4 * u + e] + g[e];
                }
            }
        }
        __syncthreads();
    };
    if (R > 1) combine(mx, true);
    float sum[VW];
#pragma unroll
    for (int v = 0; v < VW; ++v) sum[v] = 0.f;
#pragma unroll
    for (int q = 0; q < kPPT; ++q) {
#pragma unroll
        for (int v = 0; v < VW; ++v) {
            const float e = (p[q][v] == -INFINITY) ? 0.f : __expf(p[q][v] - mx[v]);
            p[q][v] = e;
            sum[v] += e;
        }
    }
    if (R > 1) combine(sum, false);
#pragma unroll
    for (int v = 0; v < VW; ++v) {
        const float inv = 1.0f / sum[v];
#pragma unroll
        for (int q = 0; q < kPPT; ++q) p[q][v] *= inv;
    }

    // ---- stream the blocks assigned to this workgroup
    if (R == 1) {
        // whole blocks per thread: thread s of a channel group takes blocks
        // bc0 + s, bc0 + s + nsub, ...; two blocks' loads are in flight at once
        auto load_block = [&](long long bc, uint4* raw) {
            const long long b = bc / N;
            const long long c = bc - b * N;
            const T* __restrict__ src = x + ((size_t)b * T_len + (size_t)c * m) * C + (size_t)j * VW;
#pragma unroll
            for (int q = 0; q < kPPT; ++q)
                raw[q] = q < ppt ? ld16_stream(src + (size_t)q * C) : make_uint4(0, 0, 0, 0);
        };
        auto finish_block = [&](long long bc, const uint4* raw) {
            float acc[VW];
#pragma unroll
            for (int v = 0; v < VW; ++v) acc[v] = 0.f;
#pragma unroll
            for (int q = 0; q < kPPT; ++q) {
                if (q >= ppt) break;
                float f[VW];
                Elem<T>::unpack(raw[q], f);
#pragma unroll
                for (int v = 0; v < VW; ++v) acc[v] = fmaf(p[q][v], f[v], acc[v]);
            }
            *reinterpret_cast<uint4*>(y + (size_t)bc * C + (size_t)j * VW) = Elem<T>::pack(acc);
        };
        if (!active) return;
        for (long long bc = bc0 + s; bc < bc1; bc += 2 * nsub) {
            uint4 r0[kPPT], r1[kPPT];
            const bool two = bc + nsub < bc1;
            load_block(bc, r0);
            if (two) load_block(bc + nsub, r1);
            finish_block(bc, r0);
            if (two) finish_block(bc + nsub, r1);
        }
        return;
    }
    // R > 1: the R threads of a channel group each sum ppt positions; block
    // bc + 1 loads into the other register buffer while block bc is reduced
    // (the loop is unrolled by two so rows in flight are never copied)
    auto step = [&](long long bc, const uint4 (&cur)[kPPT], uint4 (&nxt)[kPPT]) {
        float acc[VW];
#pragma unroll
        for (int v = 0; v < VW; ++v) acc[v] = 0.f;
        if (active) {
            if (bc + 1 < bc1) load_rows(bc + 1, nxt);
#pragma unroll
            for (int q = 0; q < kPPT; ++q) {
                float f[VW];
                Elem<T>::unpack(cur[q], f);
#pragma unroll
                for (int v = 0; v < VW; ++v) acc[v] = fmaf(p[q][v], f[v], acc[v]);
            }
        }
        T* __restrict__ dst = y + (size_t)bc * C;
#pragma unroll
        for (int v = 0; v < VW; ++v) red[tid * VW + v] = acc[v];
        __syncthreads();
        // thread t finishes channel t of the tile: sum of R partials in order
        const int nch = NGt * VW;
        for (int t = tid; t < nch; t += kThreads) {
            const int jl2 = t / VW, v2 = t - jl2 * VW;
            const int j2 = blockIdx.x * NGt + jl2;
            if (j2 < NG) {
                float a = 0.f;
                for (int r = 0; r < R; ++r) a += red[(r * NGt + jl2) * VW + v2];
                Elem<T>::store1(dst + (size_t)j2 * VW + v2, a);
            }
        }
        __syncthreads();
    };
    uint4 rowsB[kPPT];
    for (long long bc = bc0; bc < bc1; bc += 2) {
        step(bc, rowsA, rowsB);
        if (bc + 1 < bc1) step(bc + 1, rowsB, rowsA);
    }
}

}  // namespace

}  // namespace shattn

using namespace shattn;

extern "C" int hca_compress_kv(const void* k, const void* v, const float* zk, const float* zv,
                               void* kc, void* vc, int B, int T, int Hkv, int d, int m,
                               int dtype, void* stream) {
    if (dtype != SHATTN_DTYPE_BF16 && dtype != SHATTN_DTYPE_F32)
        return fail(SHATTN_EINVAL, "hca_compress_kv: unknown dtype %d", dtype);
    if (B < 0 || T < 0 || Hkv < 1 || d < 1 || m < 1)
        return fail(SHATTN_EINVAL, "hca_compress_kv: bad sizes B=%d T=%d Hkv=%d d=%d m=%d", B, T,
                    Hkv, d, m);
    if (d != 64 && d != 128)
        return fail(SHATTN_EUNSUPPORTED, "hca_compress_kv: d=%d (supported: 64, 128)", d);
    if (m > 1024) return fail(SHATTN_EUNSUPPORTED, "hca_compress_kv: m=%d > 1024", m);
    const int N = T / m;
    if (B == 0 || N == 0) return SHATTN_OK;
    if (!k || !v || !zk || !zv || !kc || !vc)
        return fail(SHATTN_EINVAL, "hca_compress_kv: null pointer");
    if (!aligned16(k) || !aligned16(v) || !aligned16(kc) || !aligned16(vc) || !aligned16(zk) || !aligned16(zv))
        return fail(SHATTN_EINVAL, "hca_compress_kv: tensors must be 16-byte aligned");
    const int C = Hkv * d;
    const int VW = dtype == SHATTN_DTYPE_BF16 ? 8 : 4;
    const int NG = C / VW;
    const int ppt = m < kPPT ? m : kPPT;
    const int R = (m + ppt - 1) / ppt;
    if (R > kThreads) return fail(SHATTN_EUNSUPPORTED, "hca_compress_kv: m=%d too large", m);
    int NGt = kThreads / R;
    if (NGt > NG) NGt = NG;
    const int tiles = (NG + NGt - 1) / NGt;
    const long long total = (long long)B * N;
    // aim at ~256 workgroups per slice (about one per CU): each takes several
    // blocks, so the set-up of the softmax weights is amortised and the next
    // block's rows load while this one is summed (measured: 16 against 28 µs
    // for one 128-row block per workgroup at 32K rows x 2 KV heads); whole-block
    // threads (R == 1) take several blocks each
    const int nsub = kThreads / NGt;
    long long per = (total * tiles + 255) / 256;
    if (R == 1) per = ((per + 2 * nsub - 1) / (2 * nsub)) * (2 * nsub);
    if (per < 1) per = 1;
    if (per > 4096) per = 4096;
    const long long ywgs = (total + per - 1) / per;
    if (ywgs > 2147483647LL) return fail(SHATTN_EUNSUPPORTED, "hca_compress_kv: too many blocks");
    dim3 grid(tiles, (unsigned)ywgs, 2);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (dtype == SHATTN_DTYPE_BF16) {
        hipLaunchKernelGGL(compress_kernel<bf16_t>, grid, dim3(kThreads), 0, s,
                           (const bf16_t*)k, (const bf16_t*)v, zk, zv, (bf16_t*)kc, (bf16_t*)vc,
                           T, C, m, N, R, NGt, total, (int)per);
    } else {
        hipLaunchKernelGGL(compress_kernel<float>, grid, dim3(kThreads), 0, s, (const float*)k,
                           (const float*)v, zk, zv, (float*)kc, (float*)vc, T, C, m, N, R, NGt,
                           total, (int)per);
    }
    return check_launch("hca_compress_kv");
}

// ---------------------------------------------------------------------------
// Both ratios in one pass: every raw row is read once and feeds the CSA entry
// (ratio m1 <= 8, m1 | 8) and the HCA entry (ratio m2, 8 | m2) it belongs to.
// Thread = (channel group j, 8 consecutive rows s of an m2-block).  The m1
// entries are complete inside the thread; the m2 partial sums of the R = m2/8
// threads of a channel group are combined in LDS in a fixed order.
namespace shattn {
namespace {

template <typename T, int M1, int PPT>
__global__ __launch_bounds__(kThreads) void compress_dual_kernel(
    const T* __restrict__ x0, const T* __restrict__ x1,
    const float* __restrict__ za0, const float* __restrict__ za1, T* __restrict__ ya0, T* __restrict__ ya1,
    const float* __restrict__ zb0, const float* __restrict__ zb1, T* __restrict__ yb0, T* __restrict__ yb1, int m2,
    int T_len, int C, int N1, int N2, int R, int NGt, long long total_blocks, int blocks_per_wg) {
    constexpr int VW = Elem<T>::kVec;
    static_assert(PPT % M1 == 0, "a thread must cover whole m1-blocks");
    const bool second = blockIdx.z != 0;
    const T* __restrict__ x = second ? x1 : x0;
    const float* __restrict__ za = second ? za1 : za0;
    const float* __restrict__ zb = second ? zb1 : zb0;
    T* __restrict__ ya = second ? ya1 : ya0;
    T* __restrict__ yb = second ? yb1 : yb0;

    __shared__ float red[2][kThreads * VW];

    const int NG = C / VW;
    const int tid = threadIdx.x;
    const int s = tid / NGt;
    const int jl = tid - s * NGt;
    const int j = blockIdx.x * NGt + jl;
    const bool active = (s < R) && (j < NG);

    const long long bc0 = (long long)blockIdx.y * blocks_per_wg;
    long long bc1 = bc0 + blocks_per_wg;
    if (bc1 > total_blocks) bc1 = total_blocks;
    auto load_rows = [&](long long bc, uint4* raw) {
        const long long b = bc / N2;
        const long long c = bc - b * N2;
        const T* __restrict__ src = x + ((size_t)b * T_len + (size_t)c * m2 + (size_t)s * PPT) * C + (size_t)j * VW;
#pragma unroll
        for (int q = 0; q < PPT; ++q) raw[q] = ld16_stream(src + (size_t)q * C);
    };
    uint4 nxt[PPT];
    if (active && bc0 < bc1) load_rows(bc0, nxt);   // first block in flight during the setup

    // ---- m2 weights of this thread's PPT positions (softmax over all m2 positions)
    float pb[PPT][VW];
    float mx[VW];
#pragma unroll
    for (int v = 0; v < VW; ++v) mx[v] = -INFINITY;
    // logits of this thread's PPT positions, VW channels: 16-byte loads
    auto load_logits = [&](const float* z, int i, float* out) {
        const float4* src = reinterpret_cast<const float4*>(z + (size_t)i * C + (size_t)j * VW);
#pragma unroll
        for (int u = 0; u < VW / 4; ++u) {
            const float4 f = src[u];
            out[4 * u + 0] = f.x;
            out[4 * u + 1] = f.y;
            out[4 * u + 2] = f.z;
            out[4 * u + 3] = f.w;
        }
    };
    if (active) {
#pragma unroll
        for (int q = 0; q < PPT; ++q) load_logits(zb, s * PPT + q, pb[q]);
    } else {
#pragma unroll
        for (int q = 0; q < PPT; ++q)
#pragma unroll
            for (int v = 0; v < VW; ++v) pb[q][v] = -INFINITY;
    }
#pragma unroll
    for (int q = 0; q < PPT; ++q)
#pragma unroll
        for (int v = 0; v < VW; ++v) mx[v] = fmaxf(mx[v], pb[q][v]);
    // per-thread partials -> LDS; the R partials of a channel group combine in a
    // fixed order (16-byte LDS reads)
    auto reduce_rows = [&](float* buf, const float* mine, float* out, bool is_max) {
#pragma unroll
        for (int u = 0; u < VW / 4; ++u)
            reinterpret_cast<float4*>(buf + tid * VW)[u] =
                make_float4(mine[4 * u], mine[4 * u + 1], mine[4 * u + 2], mine[4 * u + 3]);
        __syncthreads();
        if (active) {
#pragma unroll
            for (int v = 0; v < VW; ++v) out[v] = is_max ? -INFINITY : 0.f;
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int u = 0; u < VW / 4; ++u) {
                    const float4 f = reinterpret_cast<const float4*>(buf + (r * NGt + jl) * VW)[u];
                    const float g[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        out[4 * u + e] = is_max ? fmaxf(out[4 * u + e], g[e]) : out[4 * u + e] + g[e];
                }
            }
        }
    };
    {
        float part[VW];
#pragma unroll
        for (int v = 0; v < VW; ++v) part[v] = mx[v];
        reduce_rows(red[0], part, mx, true);
    }
    float sum[VW];
#pragma unroll
    for (int v = 0; v < VW; ++v) sum[v] = 0.f;
#pragma unroll
    for (int q = 0; q < PPT; ++q)
#pragma unroll
        for (int v = 0; v < VW; ++v) {
            const float e = active ? __expf(pb[q][v] - mx[v]) : 0.f;
            pb[q][v] = e;
            sum[v] += e;
        }
    {
        float tot[VW];
        reduce_rows(red[1], sum, tot, false);
        if (active) {
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                const float inv = 1.0f / tot[v];
#pragma unroll
                for (int q = 0; q < PPT; ++q) pb[q][v] *= inv;
            }
        }
    }
    // ---- m1 weights (the thread sees whole m1-blocks)
    float pa[M1][VW];
    {
        float am[VW], as[VW];
#pragma unroll
        for (int v = 0; v < VW; ++v) { am[v] = -INFINITY; as[v] = 0.f; }
        if (active) {
#pragma unroll
            for (int q = 0; q < M1; ++q) load_logits(za, q, pa[q]);
        } else {
#pragma unroll
            for (int q = 0; q < M1; ++q)
#pragma unroll
                for (int v = 0; v < VW; ++v) pa[q][v] = 0.f;
        }
#pragma unroll
        for (int q = 0; q < M1; ++q)
#pragma unroll
            for (int v = 0; v < VW; ++v) am[v] = fmaxf(am[v], pa[q][v]);
#pragma unroll
        for (int q = 0; q < M1; ++q)
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                pa[q][v] = __expf(pa[q][v] - am[v]);
                as[v] += pa[q][v];
            }
#pragma unroll
        for (int v = 0; v < VW; ++v) {
            const float inv = 1.0f / as[v];
#pragma unroll
            for (int q = 0; q < M1; ++q) pa[q][v] *= inv;
        }
    }
    __syncthreads();

    // One block: compute from `cur` while the next block's rows load into
    // `nxt`.  The two register buffers alternate by unrolling the block loop
    // by two, so rows in flight are never copied (a copy would wait for them).
    auto step = [&](long long bc, const uint4 (&cur)[PPT], uint4 (&nxt)[PPT], int buf) {
        const long long b = bc / N2;
        const long long c = bc - b * N2;
        float acc[VW];
#pragma unroll
        for (int v = 0; v < VW; ++v) acc[v] = 0.f;
        if (active) {
            const long long row0 = (long long)c * m2 + (long long)s * PPT;  // first row in the sequence
            if (bc + 1 < bc1) load_rows(bc + 1, nxt);   // next block's rows in flight
            float o[VW];
#pragma unroll
            for (int q = 0; q < PPT; ++q) {
                float f[VW];
                Elem<T>::unpack(cur[q], f);
                if (q % M1 == 0) {
#pragma unroll
                    for (int v = 0; v < VW; ++v) o[v] = 0.f;
                }
#pragma unroll
                for (int v = 0; v < VW; ++v) {
                    acc[v] = fmaf(pb[q][v], f[v], acc[v]);
                    o[v] = fmaf(pa[q % M1][v], f[v], o[v]);
                }
                if (q % M1 == M1 - 1) {
                    const long long e1 = (row0 + q) / M1;   // entry index of ratio m1
                    *reinterpret_cast<uint4*>(ya + ((size_t)b * N1 + e1) * C + (size_t)j * VW) = Elem<T>::pack(o);
                }
            }
        }
        float* r = red[buf];
#pragma unroll
        for (int v = 0; v < VW; ++v) r[tid * VW + v] = acc[v];
        __syncthreads();   // (waits for LDS only: the rows in flight stay in flight)
        T* __restrict__ dst = yb + (size_t)bc * C;
        // channel ch of the tile is summed by 4 consecutive threads (R/4 partials
        // each), then combined in a fixed order across those 4 lanes
        const int nch = NGt * VW;
        const int quarter = (R + 3) / 4;
        for (int t0 = 0; t0 < 4 * nch; t0 += kThreads) {
            const int t = t0 + tid;
            const int ch = t >> 2, part = t & 3;
            float a = 0.f;
            if (ch < nch) {
                const int jl2 = ch / VW, v2 = ch - jl2 * VW;
                const int r0 = part * quarter, r1 = min(R, r0 + quarter);
                for (int rr = r0; rr < r1; ++rr) a += r[(rr * NGt + jl2) * VW + v2];
            }
            const float a1 = __shfl_xor(a, 1);
            const float lo = (part & 1) ? a1 + a : a + a1;          // (p0+p1) or (p2+p3)
            const float hi = __shfl_xor(lo, 2);
            const float tot = (part & 2) ? hi + lo : lo + hi;       // (p0+p1)+(p2+p3)
            if (ch < nch && part == 0) {
                const int jl2 = ch / VW, v2 = ch - jl2 * VW;
                const int j2 = blockIdx.x * NGt + jl2;
                if (j2 < NG) Elem<T>::store1(dst + (size_t)j2 * VW + v2, tot);
            }
        }
        // the next block writes the other red buffer: one barrier per block
    };
    uint4 nxt2[PPT];
    for (long long bc = bc0; bc < bc1; bc += 2) {
        step(bc, nxt, nxt2, 0);
        if (bc + 1 < bc1) step(bc + 1, nxt2, nxt, 1);
    }
}

template <typename E, int M1, int PPT>
void launch_dual(dim3 grid, hipStream_t st, const void* k, const void* v, const float* zk1, const float* zv1,
                 void* kc1, void* vc1, const float* zk2, const float* zv2, void* kc2, void* vc2, int m2, int Tl,
                 int C, int N1, int N2, int R, int NGt, long long total, int per) {
    hipLaunchKernelGGL((compress_dual_kernel<E, M1, PPT>), grid, dim3(kThreads), 0, st, (const E*)k, (const E*)v,
                       zk1, zv1, (E*)kc1, (E*)vc1, zk2, zv2, (E*)kc2, (E*)vc2, m2, Tl, C, N1, N2, R, NGt, total,
                       per);
}

template <typename E>
void launch_dual_m1(int m1, dim3 grid, hipStream_t st, const void* k, const void* v, const float* zk1,
                    const float* zv1, void* kc1, void* vc1, const float* zk2, const float* zv2, void* kc2, void* vc2,
                    int m2, int Tl, int C, int N1, int N2, int R, int NGt, long long total, int per) {
#define SHATTN_DUAL(M1, P) launch_dual<E, M1, P>(grid, st, k, v, zk1, zv1, kc1, vc1, zk2, zv2, kc2, vc2, m2, Tl, C, \
                                                 N1, N2, R, NGt, total, per)
    switch (m1) {
        case 1: SHATTN_DUAL(1, 4); break;
        case 2: SHATTN_DUAL(2, 4); break;
        case 4: SHATTN_DUAL(4, 4); break;
        default: SHATTN_DUAL(8, 8); break;
    }
#undef SHATTN_DUAL
}

}  // namespace
}  // namespace shattn

extern "C" int hca_compress_kv_dual(const void* k, const void* v, const float* zk1, const float* zv1, void* kc1,
                                    void* vc1, int m1, const float* zk2, const float* zv2, void* kc2, void* vc2,
                                    int m2, int B, int T, int Hkv, int d, int dtype, void* stream) {
    if (dtype != SHATTN_DTYPE_BF16 && dtype != SHATTN_DTYPE_F32)
        return fail(SHATTN_EINVAL, "hca_compress_kv_dual: unknown dtype %d", dtype);
    if (B < 0 || T < 0 || Hkv < 1 || d < 1 || m1 < 1 || m2 < 1)
        return fail(SHATTN_EINVAL, "hca_compress_kv_dual: bad sizes B=%d T=%d Hkv=%d d=%d m1=%d m2=%d", B, T,
                    Hkv, d, m1, m2);
    if (d != 64 && d != 128)
        return fail(SHATTN_EUNSUPPORTED, "hca_compress_kv_dual: d=%d (supported: 64, 128)", d);
    if (8 % m1 != 0 || m2 % 8 != 0 || m2 > 1024)
        return fail(SHATTN_EUNSUPPORTED,
                    "hca_compress_kv_dual: needs m1 in {1,2,4,8} and m2 a multiple of 8 up to 1024 (m1=%d m2=%d)",
                    m1, m2);
    const int N1 = T / m1, N2 = T / m2;
    if (B == 0 || N1 == 0) return SHATTN_OK;
    if (!k || !v || !zk1 || !zv1 || !kc1 || !vc1 || !zk2 || !zv2 || (N2 > 0 && (!kc2 || !vc2)))
        return fail(SHATTN_EINVAL, "hca_compress_kv_dual: null pointer");
    if (!aligned16(k) || !aligned16(v) || !aligned16(kc1) || !aligned16(vc1) || !aligned16(zk1) ||
        !aligned16(zv1) || !aligned16(zk2) || !aligned16(zv2) || (N2 > 0 && (!aligned16(kc2) || !aligned16(vc2))))
        return fail(SHATTN_EINVAL, "hca_compress_kv_dual: tensors must be 16-byte aligned");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // the rows past the last full m2-block only feed ratio m1: compress them on their own
    const int tail_rows = T - N2 * m2;
    if (N2 > 0) {
        const int C = Hkv * d;
        const int VW = dtype == SHATTN_DTYPE_BF16 ? 8 : 4;
        const int NG = C / VW;
        const int ppt = m1 == 8 ? 8 : 4;
        const int R = m2 / ppt;
        if (R > kThreads) return fail(SHATTN_EUNSUPPORTED, "hca_compress_kv_dual: m2=%d too large", m2);
        int NGt = kThreads / R;
        if (NGt > NG) NGt = NG;
        const int tiles = (NG + NGt - 1) / NGt;
        const long long total = (long long)B * N2;
        // about one resident round of workgroups (3 per CU, K and V slices): the
        // per-workgroup set-up (softmax weights of both ratios) is amortised
        // over many blocks
        long long per = (total * tiles * 2 + 767) / 768;
        if (per < 2) per = 2;
        if (per > 64) per = 64;
        const long long ywgs = (total + per - 1) / per;
        dim3 grid(tiles, (unsigned)ywgs, 2);
        if (dtype == SHATTN_DTYPE_BF16)
            launch_dual_m1<bf16_t>(m1, grid, s, k, v, zk1, zv1, kc1, vc1, zk2, zv2, kc2, vc2, m2, T, C, N1, N2, R,
                                   NGt, total, (int)per);
        else
            launch_dual_m1<float>(m1, grid, s, k, v, zk1, zv1, kc1, vc1, zk2, zv2, kc2, vc2, m2, T, C, N1, N2, R,
                                  NGt, total, (int)per);
        const int rc = check_launch("hca_compress_kv_dual");
        if (rc) return rc;
    }
    if (tail_rows >= m1) {
        // entries of ratio m1 past the last m2-block: [N2*m2/m1, N1)
        const long long e0 = (long long)N2 * m2 / m1;
        const size_t esz = dtype == SHATTN_DTYPE_BF16 ? 2 : 4;
        const size_t C = (size_t)Hkv * d;
        for (int b = 0; b < B; ++b) {
            const char* kb = (const char*)k + ((size_t)b * T + (size_t)N2 * m2) * C * esz;
            const char* vb = (const char*)v + ((size_t)b * T + (size_t)N2 * m2) * C * esz;
            char* kcb = (char*)kc1 + ((size_t)b * N1 + e0) * C * esz;
            char* vcb = (char*)vc1 + ((size_t)b * N1 + e0) * C * esz;
            const int rc = hca_compress_kv(kb, vb, zk1, zv1, kcb, vcb, 1, tail_rows, Hkv, d, m1, dtype, stream);
            if (rc) return rc;
        }
    }
    return SHATTN_OK;
}
