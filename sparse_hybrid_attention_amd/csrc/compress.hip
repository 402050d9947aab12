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
    const int s = tid / NGt;          // position subset
    const int jl = tid - s * NGt;     // channel group within the tile
    const int j = blockIdx.x * NGt + jl;
    const bool active = (s < R) && (j < NG);
    const int ppt = (m < kPPT) ? m : kPPT;

    // ---- softmax weights of this thread's positions and channels
    float p[kPPT][VW];
    float mx[VW];
#pragma unroll
    for (int v = 0; v < VW; ++v) mx[v] = -INFINITY;
#pragma unroll
    for (int q = 0; q < kPPT; ++q) {
        const int i = s * ppt + q;
        const bool ok = active && q < ppt && i < m;
#pragma unroll
        for (int v = 0; v < VW; ++v) {
            p[q][v] = ok ? z[(size_t)i * C + (size_t)j * VW + v] : -INFINITY;
            mx[v] = fmaxf(mx[v], p[q][v]);
        }
    }
    if (R > 1) {
#pragma unroll
        for (int v = 0; v < VW; ++v) red[tid * VW + v] = mx[v];
        __syncthreads();
        if (active) {
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                float a = -INFINITY;
                for (int r = 0; r < R; ++r) a = fmaxf(a, red[(r * NGt + jl) * VW + v]);
                mx[v] = a;
            }
        }
        __syncthreads();
    }
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
    if (R > 1) {
#pragma unroll
        for (int v = 0; v < VW; ++v) red[tid * VW + v] = sum[v];
        __syncthreads();
        if (active) {
#pragma unroll
            for (int v = 0; v < VW; ++v) {
                float a = 0.f;
                for (int r = 0; r < R; ++r) a += red[(r * NGt + jl) * VW + v];
                sum[v] = a;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int v = 0; v < VW; ++v) {
        const float inv = 1.0f / sum[v];
#pragma unroll
        for (int q = 0; q < kPPT; ++q) p[q][v] *= inv;
    }

    // ---- stream the blocks assigned to this workgroup
    const long long bc0 = (long long)blockIdx.y * blocks_per_wg;
    long long bc1 = bc0 + blocks_per_wg;
    if (bc1 > total_blocks) bc1 = total_blocks;
    for (long long bc = bc0; bc < bc1; ++bc) {
        const long long b = bc / N;
        const long long c = bc - b * N;
        float acc[VW];
#pragma unroll
        for (int v = 0; v < VW; ++v) acc[v] = 0.f;
        if (active) {
            const T* __restrict__ src =
                x + ((size_t)b * T_len + (size_t)c * m + (size_t)s * ppt) * C + (size_t)j * VW;
            uint4 raw[kPPT];
#pragma unroll
            for (int q = 0; q < kPPT; ++q) {
                if (q < ppt && s * ppt + q < m)
                    raw[q] = ld16_stream(src + (size_t)q * C);
                else
                    raw[q] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < kPPT; ++q) {
                float f[VW];
                Elem<T>::unpack(raw[q], f);
#pragma unroll
                for (int v = 0; v < VW; ++v) acc[v] = fmaf(p[q][v], f[v], acc[v]);
            }
        }
        T* __restrict__ dst = y + (size_t)bc * C;
        if (R == 1) {
            if (active)
                *reinterpret_cast<uint4*>(dst + (size_t)j * VW) = Elem<T>::pack(acc);
        } else {
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
        }
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
    if (!aligned16(k) || !aligned16(v) || !aligned16(kc) || !aligned16(vc))
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
    // aim at ~2048 workgroups (8 per CU) per slice
    long long per = (total * tiles + 2047) / 2048;
    if (per < 1) per = 1;
    if (per > 64) per = 64;
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
