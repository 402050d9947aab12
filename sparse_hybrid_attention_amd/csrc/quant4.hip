// 4-bit storage of a compressed cache: encode with one minimum and one step
// over the whole tensor, decode back to the storage dtype.
//
// Page: [V4-code] CSDN article with CSA/HCA example code, section "1. HCA"
// (the merged cache is stored in 4 bits: one minimum and one maximum over the
// tensor, step (max - min) / 15, codes rounded and clamped to 0..15, decoded
// as code * step + min; two codes per byte named as the real layout).  The
// code decision is float32 (x - min) / step with round-half-even; element 2j
// goes to the low nibble of byte j.
//
// Encode is three launches on the caller's stream: the two-word params buffer
// is first set to the identity keys of a min and a max, every workgroup then
// folds its wave-reduced extremes in with one atomic min and one atomic max
// on order-preserving integer keys of the floats, and one thread turns the
// keys into (min, step) in place; a fourth launch writes the codes, one
// thread per output byte.  Decode is one launch, one thread per byte.  The
// work is HBM-bound (a read of the tensor per pass, a write of n/2 bytes).
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "hybrid_attn.h"

namespace shattn {
namespace {

constexpr int kQ4Threads = 256;
// the min / max pass: every workgroup ends in two atomics on the same two
// words, which the memory system serialises, so the pass keeps to one
// workgroup per CU (2048 workgroups spent about 50 us in those atomics alone)
constexpr long long kQ4MinMaxGroups = 256;

// float -> uint32 with the same order (finite values and infinities)
__device__ __forceinline__ uint32_t ord_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_val(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__global__ void q4_init_kernel(uint32_t* keys) {
    keys[0] = 0xFFFFFFFFu;   // running minimum key
    keys[1] = 0u;            // running maximum key
}

template <typename T>
__global__ __launch_bounds__(kQ4Threads) void q4_minmax_kernel(const T* __restrict__ x, long long n, bool vec,
                                                               uint32_t* keys) {
    constexpr int VW = Elem<T>::kVec;
    float mn = INFINITY, mx = -INFINITY;
    const long long stride = (long long)gridDim.x * kQ4Threads;
    const long long gid = (long long)blockIdx.x * kQ4Threads + threadIdx.x;
    // 16-byte loads over the aligned body (min and max do not depend on the
    // order), single elements for the rest
    const long long nv = vec ? n / VW : 0;
    for (long long v = gid; v < nv; v += stride) {
        float f[VW];
        Elem<T>::unpack(ld16(x + v * VW), f);
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            mn = fminf(mn, f[e]);
            mx = fmaxf(mx, f[e]);
        }
    }
    for (long long i = nv * VW + gid; i < n; i += stride) {
        const float v = Elem<T>::load1(x + i);
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    __shared__ float smn[kQ4Threads / 64], smx[kQ4Threads / 64];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        smn[wave] = mn;
        smx[wave] = mx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kQ4Threads / 64; ++w) {
            mn = fminf(mn, smn[w]);
            mx = fmaxf(mx, smx[w]);
        }
        atomicMin(keys, ord_key(mn));
        atomicMax(keys + 1, ord_key(mx));
    }
}

__global__ void q4_finalize_kernel(uint32_t* keys) {
    const float mn = ord_val(keys[0]), mx = ord_val(keys[1]);
    float* params = reinterpret_cast<float*>(keys);
    params[0] = mn;
    params[1] = (mx - mn) / 15.0f;   // float32, correctly rounded
}

template <typename T>
__global__ __launch_bounds__(kQ4Threads) void q4_encode_kernel(const T* __restrict__ x, long long n,
                                                               const float* __restrict__ params,
                                                               uint8_t* __restrict__ codes) {
    const float mn = params[0], st = params[1];
    const long long nbytes = (n + 1) / 2;
    const long long stride = (long long)gridDim.x * kQ4Threads;
    for (long long j = (long long)blockIdx.x * kQ4Threads + threadIdx.x; j < nbytes; j += stride) {
        uint32_t c[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const long long i = 2 * j + e;
            if (i < n && st != 0.0f) {
                const float t = (Elem<T>::load1(x + i) - mn) / st;
                c[e] = (uint32_t)fminf(fmaxf(rintf(t), 0.0f), 15.0f);
            }
        }
        codes[j] = (uint8_t)(c[0] | (c[1] << 4));
    }
}

// The decoded value code * step + min rounded once to the storage dtype: the
// product of a 4-bit code and a float32 step is exact in float64 and the sum
// is rounded once to float64 there, then once to the dtype.
template <typename T> __device__ __forceinline__ void store_decoded(T* p, double v);
template <> __device__ __forceinline__ void store_decoded<float>(float* p, double v) { *p = (float)v; }
template <> __device__ __forceinline__ void store_decoded<bf16_t>(bf16_t* p, double v) {
    *p = (bf16_t)f64_to_bf16_rne(v);
}

template <typename T>
__global__ __launch_bounds__(kQ4Threads) void q4_decode_kernel(const uint8_t* __restrict__ codes,
                                                               const float* __restrict__ params, long long n,
                                                               T* __restrict__ out) {
    const double mn = params[0], st = params[1];
    const long long nbytes = (n + 1) / 2;
    const long long stride = (long long)gridDim.x * kQ4Threads;
    for (long long j = (long long)blockIdx.x * kQ4Threads + threadIdx.x; j < nbytes; j += stride) {
        const uint32_t b = codes[j];
        store_decoded<T>(out + 2 * j, fma((double)(b & 15u), st, mn));
        if (2 * j + 1 < n) store_decoded<T>(out + 2 * j + 1, fma((double)(b >> 4), st, mn));
    }
}

unsigned grid_for(long long units, long long cap) {
    long long g = (units + kQ4Threads - 1) / kQ4Threads;
    if (g > cap) g = cap;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace
}  // namespace shattn

extern "C" int cache_quant4(const void* x, int64_t n, int32_t dtype, uint8_t* codes, float* params, void* stream) {
    using namespace shattn;
    if (dtype != SHATTN_DTYPE_BF16 && dtype != SHATTN_DTYPE_F32)
        return fail(SHATTN_EINVAL, "cache_quant4: unknown dtype %d", dtype);
    if (n < 0) return fail(SHATTN_EINVAL, "cache_quant4: n=%lld < 0", (long long)n);
    if (n == 0) return SHATTN_OK;
    if (!x || !codes || !params) return fail(SHATTN_EINVAL, "cache_quant4: null pointer");
    const size_t esz = dtype == SHATTN_DTYPE_BF16 ? 2 : 4;
    if ((reinterpret_cast<uintptr_t>(x) % esz) != 0 || (reinterpret_cast<uintptr_t>(params) % 4) != 0)
        return fail(SHATTN_EINVAL, "cache_quant4: x must be %zu-byte and params 4-byte aligned", esz);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint32_t* keys = reinterpret_cast<uint32_t*>(params);
    hipLaunchKernelGGL(q4_init_kernel, dim3(1), dim3(1), 0, s, keys);
    if (dtype == SHATTN_DTYPE_BF16)
        hipLaunchKernelGGL((q4_minmax_kernel<bf16_t>), dim3(grid_for(n / 8, kQ4MinMaxGroups)), dim3(kQ4Threads), 0, s,
                           static_cast<const bf16_t*>(x), (long long)n, aligned16(x), keys);
    else
        hipLaunchKernelGGL((q4_minmax_kernel<float>), dim3(grid_for(n / 4, kQ4MinMaxGroups)), dim3(kQ4Threads), 0, s,
                           static_cast<const float*>(x), (long long)n, aligned16(x), keys);
    hipLaunchKernelGGL(q4_finalize_kernel, dim3(1), dim3(1), 0, s, keys);
    const long long nbytes = ((long long)n + 1) / 2;
    if (dtype == SHATTN_DTYPE_BF16)
        hipLaunchKernelGGL((q4_encode_kernel<bf16_t>), dim3(grid_for(nbytes, 1 << 20)), dim3(kQ4Threads), 0, s,
                           static_cast<const bf16_t*>(x), (long long)n, params, codes);
    else
        hipLaunchKernelGGL((q4_encode_kernel<float>), dim3(grid_for(nbytes, 1 << 20)), dim3(kQ4Threads), 0, s,
                           static_cast<const float*>(x), (long long)n, params, codes);
    return check_launch("cache_quant4");
}

extern "C" int cache_dequant4(const uint8_t* codes, const float* params, int64_t n, int32_t dtype, void* out,
                              void* stream) {
    using namespace shattn;
    if (dtype != SHATTN_DTYPE_BF16 && dtype != SHATTN_DTYPE_F32)
        return fail(SHATTN_EINVAL, "cache_dequant4: unknown dtype %d", dtype);
    if (n < 0) return fail(SHATTN_EINVAL, "cache_dequant4: n=%lld < 0", (long long)n);
    if (n == 0) return SHATTN_OK;
    if (!codes || !params || !out) return fail(SHATTN_EINVAL, "cache_dequant4: null pointer");
    const size_t esz = dtype == SHATTN_DTYPE_BF16 ? 2 : 4;
    if ((reinterpret_cast<uintptr_t>(out) % esz) != 0 || (reinterpret_cast<uintptr_t>(params) % 4) != 0)
        return fail(SHATTN_EINVAL, "cache_dequant4: out must be %zu-byte and params 4-byte aligned", esz);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const long long nbytes = ((long long)n + 1) / 2;
    if (dtype == SHATTN_DTYPE_BF16)
        hipLaunchKernelGGL((q4_decode_kernel<bf16_t>), dim3(grid_for(nbytes, 1 << 20)), dim3(kQ4Threads), 0, s,
                           codes, params, (long long)n, static_cast<bf16_t*>(out));
    else
        hipLaunchKernelGGL((q4_decode_kernel<float>), dim3(grid_for(nbytes, 1 << 20)), dim3(kQ4Threads), 0, s,
                           codes, params, (long long)n, static_cast<float*>(out));
    return check_launch("cache_dequant4");
}
