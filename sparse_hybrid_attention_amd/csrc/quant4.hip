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
// Encode is three launches on the caller's stream: the two-word params
// buffer is first set to the identity keys of a min and a max; every
// workgroup then folds its wave-reduced extremes in with one atomic min and
// one atomic max on order-preserving integer keys of the floats, and the last
// workgroup to finish (a counter the first launch zeroed, kept in the first
// four bytes of the codes, which the third launch then overwrites) turns the
// keys into (min, step) in place; the third launch writes the codes, eight
// elements (bf16) or four (fp32) per 16-byte load.  Decode is one launch:
// each workgroup decodes the sixteen codes into LDS once, and every thread
// expands four code bytes into eight stored elements.  The work is HBM-bound
// (a read of the tensor per pass, a write of n/2 bytes).
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

__global__ void q4_init_kernel(uint32_t* keys, uint32_t* counter) {
    keys[0] = 0xFFFFFFFFu;   // running minimum key
    keys[1] = 0u;            // running maximum key
    if (counter) *counter = 0u;
}

// (min, step) from the final keys, written over them: float32 (max - min) / 15
// correctly rounded
__device__ __forceinline__ void q4_write_params(uint32_t* keys, uint32_t kmin, uint32_t kmax) {
    const float mn = ord_val(kmin), mx = ord_val(kmax);
    float* params = reinterpret_cast<float*>(keys);
    params[0] = mn;
    params[1] = (mx - mn) / 15.0f;
}

template <typename T>
__global__ __launch_bounds__(kQ4Threads) void q4_minmax_kernel(const T* __restrict__ x, long long n, bool vec,
                                                               uint32_t* keys, uint32_t* counter) {
    constexpr int VW = Elem<T>::kVec;
    float mn = INFINITY, mx = -INFINITY;
    const long long stride = (long long)gridDim.x * kQ4Threads;
    const long long gid = (long long)blockIdx.x * kQ4Threads + threadIdx.x;
    // 16-byte loads over the aligned body (min and max do not depend on the
    // order), single elements for the rest
    const long long nv = vec ? n / VW : 0;
    // four 16-byte loads in flight per lane
    constexpr int U = 4;
    long long v = gid;
    for (; v + (U - 1) * stride < nv; v += U * stride) {
        uint4 u[U];
#pragma unroll
        for (int k = 0; k < U; ++k) u[k] = ld16(x + (v + k * stride) * VW);
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float f[VW];
            Elem<T>::unpack(u[k], f);
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                mn = fminf(mn, f[e]);
                mx = fmaxf(mx, f[e]);
            }
        }
    }
    for (; v < nv; v += stride) {
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
        if (counter) {
            // the last workgroup sees every other workgroup's atomics (each
            // made them before its fence and its count)
            __threadfence();
            if (atomicAdd(counter, 1u) == gridDim.x - 1) {
                __threadfence();
                q4_write_params(keys, atomicOr(keys, 0u), atomicOr(keys + 1, 0u));
            }
        }
    }
}

// without a counter (fewer than four code bytes, or codes not 4-byte aligned)
__global__ void q4_finalize_kernel(uint32_t* keys) { q4_write_params(keys, keys[0], keys[1]); }

template <typename T> __device__ __forceinline__ uint32_t q4_code(float v, float mn, float st) {
    const float t = (v - mn) / st;
    return (uint32_t)fminf(fmaxf(rintf(t), 0.0f), 15.0f);
}

// VW elements of one 16-byte load -> VW / 2 code bytes (4 for bf16, 2 for
// fp32) stored as one word when `vec` (x 16-byte and codes VW/2-byte
// aligned); the rest one byte per thread
template <typename T>
__global__ __launch_bounds__(kQ4Threads) void q4_encode_kernel(const T* __restrict__ x, long long n, bool vec,
                                                               const float* __restrict__ params,
                                                               uint8_t* __restrict__ codes) {
    constexpr int VW = Elem<T>::kVec;
    const float mn = params[0], st = params[1];
    const long long stride = (long long)gridDim.x * kQ4Threads;
    const long long gid = (long long)blockIdx.x * kQ4Threads + threadIdx.x;
    const long long nv = vec ? n / VW : 0;
    for (long long v = gid; v < nv; v += stride) {
        float f[VW];
        Elem<T>::unpack(ld16(x + v * VW), f);
        uint32_t word = 0u;
        if (st != 0.0f) {
#pragma unroll
            for (int e = 0; e < VW; ++e) word |= q4_code<T>(f[e], mn, st) << (4 * e);
        }
        if constexpr (VW == 8)
            reinterpret_cast<uint32_t*>(codes)[v] = word;
        else
            reinterpret_cast<uint16_t*>(codes)[v] = (uint16_t)word;
    }
    const long long nbytes = (n + 1) / 2;
    for (long long j = nv * (VW / 2) + gid; j < nbytes; j += stride) {
        uint32_t c[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const long long i = 2 * j + e;
            if (i < n && st != 0.0f) c[e] = q4_code<T>(Elem<T>::load1(x + i), mn, st);
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

template <typename T> __device__ __forceinline__ uint32_t dec_bits(const T* lut, uint32_t code);
template <> __device__ __forceinline__ uint32_t dec_bits<bf16_t>(const bf16_t* lut, uint32_t code) {
    return (uint32_t)lut[code];
}
template <> __device__ __forceinline__ uint32_t dec_bits<float>(const float* lut, uint32_t code) {
    return __float_as_uint(lut[code]);
}

// Four code bytes -> eight elements per thread when `vec` (codes 4-byte and
// out 16-byte aligned), from the sixteen decoded values the workgroup puts in
// LDS first; the rest one byte per thread
template <typename T>
__global__ __launch_bounds__(kQ4Threads) void q4_decode_kernel(const uint8_t* __restrict__ codes,
                                                               const float* __restrict__ params, long long n,
                                                               bool vec, T* __restrict__ out) {
    __shared__ T lut[16];
    if (threadIdx.x < 16) {
        const double mn = params[0], st = params[1];
        store_decoded<T>(&lut[threadIdx.x], fma((double)threadIdx.x, st, mn));
    }
    __syncthreads();
    const long long stride = (long long)gridDim.x * kQ4Threads;
    const long long gid = (long long)blockIdx.x * kQ4Threads + threadIdx.x;
    const long long nw = vec ? n / 8 : 0;   // whole 4-byte code words
    for (long long v = gid; v < nw; v += stride) {
        const uint32_t cw = reinterpret_cast<const uint32_t*>(codes)[v];
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = dec_bits<T>(lut, (cw >> (4 * e)) & 15u);
        if constexpr (sizeof(T) == 2) {
            reinterpret_cast<uint4*>(out)[v] =
                make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
        } else {
            reinterpret_cast<uint4*>(out)[2 * v] = make_uint4(b[0], b[1], b[2], b[3]);
            reinterpret_cast<uint4*>(out)[2 * v + 1] = make_uint4(b[4], b[5], b[6], b[7]);
        }
    }
    const long long nbytes = (n + 1) / 2;
    for (long long j = nw * 4 + gid; j < nbytes; j += stride) {
        const uint32_t bb = codes[j];
        out[2 * j] = lut[bb & 15u];
        if (2 * j + 1 < n) out[2 * j + 1] = lut[bb >> 4];
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
    const long long nbytes = ((long long)n + 1) / 2;
    // the last-workgroup counter lives in the first code word until the
    // encode launch overwrites it
    uint32_t* counter = (nbytes >= 4 && (reinterpret_cast<uintptr_t>(codes) % 4) == 0)
                            ? reinterpret_cast<uint32_t*>(codes) : nullptr;
    hipLaunchKernelGGL(q4_init_kernel, dim3(1), dim3(1), 0, s, keys, counter);
    if (dtype == SHATTN_DTYPE_BF16)
        hipLaunchKernelGGL((q4_minmax_kernel<bf16_t>), dim3(grid_for(n / 8, kQ4MinMaxGroups)), dim3(kQ4Threads), 0, s,
                           static_cast<const bf16_t*>(x), (long long)n, aligned16(x), keys, counter);
    else
        hipLaunchKernelGGL((q4_minmax_kernel<float>), dim3(grid_for(n / 4, kQ4MinMaxGroups)), dim3(kQ4Threads), 0, s,
                           static_cast<const float*>(x), (long long)n, aligned16(x), keys, counter);
    if (!counter) hipLaunchKernelGGL(q4_finalize_kernel, dim3(1), dim3(1), 0, s, keys);
    const uintptr_t ca = reinterpret_cast<uintptr_t>(codes);
    if (dtype == SHATTN_DTYPE_BF16)
        hipLaunchKernelGGL((q4_encode_kernel<bf16_t>), dim3(grid_for(n / 8 + 1, 1 << 20)), dim3(kQ4Threads), 0, s,
                           static_cast<const bf16_t*>(x), (long long)n, aligned16(x) && ca % 4 == 0, params, codes);
    else
        hipLaunchKernelGGL((q4_encode_kernel<float>), dim3(grid_for(n / 4 + 1, 1 << 20)), dim3(kQ4Threads), 0, s,
                           static_cast<const float*>(x), (long long)n, aligned16(x) && ca % 2 == 0, params, codes);
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
    const bool vec = (reinterpret_cast<uintptr_t>(codes) % 4) == 0 && aligned16(out);
    if (dtype == SHATTN_DTYPE_BF16)
        hipLaunchKernelGGL((q4_decode_kernel<bf16_t>), dim3(grid_for(n / 8 + 1, 1 << 20)), dim3(kQ4Threads), 0, s,
                           codes, params, (long long)n, vec, static_cast<bf16_t*>(out));
    else
        hipLaunchKernelGGL((q4_decode_kernel<float>), dim3(grid_for(n / 8 + 1, 1 << 20)), dim3(kQ4Threads), 0, s,
                           codes, params, (long long)n, vec, static_cast<float*>(out));
    return check_launch("cache_dequant4");
}
