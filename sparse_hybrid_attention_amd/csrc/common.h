// Shared device/host helpers of the gfx950 hybrid sparse attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdarg>
#include <cstdio>
#include <string>

#include "hybrid_attn.h"

namespace shattn {

// ------------------------------------------------------------------ host side
// Thread-local message of the last failure, exposed through shattn_last_error().
std::string& last_error();
int fail(int code, const char* fmt, ...);
// Checks hipGetLastError() after a launch; returns SHATTN_OK or SHATTN_EHIP.
int check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------- device side
typedef uint16_t bf16_t;  // bfloat16 storage (bit pattern)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// float32 -> bfloat16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Element access for the two storage dtypes.
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
    static constexpr int kVec = 8;  // elements per 16-byte vector
    __device__ static __forceinline__ void unpack(const uint4& u, float* f) {
        f[0] = __uint_as_float(u.x << 16); f[1] = __uint_as_float(u.x & 0xFFFF0000u);
        f[2] = __uint_as_float(u.y << 16); f[3] = __uint_as_float(u.y & 0xFFFF0000u);
        f[4] = __uint_as_float(u.z << 16); f[5] = __uint_as_float(u.z & 0xFFFF0000u);
        f[6] = __uint_as_float(u.w << 16); f[7] = __uint_as_float(u.w & 0xFFFF0000u);
    }
    __device__ static __forceinline__ uint4 pack(const float* f) {
        uint4 u;
        u.x = pack_bf16x2(f[0], f[1]); u.y = pack_bf16x2(f[2], f[3]);
        u.z = pack_bf16x2(f[4], f[5]); u.w = pack_bf16x2(f[6], f[7]);
        return u;
    }
    __device__ static __forceinline__ float load1(const bf16_t* p) { return bf16_to_f32(*p); }
    __device__ static __forceinline__ void store1(bf16_t* p, float f) {
        *p = (bf16_t)f32_to_bf16_rne(f);
    }
};
template <> struct Elem<float> {
    static constexpr int kVec = 4;
    __device__ static __forceinline__ void unpack(const uint4& u, float* f) {
        f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
    }
    __device__ static __forceinline__ uint4 pack(const float* f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
    __device__ static __forceinline__ float load1(const float* p) { return *p; }
    __device__ static __forceinline__ void store1(float* p, float f) { *p = f; }
};

// Wave-level (64 lanes) LDS ordering: makes this lane's earlier LDS writes
// visible to the other lanes of the wave before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte global loads: plain (cached) and streaming (non-temporal hint).
__device__ __forceinline__ uint4 ld16(const void* p) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}


// Workgroup -> work id remap for the 8 XCDs of MI355X.  The dispatcher deals
// workgroup i to XCD i % 8; XCD x receives ceil/floor(n / 8) workgroups and the
// j-th of them (i = x + 8 j) gets work id start(x) + j, so each XCD covers one
// contiguous range of work ids.  A bijection of [0, n) for every n.
__device__ __forceinline__ long long xcd_work_id(long long i, long long n) {
    constexpr int kXcds = 8;
    const long long q = n / kXcds, r = n % kXcds;
    const long long x = i % kXcds, j = i / kXcds;
    return x * q + (x < r ? x : r) + j;
}

}  // namespace shattn
