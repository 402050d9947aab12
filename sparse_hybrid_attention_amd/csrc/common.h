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

// float64 -> bfloat16, round to nearest, ties to even, in one rounding step
// (normal and zero results; no detour through a float32 rounding): the
// double is rounded to 8 significant bits, which float32 then holds exactly.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
    uint64_t u = (uint64_t)__double_as_longlong(x);
    u += 0x00000FFFFFFFFFFFull + ((u >> 45) & 1ull);
    u &= ~0x00001FFFFFFFFFFFull;
    return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;
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

// RoPE of one channel pair (the reading stated with rope_apply): pair i at
// position p turns by p * f_i, f_i = 2^(-i * step), step = 2 log2(base) / R.
// The angle is formed in turns (p * f_i / 2 pi) in double precision and its
// whole turns dropped there (exact), then the hardware sine and cosine of the
// remaining fraction of a turn (v_sin_f32 / v_cos_f32 take turns) turn
// (a, b) -> (a c - b s, a s + b c) in explicit fused multiply-adds, so that
// every kernel rotating a pair gets the same bits.
__device__ __forceinline__ void rope_sincos(long long p, int i, double step, float* s, float* c) {
    constexpr double kInvTwoPi = 0.15915494309189533576888376337251;
    double r = (double)p * (exp2(-(double)i * step) * kInvTwoPi);
    r -= rint(r);
    const float rf = (float)r;
    *s = __builtin_amdgcn_sinf(rf);
    *c = __builtin_amdgcn_cosf(rf);
}
__device__ __forceinline__ void rope_turn(float a, float b, float s, float c, float* ra, float* rb) {
    *ra = fmaf(a, c, -(b * s));
    *rb = fmaf(a, s, b * c);
}

// Wave-level (64 lanes) LDS ordering: makes this lane's earlier LDS writes
// visible to the other lanes of the wave before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (vmcnt only).  Loads, direct-to-LDS loads included, complete in the order
// they were issued, so this also waits for every load older than the N
// youngest.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    // s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
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


// ---- wave-wide operations in registers (DPP / permlane; no LDS round trip)
// dpp_ctrl values: quad_perm [1,0,3,2] = 0xB1 (lane ^ 1), [2,3,0,1] = 0x4E
// (lane ^ 2), row_ror:n = 0x120 + n, row_shr:n = 0x110 + n, row_bcast:15 =
// 0x142, row_bcast:31 = 0x143.
template <int CTRL> __device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
// the two values held by lanes l and l ^ 16 (r[0] from the lower row of the pair)
__device__ __forceinline__ void xor16_pair(uint32_t v, uint32_t& lo, uint32_t& hi) {
    auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    lo = a[0];
    hi = a[1];
}
__device__ __forceinline__ void xor32_pair(uint32_t v, uint32_t& lo, uint32_t& hi) {
    auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    lo = a[0];
    hi = a[1];
}
// all-lane reduction with an associative, commutative op on 32-bit patterns
template <typename F> __device__ __forceinline__ uint32_t wave_allreduce(uint32_t v, F op) {
    v = op(v, dpp_mov<0xB1>(v));
    v = op(v, dpp_mov<0x4E>(v));
    v = op(v, dpp_mov<0x124>(v));
    v = op(v, dpp_mov<0x128>(v));
    uint32_t lo, hi;
    xor16_pair(v, lo, hi);
    v = op(lo, hi);
    xor32_pair(v, lo, hi);
    return op(lo, hi);
}
__device__ __forceinline__ float wave_max_f(float v) {
    return __uint_as_float(wave_allreduce(__float_as_uint(v), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
}
// sum over the lanes l, l^16, l^32, l^48 in the fixed order (l0 + l16) + (l32 + l48)
__device__ __forceinline__ float sum_xrows(float v) {
    uint32_t lo, hi;
    xor16_pair(__float_as_uint(v), lo, hi);
    const float s = __uint_as_float(lo) + __uint_as_float(hi);
    xor32_pair(__float_as_uint(s), lo, hi);
    return __uint_as_float(lo) + __uint_as_float(hi);
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row 0 -> 1, row 2 -> 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // rows 0..1 -> 2, 3
    return v;
}

}  // namespace shattn
