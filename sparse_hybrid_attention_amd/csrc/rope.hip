// Rotary position embedding of a channel range of every head, in place.
//
// Pages: [Tiny-R2] "Tiny-R2: A Hybrid Architecture Combining SWA, CSA, HCA,
// mHC and DSMoE Under the DeepSeek V4 Design Paradigm", architecture diagram
// (RoPE on the prepared query, the window keys, the selected CSA keys and the
// HCA keys) and parameter block (a rope part of the head dim beside a
// non-rope part); [CS336] CS336 course notes, "位置编码" paragraph (position
// as a rotation angle, so that a query-key product depends on the position
// difference).  Pairing, angle and base are the reading stated with the
// declaration in hybrid_attn.h.
//
// One thread per (row, channel pair), pairs innermost, so a wave reads and
// writes contiguous bytes of each head; the thread turns its pair in every
// head of the row with one sine / cosine (the angle depends on the row and
// the pair only), loading eight heads' pairs before the first store so that
// they are in flight together.  The work is a read and a write of the
// rotated channels (HBM-bound).  The angle pos * f_i is formed and reduced
// modulo 2 pi in double precision and only then handed to the float sine /
// cosine: positions reach a million and more, where a float product would
// lose the angle's fractional part.
#include <hip/hip_runtime.h>

#include <cmath>

#include "common.h"
#include "hybrid_attn.h"

namespace shattn {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeHeadsInFlight = 8;

template <typename T>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(T* __restrict__ x, const int64_t* __restrict__ pos,
                                                            long long total, int heads, int d, int off, int npairs,
                                                            double step) {
    const long long stride = (long long)gridDim.x * kRopeThreads;
    for (long long u = (long long)blockIdx.x * kRopeThreads + threadIdx.x; u < total; u += stride) {
        const long long row = u / npairs;
        const int i = (int)(u - row * npairs);    // channel pair
        const long long p = pos[row];
        if (p < 0) continue;                      // inactive row: unchanged
        // f_i = base^(-2i/R) = 2^(-i * step), step = 2 log2(base) / R
        float s, c;
        rope_sincos(p, i, step, &s, &c);
        T* e0 = x + row * heads * (long long)d + off + 2 * i;
        for (int h0 = 0; h0 < heads; h0 += kRopeHeadsInFlight) {
            float x0[kRopeHeadsInFlight], x1[kRopeHeadsInFlight];
#pragma unroll
            for (int j = 0; j < kRopeHeadsInFlight; ++j) {
                if (h0 + j < heads) {
                    const T* e = e0 + (long long)(h0 + j) * d;
                    x0[j] = Elem<T>::load1(e);
                    x1[j] = Elem<T>::load1(e + 1);
                }
            }
#pragma unroll
            for (int j = 0; j < kRopeHeadsInFlight; ++j) {
                if (h0 + j < heads) {
                    T* e = e0 + (long long)(h0 + j) * d;
                    float r0, r1;
                    rope_turn(x0[j], x1[j], s, c, &r0, &r1);
                    Elem<T>::store1(e, r0);
                    Elem<T>::store1(e + 1, r1);
                }
            }
        }
    }
}

}  // namespace
}  // namespace shattn

extern "C" int rope_apply(void* x, const int64_t* pos, int64_t rows, int32_t heads, int32_t d, int32_t rope_off,
                          int32_t rope_dim, double base, int32_t dtype, void* stream) {
    using namespace shattn;
    if (dtype != SHATTN_DTYPE_BF16 && dtype != SHATTN_DTYPE_F32)
        return fail(SHATTN_EINVAL, "rope_apply: unknown dtype %d", dtype);
    if (rows < 0 || heads < 1 || d < 2)
        return fail(SHATTN_EINVAL, "rope_apply: bad sizes rows=%lld heads=%d d=%d", (long long)rows, heads, d);
    if (rope_dim < 2 || rope_dim % 2 != 0 || rope_off < 0 || (long long)rope_off + rope_dim > d)
        return fail(SHATTN_EINVAL, "rope_apply: rotated channels [%d, %d + %d) must be an even-sized range inside d=%d",
                    rope_off, rope_off, rope_dim, d);
    if (!(base > 0.0) || !std::isfinite(base)) return fail(SHATTN_EINVAL, "rope_apply: base must be finite and > 0");
    if (rows == 0) return SHATTN_OK;
    if (!x || !pos) return fail(SHATTN_EINVAL, "rope_apply: null pointer");
    const size_t esz = dtype == SHATTN_DTYPE_BF16 ? 2 : 4;
    if ((reinterpret_cast<uintptr_t>(x) % esz) != 0 || (reinterpret_cast<uintptr_t>(pos) % 8) != 0)
        return fail(SHATTN_EINVAL, "rope_apply: x must be %zu-byte and pos 8-byte aligned", esz);
    const int npairs = rope_dim / 2;
    if (rows > (1LL << 62) / ((long long)heads * d))
        return fail(SHATTN_EINVAL, "rope_apply: rows * heads * d overflows");
    const long long total = rows * (long long)npairs;   // (row, pair) units
    const double step = 2.0 * std::log2(base) / rope_dim;
    long long blocks = (total + kRopeThreads - 1) / kRopeThreads;
    if (blocks > (1LL << 20)) blocks = 1LL << 20;   // grid-stride beyond
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (dtype == SHATTN_DTYPE_BF16)
        hipLaunchKernelGGL((rope_kernel<bf16_t>), dim3((unsigned)blocks), dim3(kRopeThreads), 0, s,
                           static_cast<bf16_t*>(x), pos, total, (int)heads, (int)d, (int)rope_off, npairs, step);
    else
        hipLaunchKernelGGL((rope_kernel<float>), dim3((unsigned)blocks), dim3(kRopeThreads), 0, s,
                           static_cast<float*>(x), pos, total, (int)heads, (int)d, (int)rope_off, npairs, step);
    return check_launch("rope_apply");
}
