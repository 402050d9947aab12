// Measurement aid, not part of the attention path: the bf16 MFMA issue rate
// of the device, measured by a loop of independent 16x16x32 bf16 MFMAs, so
// that roofline fractions can be read against a measured as well as the
// published peak.
#include "common.h"

namespace shattn {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeChains = 8;   // independent accumulators per wave: no MFMA waits on another

// SHAPE 0: v_mfma_f32_16x16x32_bf16 (16384 flops), 1: v_mfma_f32_32x32x16_bf16 (32768 flops)
template <int SHAPE>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters, float* sink) {
    bf16x8_t a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(1e-3f * (float)((threadIdx.x + j) & 7));
        b[j] = (__bf16)(2e-3f * (float)j);
    }
    float s = 0.f;
    if constexpr (SHAPE == 0) {
        // eight named accumulators, each updated in place every round
        f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
#pragma unroll 2
        for (int it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
            c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c4, 0, 0, 0);
            c5 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c5, 0, 0, 0);
            c6 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c6, 0, 0, 0);
            c7 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c7, 0, 0, 0);
        }
        const f32x4_t c[kProbeChains] = {c0, c1, c2, c3, c4, c5, c6, c7};
#pragma unroll
        for (int k = 0; k < kProbeChains; ++k) s += (c[k][0] + c[k][1]) + (c[k][2] + c[k][3]);
    } else {
        constexpr int CH = kProbeChains / 2;   // 16 accumulator registers each
        f32x16_t c[CH];
#pragma unroll
        for (int k = 0; k < CH; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) c[k][r] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int k = 0; k < CH; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < CH; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += c[k][r];
    }
    sink[(long long)blockIdx.x * kProbeThreads + threadIdx.x] = s;   // keeps every MFMA live
}

}  // namespace
}  // namespace shattn

using namespace shattn;

extern "C" int shattn_mfma_peak_probe(int workgroups, int iters, int shape, float* sink, void* stream) {
    if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 20) || !sink || shape < 0 || shape > 1)
        return fail(SHATTN_EINVAL, "shattn_mfma_peak_probe: workgroups %d, iters %d, shape %d", workgroups, iters,
                    shape);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (shape == 0)
        hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s, iters, sink);
    else
        hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s, iters, sink);
    return check_launch("shattn_mfma_peak_probe");
}
