// Device measurement probes (not part of the attention path): the bf16 MFMA
// issue rate and the random-row gather rate of the memory hierarchy, so that
// roofline fractions can be read against measured ceilings as well as the
// published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "probes.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

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

// 32-bit integer mix (the finaliser of MurmurHash3), so that consecutive read
// indices land on unrelated rows
__device__ __forceinline__ uint32_t mix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    return h;
}

// Each wave reads rows in groups: 64 lanes x 16 bytes cover 1024 / row_bytes
// rows per load; a lane issues DEPTH such loads before it consumes any.  The
// table is split into `slices` equal parts and workgroup i (which the
// dispatcher places on XCD i % 8) reads only part (i % 8) % slices, so that
// each XCD's L2 sees one part (slices = 1: the whole table).
template <int DEPTH>
__global__ __launch_bounds__(kProbeThreads) void gather_probe_kernel(const char* __restrict__ table, uint32_t srows,
                                                                     int row_bytes, long long row_stride,
                                                                     int slices, long long n, uint32_t* sink) {
    const int lane = threadIdx.x & 63;
    const int pieces = row_bytes >> 4;           // 16-byte pieces per row
    const int rpl = 64 / pieces;                 // rows per wave load
    const int r = lane / pieces, pc = lane - r * pieces;
    const long long wave = ((long long)blockIdx.x * kProbeThreads + threadIdx.x) >> 6;
    const long long nwaves = ((long long)gridDim.x * kProbeThreads) >> 6;
    const long long per_iter = (long long)rpl * DEPTH;
    const char* base = table + (long long)((blockIdx.x % 8) % slices) * srows * row_stride + pc * 16;
    const bool pow2 = (srows & (srows - 1)) == 0;
    uint32_t acc = 0u;
    for (long long it = wave * per_iter; it < n; it += nwaves * per_iter) {
        uint4 v[DEPTH];
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            const long long j = it + (long long)u * rpl + r;
            const uint32_t h = mix32((uint32_t)j);
            const uint32_t row = j < n ? (pow2 ? (h & (srows - 1)) : h % srows) : 0u;
            v[u] = *reinterpret_cast<const uint4*>(base + (long long)row * row_stride);
        }
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    sink[(long long)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

// Streaming read of whole 2 KB tiles (16 rows of 128 bytes).  A wave reads a
// tile with two 16-byte loads per lane, in one of two lane patterns: `mfma`
// false, each load covers 1 KB of consecutive bytes; `mfma` true, the pattern
// of an MFMA operand load of 16 rows of 64 bf16 (lane l reads row l % 16,
// 16-byte piece l / 16 of the row's first and then second 64 bytes), so each
// load touches all 16 rows.  `segments` false: wave w reads tiles w, w + W,
// w + 2W, ... (W waves in the grid); true: each wave reads one contiguous run
// of tiles, as a pass that gives each wave its own range of rows does.  A lane
// keeps DEPTH tiles' loads in flight.
template <int DEPTH, bool MFMA, bool SEG>
__global__ __launch_bounds__(kProbeThreads) void stream_probe_kernel(const char* __restrict__ buf, long long ntiles,
                                                                     uint32_t* sink) {
    const int lane = threadIdx.x & 63;
    const long long wave = ((long long)blockIdx.x * kProbeThreads + threadIdx.x) >> 6;
    const long long nwaves = ((long long)gridDim.x * kProbeThreads) >> 6;
    int off0, off1;
    if (MFMA) {
        off0 = (lane & 15) * 128 + 16 * (lane >> 4);
        off1 = off0 + 64;
    } else {
        off0 = 16 * lane;
        off1 = 1024 + 16 * lane;
    }
    long long t0, tend, tstep;
    if (SEG) {
        const long long per = (ntiles + nwaves - 1) / nwaves;
        t0 = wave * per;
        tend = t0 + per < ntiles ? t0 + per : ntiles;
        tstep = 1;
    } else {
        t0 = wave;
        tend = ntiles;
        tstep = nwaves;
    }
    uint32_t acc = 0u;
    for (long long t = t0; t < tend; t += tstep * DEPTH) {
        uint4 v[DEPTH][2];
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            const long long tt = t + (long long)u * tstep;
            const char* base = buf + (tt < tend ? tt : t0) * 2048ll;
            v[u][0] = *reinterpret_cast<const uint4*>(base + off0);
            v[u][1] = *reinterpret_cast<const uint4*>(base + off1);
        }
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) acc ^= v[u][0].x ^ v[u][0].w ^ v[u][1].y ^ v[u][1].z;
    }
    sink[(long long)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : -4; }

}  // namespace

extern "C" int shattn_probe_mfma(int workgroups, int iters, int shape, float* sink, void* stream) {
    if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 20) || !sink || shape < 0 || shape > 1)
        return -1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (shape == 0)
        hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s, iters, sink);
    else
        hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s, iters, sink);
    return launched();
}

extern "C" int shattn_probe_gather(const void* table, int64_t nrows, int32_t row_bytes, int64_t row_stride,
                                   int32_t slices, int64_t n, int32_t depth, int32_t workgroups, uint32_t* sink,
                                   void* stream) {
    const bool rb_ok = row_bytes == 64 || row_bytes == 128 || row_bytes == 256 || row_bytes == 512 ||
                       row_bytes == 1024;
    if (!table || !sink || !rb_ok || nrows < 1 || row_stride < row_bytes || (row_stride & 15) || n < 0 ||
        workgroups < 1 || workgroups > 65536 || (reinterpret_cast<uintptr_t>(table) & 15) || slices < 1 ||
        slices > 8 || nrows % slices != 0 || nrows / slices > 0xFFFFFFFFll)
        return -1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const char* t = reinterpret_cast<const char*>(table);
    const uint32_t srows = (uint32_t)(nrows / slices);
    const dim3 g((unsigned)workgroups), b(kProbeThreads);
    switch (depth) {
        case 1: hipLaunchKernelGGL(gather_probe_kernel<1>, g, b, 0, s, t, srows, row_bytes, row_stride, slices, n, sink); break;
        case 2: hipLaunchKernelGGL(gather_probe_kernel<2>, g, b, 0, s, t, srows, row_bytes, row_stride, slices, n, sink); break;
        case 4: hipLaunchKernelGGL(gather_probe_kernel<4>, g, b, 0, s, t, srows, row_bytes, row_stride, slices, n, sink); break;
        case 8: hipLaunchKernelGGL(gather_probe_kernel<8>, g, b, 0, s, t, srows, row_bytes, row_stride, slices, n, sink); break;
        case 16: hipLaunchKernelGGL(gather_probe_kernel<16>, g, b, 0, s, t, srows, row_bytes, row_stride, slices, n, sink); break;
        default: return -1;
    }
    return launched();
}

extern "C" int shattn_probe_stream(const void* buf, int64_t bytes, int32_t mode, int32_t depth, int32_t workgroups,
                                   uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes < 2048 || (bytes % 2048) || mode < 0 || mode > 3 || workgroups < 1 ||
        workgroups > 65536 || (reinterpret_cast<uintptr_t>(buf) & 15))
        return -1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const char* b = reinterpret_cast<const char*>(buf);
    const long long nt = bytes / 2048;
    const dim3 g((unsigned)workgroups), bl(kProbeThreads);
#define SHATTN_STREAM_CASE(D)                                                                         \
    case D:                                                                                           \
        switch (mode) {                                                                               \
            case 0: hipLaunchKernelGGL((stream_probe_kernel<D, false, false>), g, bl, 0, s, b, nt, sink); break; \
            case 1: hipLaunchKernelGGL((stream_probe_kernel<D, true, false>), g, bl, 0, s, b, nt, sink); break;  \
            case 2: hipLaunchKernelGGL((stream_probe_kernel<D, false, true>), g, bl, 0, s, b, nt, sink); break;  \
            default: hipLaunchKernelGGL((stream_probe_kernel<D, true, true>), g, bl, 0, s, b, nt, sink); break;  \
        }                                                                                             \
        break;
    switch (depth) {
        SHATTN_STREAM_CASE(1)
        SHATTN_STREAM_CASE(2)
        SHATTN_STREAM_CASE(4)
        SHATTN_STREAM_CASE(8)
        default: return -1;
    }
#undef SHATTN_STREAM_CASE
    return launched();
}
