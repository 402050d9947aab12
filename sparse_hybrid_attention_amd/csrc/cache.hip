// Decode cache maintenance: one new token per sequence goes into the raw
// window ring, and every block of m tokens that the token completes is
// compressed into the CSA / HCA caches (and the CSA indexer-key cache).
//
// Pages: [V4-blog] "deepseek-v4", section "1. hybrid attn" (the raw window
// K/V and the compressed caches are kept apart; the raw rows age out as
// decode advances while the compressed entries stay); [V4-code] CSDN CSA/HCA
// article, section "1. HCA" (block merge: per-channel softmax over the block
// positions of a learned logit table, weighted sum over the block).
//
// Work decomposition: one thread per (tensor, sequence, 16-byte channel
// group).  blockIdx.z picks the tensor (0 = K, 1 = V, 2 = indexer keys),
// blockIdx.y the sequence, blockIdx.x * 256 + threadIdx.x the channel group.
// A thread copies its slice of the new row into ring slot t % W, then for
// each ratio whose block the token completes it computes the m softmax
// weights of its channels (float32, max-subtracted) and the weighted sum of
// the block's m rows: m - 1 rows from the ring (written by earlier calls) and
// the new row from the input, never from the slot this call writes.  The work
// is latency-bound (a few KB per sequence); the block sums read m rows of
// 16 bytes per thread, issued before any is used.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.h"
#include "hybrid_attn.h"

namespace shattn {
namespace {

constexpr int kAppendThreads = 256;

struct AppendRatio {
    int m;                // 0: absent
    long long cap;        // entries in the cache
    const float* z;       // [m, C] logits
    void* cache;          // [B, cap, C]
};

struct AppendTensor {
    int C;                // channels per row
    const void* x_new;    // [B, C]
    void* ring;           // [B, W, C]
    AppendRatio r[2];
    bool counts;          // this tensor reports the dropped entries of its ratios
};

struct AppendParams {
    int B, W;
    const int64_t* pos;
    AppendTensor t[3];
    int ntensors;
    int32_t* dropped;
};

template <typename T>
__global__ __launch_bounds__(kAppendThreads) void cache_append_kernel(AppendParams p) {
    constexpr int VW = Elem<T>::kVec;
    const AppendTensor& ts = p.t[blockIdx.z];
    const int b = blockIdx.y;
    const int j = blockIdx.x * kAppendThreads + threadIdx.x;   // channel group
    const int NG = ts.C / VW;
    const long long t = p.pos[b];
    const bool active = j < NG && t >= 0;

    const size_t ch0 = (size_t)j * VW;
    uint4 xn = make_uint4(0u, 0u, 0u, 0u);
    if (active) {
        xn = ld16(reinterpret_cast<const T*>(ts.x_new) + (size_t)b * ts.C + ch0);
        T* ring_b = reinterpret_cast<T*>(ts.ring) + (size_t)b * p.W * ts.C;
        *reinterpret_cast<uint4*>(ring_b + (size_t)(t % p.W) * ts.C + ch0) = xn;
    }
#pragma unroll
    for (int ri = 0; ri < 2; ++ri) {
        const AppendRatio& r = ts.r[ri];
        if (r.m == 0 || t < 0 || (t + 1) % r.m != 0) continue;
        const long long c = (t + 1) / r.m - 1;
        if (c >= r.cap) {
            if (ts.counts && j == 0 && p.dropped) atomicAdd(p.dropped, 1);
            continue;
        }
        if (!active) continue;
        // per-channel softmax weights over the m block positions
        float mx[VW], sum[VW], acc[VW];
#pragma unroll
        for (int v = 0; v < VW; ++v) {
            mx[v] = -INFINITY;
            sum[v] = 0.f;
            acc[v] = 0.f;
        }
        const float* z = r.z + ch0;
        for (int i = 0; i < r.m; ++i) {
            const float4* zi = reinterpret_cast<const float4*>(z + (size_t)i * ts.C);
#pragma unroll
            for (int u = 0; u < VW / 4; ++u) {
                const float4 f = zi[u];
                mx[4 * u + 0] = fmaxf(mx[4 * u + 0], f.x);
                mx[4 * u + 1] = fmaxf(mx[4 * u + 1], f.y);
                mx[4 * u + 2] = fmaxf(mx[4 * u + 2], f.z);
                mx[4 * u + 3] = fmaxf(mx[4 * u + 3], f.w);
            }
        }
        // rows of the block: positions c*m .. t; the last is the new row
        const T* ring_b = reinterpret_cast<const T*>(ts.ring) + (size_t)b * p.W * ts.C;
        const long long p0 = c * r.m;
        for (int i0 = 0; i0 < r.m; i0 += 8) {
            uint4 rows[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u;
                if (i < r.m - 1) rows[u] = ld16(ring_b + (size_t)((p0 + i) % p.W) * ts.C + ch0);
                else rows[u] = xn;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u;
                if (i >= r.m) break;
                float f[VW], w[VW];
                Elem<T>::unpack(rows[u], f);
                const float4* zi = reinterpret_cast<const float4*>(z + (size_t)i * ts.C);
#pragma unroll
                for (int q = 0; q < VW / 4; ++q) {
                    const float4 zz = zi[q];
                    w[4 * q + 0] = zz.x;
                    w[4 * q + 1] = zz.y;
                    w[4 * q + 2] = zz.z;
                    w[4 * q + 3] = zz.w;
                }
#pragma unroll
                for (int v = 0; v < VW; ++v) {
                    const float e = __expf(w[v] - mx[v]);
                    sum[v] += e;
                    acc[v] = fmaf(e, f[v], acc[v]);
                }
            }
        }
        float out[VW];
#pragma unroll
        for (int v = 0; v < VW; ++v) out[v] = acc[v] / sum[v];
        T* dst = reinterpret_cast<T*>(r.cache) + ((size_t)b * r.cap + c) * ts.C + ch0;
        *reinterpret_cast<uint4*>(dst) = Elem<T>::pack(out);
    }
}

template <typename T>
int launch_append(const AppendParams& p, hipStream_t s) {
    int cmax = 0;
    for (int i = 0; i < p.ntensors; ++i) cmax = std::max(cmax, p.t[i].C);
    const int ng = cmax / Elem<T>::kVec;
    const dim3 grid((unsigned)((ng + kAppendThreads - 1) / kAppendThreads), (unsigned)p.B, (unsigned)p.ntensors);
    hipLaunchKernelGGL((cache_append_kernel<T>), grid, dim3(kAppendThreads), 0, s, p);
    return check_launch("hybrid_cache_append");
}

}  // namespace
}  // namespace shattn

using namespace shattn;

extern "C" int hybrid_cache_append(const shattn_append_args* a, void* stream) {
    if (!a) return fail(SHATTN_EINVAL, "hybrid_cache_append: null args");
    if (a->struct_size != (int)sizeof(shattn_append_args))
        return fail(SHATTN_EINVAL, "hybrid_cache_append: struct_size %d != %d", a->struct_size,
                    (int)sizeof(shattn_append_args));
    if (a->reserved0 != 0) return fail(SHATTN_EINVAL, "hybrid_cache_append: reserved0 must be 0");
    if (a->dtype != SHATTN_DTYPE_BF16 && a->dtype != SHATTN_DTYPE_F32)
        return fail(SHATTN_EINVAL, "hybrid_cache_append: unknown dtype %d", a->dtype);
    if (a->B < 0 || a->Hkv < 1 || a->W < 1 || a->m_csa < 0 || a->m_hca < 0 || a->d_idx < 0)
        return fail(SHATTN_EINVAL, "hybrid_cache_append: bad sizes B=%d Hkv=%d W=%d m_csa=%d m_hca=%d d_idx=%d",
                    a->B, a->Hkv, a->W, a->m_csa, a->m_hca, a->d_idx);
    if (a->d != 64 && a->d != 128)
        return fail(SHATTN_EUNSUPPORTED, "hybrid_cache_append: d=%d (supported: 64, 128)", a->d);
    if (a->d_idx != 0 && a->d_idx != 64 && a->d_idx != 128)
        return fail(SHATTN_EUNSUPPORTED, "hybrid_cache_append: d_idx=%d (supported: 0, 64, 128)", a->d_idx);
    if (a->m_csa > a->W || a->m_hca > a->W || a->m_csa > 1024 || a->m_hca > 1024)
        return fail(SHATTN_EUNSUPPORTED, "hybrid_cache_append: block ratios %d / %d must be <= W=%d and <= 1024",
                    a->m_csa, a->m_hca, a->W);
    if (a->d_idx > 0 && a->m_csa == 0)
        return fail(SHATTN_EINVAL, "hybrid_cache_append: indexer keys (d_idx > 0) need the CSA ratio");
    if (a->cap_csa < 0 || a->cap_hca < 0)
        return fail(SHATTN_EINVAL, "hybrid_cache_append: negative cache capacity");
    if (a->B == 0) return SHATTN_OK;
    if (a->B > 65535) return fail(SHATTN_EUNSUPPORTED, "hybrid_cache_append: B=%d > 65535", a->B);
    if (!a->pos || !a->k_new || !a->v_new || !a->k_ring || !a->v_ring)
        return fail(SHATTN_EINVAL, "hybrid_cache_append: null pos / k_new / v_new / k_ring / v_ring");
    if ((reinterpret_cast<uintptr_t>(a->pos) & 7u) || !aligned16(a->k_new) || !aligned16(a->v_new) ||
        !aligned16(a->k_ring) || !aligned16(a->v_ring))
        return fail(SHATTN_EINVAL, "hybrid_cache_append: misaligned pointer (pos 8 bytes, tensors 16 bytes)");
    auto ratio_ok = [&](int m, long long cap, const float* zk, const float* zv, const void* kc, const void* vc,
                        const char* name) -> int {
        if (m == 0) return SHATTN_OK;
        if (!zk || !zv || (cap > 0 && (!kc || !vc)))
            return fail(SHATTN_EINVAL, "hybrid_cache_append: %s ratio needs logits and caches", name);
        if (!aligned16(zk) || !aligned16(zv) || (cap > 0 && (!aligned16(kc) || !aligned16(vc))))
            return fail(SHATTN_EINVAL, "hybrid_cache_append: %s logits / caches must be 16-byte aligned", name);
        return SHATTN_OK;
    };
    int rc;
    if ((rc = ratio_ok(a->m_csa, a->cap_csa, a->zk_csa, a->zv_csa, a->k_csa, a->v_csa, "CSA"))) return rc;
    if ((rc = ratio_ok(a->m_hca, a->cap_hca, a->zk_hca, a->zv_hca, a->k_hca, a->v_hca, "HCA"))) return rc;
    if (a->d_idx > 0) {
        if (!a->kI_new || !a->kI_ring || !a->zI || (a->cap_csa > 0 && !a->kI_csa))
            return fail(SHATTN_EINVAL, "hybrid_cache_append: indexer keys need kI_new, kI_ring, zI and kI_csa");
        if (!aligned16(a->kI_new) || !aligned16(a->kI_ring) || !aligned16(a->zI) ||
            (a->cap_csa > 0 && !aligned16(a->kI_csa)))
            return fail(SHATTN_EINVAL, "hybrid_cache_append: indexer-key pointers must be 16-byte aligned");
    }
    if (reinterpret_cast<uintptr_t>(a->dropped) & 3u)
        return fail(SHATTN_EINVAL, "hybrid_cache_append: dropped must be 4-byte aligned");

    AppendParams p{};
    p.B = a->B;
    p.W = a->W;
    p.pos = a->pos;
    p.dropped = a->dropped;
    const int C = a->Hkv * a->d;
    auto kv = [&](int which) {
        AppendTensor t{};
        t.C = C;
        t.x_new = which == 0 ? a->k_new : a->v_new;
        t.ring = which == 0 ? a->k_ring : a->v_ring;
        t.r[0] = AppendRatio{a->m_csa, a->cap_csa, which == 0 ? a->zk_csa : a->zv_csa,
                             which == 0 ? a->k_csa : a->v_csa};
        t.r[1] = AppendRatio{a->m_hca, a->cap_hca, which == 0 ? a->zk_hca : a->zv_hca,
                             which == 0 ? a->k_hca : a->v_hca};
        t.counts = which == 0;   // the K thread counts a K/V entry pair once
        return t;
    };
    p.t[0] = kv(0);
    p.t[1] = kv(1);
    p.ntensors = 2;
    if (a->d_idx > 0) {
        AppendTensor t{};
        t.C = a->d_idx;
        t.x_new = a->kI_new;
        t.ring = a->kI_ring;
        t.r[0] = AppendRatio{a->m_csa, a->cap_csa, a->zI, a->kI_csa};
        t.r[1] = AppendRatio{0, 0, nullptr, nullptr};
        t.counts = true;
        p.t[2] = t;
        p.ntensors = 3;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    return a->dtype == SHATTN_DTYPE_BF16 ? launch_append<bf16_t>(p, s) : launch_append<float>(p, s);
}
