/*
 * probes.h -- device measurement probes (libshattn_probe.so).
 *
 * Not part of the attention library or its interface: these kernels only
 * measure the device, so that the benchmark can read roofline fractions
 * against measured ceilings as well as the published peaks.  Every pointer is
 * a device pointer owned by the caller; calls enqueue one launch on `stream`
 * and return 0, or -1 for an invalid argument, -4 for a failed launch.
 */
#ifndef SHATTN_PROBES_H
#define SHATTN_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define SHATTN_PROBE_API __attribute__((visibility("default")))
#else
#define SHATTN_PROBE_API
#endif

/*
 * bf16 MFMA issue rate: `workgroups` workgroups of 256 threads; every wave
 * issues `iters` rounds of independent MFMAs: shape 0 = 8 x
 * v_mfma_f32_16x16x32_bf16 per round, shape 1 = 4 x v_mfma_f32_32x32x16_bf16
 * per round (131072 flops per round and wave either way), i.e.
 * workgroups * 4 * iters * 131072 flops.  sink: float32 [workgroups * 256].
 * Supported: 1 <= workgroups <= 65536, 1 <= iters <= 2^20, shape 0 or 1.
 */
SHATTN_PROBE_API int shattn_probe_mfma(int workgroups, int iters, int shape, float* sink, void* stream);

/*
 * Random-row gather throughput: `n` reads of one `row_bytes`-byte row each,
 * row r of the table starting at table + r * row_stride (r < nrows).  The
 * table is split into `slices` equal parts of nrows / slices rows; workgroup
 * i (placed on XCD i % 8 by the dispatcher) reads part (i % 8) % slices, its
 * rows chosen by a hash of the read's index (uniform over the part).  Each
 * lane keeps `depth` 16-byte reads in flight.  Bytes moved = n * row_bytes.
 * The table must hold (nrows - 1) * row_stride + row_bytes bytes.  A table
 * that fits the last-level cache measures the cache's gather rate.
 * sink: uint32 [workgroups * 256], written.
 * Supported: row_bytes in {64, 128, 256, 512, 1024}; row_stride >= row_bytes,
 * a multiple of 16; 1 <= slices <= 8 dividing nrows, nrows / slices < 2^32;
 * depth in {1, 2, 4, 8, 16}; 1 <= workgroups <= 65536.
 */
SHATTN_PROBE_API int shattn_probe_gather(const void* table, int64_t nrows, int32_t row_bytes, int64_t row_stride,
                                         int32_t slices, int64_t n, int32_t depth, int32_t workgroups,
                                         uint32_t* sink, void* stream);

/*
 * Streaming read throughput over `bytes` bytes (a multiple of 2048) in 2 KB
 * tiles of 16 rows of 128 bytes, each lane keeping `depth` tiles' two 16-byte
 * loads in flight.  mode bit 0: lane pattern of an MFMA operand load (lane l
 * reads row l % 16, piece l / 16 of the row's first and second 64 bytes, so
 * one load touches 16 rows) instead of 1 KB of consecutive bytes per load;
 * mode bit 1: each wave reads one contiguous run of tiles instead of every
 * W-th tile (W waves in the grid).  sink: uint32 [workgroups * 256], written.
 * Supported: mode 0..3, depth in {1, 2, 4, 8}, 1 <= workgroups <= 65536.
 */
SHATTN_PROBE_API int shattn_probe_stream(const void* buf, int64_t bytes, int32_t mode, int32_t depth,
                                         int32_t workgroups, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SHATTN_PROBES_H */
