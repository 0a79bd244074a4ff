/*
 * wanpeak: measurement aids for the benchmark, outside the attention path.
 *
 * The kernels of libwanattn are quoted against the MI355X spec peaks (dense
 * bf16 MFMA 2.5 PFLOP/s, HBM3E 8 TB/s) and also against what the chip
 * sustains on two plain loops, which these calls run:
 *
 *   wanpeak_mfma_bf16_loop  every wave issues four independent chains of
 *                           v_mfma_f32_32x32x16_bf16 on fixed operands
 *                           (2 * 32 * 32 * 16 = 32768 FLOP each);
 *   wanpeak_copy            a streaming device-to-device copy with 16-byte
 *                           nontemporal loads and stores;
 *   wanpeak_read            the same loads alone (reads only);
 *   wanpeak_fill            the same stores alone (writes only).
 * A copy reads and writes the same number of bytes, as the row calls of the
 * library do; the read-only and write-only rates bound it from either side.
 *
 * Library libwanpeak.so, built beside libwanattn.so. Pointers are caller-owned
 * device memory; nothing is allocated or synchronised; work goes on `stream`
 * (NULL = the default stream). Arguments are checked on the host before
 * anything is enqueued. Returns 0 on success, 1 for an invalid argument
 * (nothing launched), 3 when the launch itself fails.
 */
#ifndef WANPEAK_H_
#define WANPEAK_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads per workgroup of wanpeak_mfma_bf16_loop (4 waves). */
#define WANPEAK_MFMA_THREADS 256

/* Bytes of the source that one workgroup of wanpeak_read (and of
   wanpeak_fill) covers: 256 threads x 4 vectors of 16 bytes. */
#define WANPEAK_STREAM_BLOCK_BYTES 16384

/*
 * Runs `blocks` workgroups of WANPEAK_MFMA_THREADS threads; each wave does
 * `iters` iterations of 4 MFMAs, so the launch performs
 *   blocks * 4 * iters * 4 * 32768 FLOP.
 * operands: 2 * WANPEAK_MFMA_THREADS vectors of 8 bf16 (8 KiB, 16-byte
 *           aligned); thread t takes A from vector t and B from vector
 *           WANPEAK_MFMA_THREADS + t. Random bf16 values draw the power of a
 *           real workload; all-zero operands do not.
 * out:      blocks * WANPEAK_MFMA_THREADS floats (4-byte aligned): per thread
 *           the sum of its accumulators, so that the loop is not removed.
 * 1 <= blocks <= 65536 and iters >= 1, else 1 (invalid).
 */
int wanpeak_mfma_bf16_loop(const void* operands, float* out, int blocks, int iters,
                           hipStream_t stream);

/*
 * dst[0, bytes) = src[0, bytes). bytes must be a multiple of 16, both
 * pointers 16-byte aligned and the two ranges disjoint, else 1 (invalid).
 * bytes = 0 launches nothing. The launch moves 2 * bytes through HBM.
 */
int wanpeak_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

/*
 * Reads src[0, bytes) once. out[i] (ceil(bytes / WANPEAK_STREAM_BLOCK_BYTES)
 * words, 4-byte aligned, not overlapping src) receives the XOR of all 4-byte
 * words of block i of the source: the check that every byte was read. bytes
 * must be a multiple of 16 and src 16-byte aligned, else 1 (invalid); bytes
 * = 0 launches nothing. The launch moves `bytes` through HBM (plus 4 bytes per
 * block written).
 */
int wanpeak_read(uint32_t* out, const void* src, size_t bytes, hipStream_t stream);

/*
 * Sets every 4-byte word of dst[0, bytes) to `value`. bytes must be a multiple
 * of 16 and dst 16-byte aligned, else 1 (invalid); bytes = 0 launches nothing.
 * The launch moves `bytes` through HBM.
 */
int wanpeak_fill(void* dst, size_t bytes, uint32_t value, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* WANPEAK_H_ */
