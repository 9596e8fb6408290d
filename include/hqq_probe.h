/*
 * hqq_probe.h - HBM probes of known byte counts (libhqq_probe.so), beside the HQQ library.
 *
 * They compute nothing of the method.  The measurements use them as the practical rate of a
 * memory-bound kernel on the device at hand (HQQ page, "从压缩文件到一次前向": the fused
 * product's gain is fewer HBM reads, so its bound is the rate at which the packed weight can be
 * streamed), and as the copy of known size that calibrates the HBM byte counters.
 *
 * Conventions as in hqq.h: every pointer is caller-owned device memory, 16-byte aligned; calls
 * only enqueue work on `stream` (a hipStream_t, NULL = the default stream).  Return 0, 1 for an
 * invalid argument (nothing launched), 4 when the launch failed.
 */
#ifndef HQQ_PROBE_H
#define HQQ_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0 .. bytes) = src[0 .. bytes): 16-byte non-temporal loads and stores, `unroll` (4 or 8)
 * loads in flight per thread.  bytes: a positive multiple of 16; the buffers must not overlap. */
int hqq_probe_copy(const void* src, void* dst, size_t bytes, int unroll, void* stream);

/* Reads bufs[i][0 .. bytes[i]) for i < nbuf (1 .. 3) once, with 16-byte non-temporal loads,
 * `unroll` (4 or 8) in flight per thread, in one launch (the buffers' blocks one after another).
 * sink: 16 bytes of device memory that are written only if the folded words equal a fixed
 * constant (they keep the loads from being dropped).  bytes[i]: positive multiples of 16. */
int hqq_probe_read(const void* const* bufs, const size_t* bytes, int nbuf, void* sink, int unroll, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HQQ_PROBE_H */
