/*
 * fc_envelope.h -- C ABI of libfcenv.so: reference rates for the hot-path
 * kernels of libfc.so.  Not part of the method: these probes move bytes or
 * run the matrix instruction and nothing else, so what they reach is what a
 * plain kernel gets from the device for the same traffic mix (or
 * instruction) on this machine, a reachable rate beside the published peaks.
 *
 * All calls are asynchronous on `stream` (a hipStream_t; 0 = the null
 * stream), allocate nothing, and return the fc.h status codes: FC_OK, or an
 * error before anything is launched (FC_ERR_NULL, FC_ERR_SHAPE for sizes that
 * are not whole chunks or a read larger than the write, FC_ERR_ALIGN for
 * pointers not 16-byte aligned, FC_ERR_ALIAS for overlapping source and
 * destination, FC_ERR_UNSUPPORTED beyond 2^31 chunks), or FC_ERR_HIP if the
 * launch fails.  The caller owns every buffer.
 */
#ifndef FC_ENVELOPE_H
#define FC_ENVELOPE_H

#include <stddef.h>
#include "fc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Granule of the stream probes (bytes): 32 KiB, one workgroup's share. */
size_t fce_chunk_bytes(void);

/*
 * fce_mix -- write `write_bytes` to device buffer dst and read `read_bytes`
 * from device buffer src (0 <= read_bytes <= write_bytes, both whole chunks,
 * write_bytes > 0).  Read chunks are spread evenly over the write chunks: a
 * workgroup that owns one loads it whole, then stores it to its destination
 * chunk; the other workgroups store a constant.  read_bytes == write_bytes is
 * a plain copy, read_bytes == 0 a pure write.
 */
int fce_mix(const void *src, size_t read_bytes, void *dst, size_t write_bytes, fc_stream stream);

/* fce_mix_n -- fce_mix launched n >= 1 times back to back from this one call
 * (n < 1: FC_ERR_SHAPE), so that a stream of small copies is timed without a
 * host call per kernel. */
int fce_mix_n(const void *src, size_t read_bytes, void *dst, size_t write_bytes, int n, fc_stream stream);

/*
 * fce_flat -- a flat stream of `bytes` (a multiple of 4 KiB) in the shape
 * with the smallest workgroup footprint: one 16-byte vector per lane, one
 * 4 KiB workgroup per 256 vectors, a grid that covers the buffer once.  With
 * src == NULL it writes a constant to dst (a pure write); otherwise it copies
 * src to dst with nontemporal loads and stores.  Errors: FC_ERR_NULL (dst),
 * FC_ERR_SHAPE, FC_ERR_ALIGN, FC_ERR_ALIAS, FC_ERR_UNSUPPORTED (beyond 2^31
 * workgroups).
 */
int fce_flat(const void *src, void *dst, size_t bytes, fc_stream stream);

/* fce_read -- read `read_bytes` (whole chunks) of device buffer src; sink is
 * a device float that is written only for one impossible data pattern. */
int fce_read(const void *src, size_t read_bytes, float *sink, fc_stream stream);

/*
 * fce_mfma -- 1024 workgroups x 4 waves, each wave `iters` x 8 independent
 * v_mfma_f32_32x32x16_f16 on random operands that change every iteration.
 * sink: device, fce_mfma_sink_floats() floats (one sum per lane).
 * fce_mfma_flops(iters) gives the flops of one launch.
 */
int fce_mfma(float *sink, int iters, fc_stream stream);
size_t fce_mfma_sink_floats(void);
double fce_mfma_flops(int iters);

/* fce_empty -- an empty kernel of `blocks` 64-lane workgroups (sink: a device
 * float never written): back-to-back launches of it time the per-kernel
 * overhead of a stream. */
int fce_empty(int blocks, float *sink, fc_stream stream);

/* fce_empty_n -- n >= 1 such kernels launched back to back from this one call:
 * their time over n is the per-kernel cost on the device's timeline when the
 * host is not the bottleneck (as for the kernels of one split plan, which one
 * library call enqueues).  FC_ERR_NULL (sink), FC_ERR_SHAPE (blocks or n < 1). */
int fce_empty_n(int blocks, int n, float *sink, fc_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* FC_ENVELOPE_H */
