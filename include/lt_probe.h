/*
 * lt_probe.h -- measurement probes of liblt.so, not part of the method's
 * path: the rates the chip delivers in practice, reported next to the
 * published peaks that roofline fractions are taken against.  Status codes
 * and lt_last_error() are those of lt.h.
 */
#ifndef LT_PROBE_H
#define LT_PROBE_H

#include "lt.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * The matrix-core and HBM-read probes.  Both are asynchronous on `stream`;
 * the caller times them (e.g. with events on that stream).
 *   lt_probe_mfma_bf16: `blocks` workgroups of 4 waves; each wave runs
 *     `iters` rounds of 8 independent 16x16x32 bf16 matrix-core products
 *     (16384 FLOP each), i.e. blocks*4*iters*8*16384 FLOP, on pseudo-random
 *     register operands of unit size (the sustained rate depends on the
 *     data; constant operands run faster).  sink: device fp32
 *     [blocks*256], overwritten with meaningless values.
 *   lt_probe_read: reads `bytes` of device memory at `buf` once (16-byte
 *     aligned, bytes a multiple of 16) with `blocks` workgroups of 256
 *     lanes, in nontemporal 16-byte loads.  sink: device u32 [blocks],
 *     written only on an unlikely value.
 * Errors: LT_ERR_NULL (null pointer), LT_ERR_SHAPE (blocks < 1, iters < 1,
 * bytes not a positive multiple of 16), LT_ERR_LAYOUT (buf not 16-byte
 * aligned), LT_ERR_HIP (launch failure).
 */
int lt_probe_mfma_bf16(int blocks, int iters, float *sink, hipStream_t stream);
int lt_probe_read(const void *buf, size_t bytes, int blocks, unsigned *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* LT_PROBE_H */
