/*
 * liboscar_kv checking aid: the library's own fp64 -> bf16 / fp16 rounding
 * routines, run on the host.
 *
 * The cache stores rotated rows as the bf16 rounding of x . R and scales /
 * zero points as fp16 (OSCAR summary page, sections 3-4; the fp16 scale and
 * zero point of the per-token quantizer), each a single round-to-nearest-even
 * from fp64.  The kernels do these roundings with bit-level routines; this
 * entry point runs the same routines (the same source, compiled for the
 * host) so tests can compare them with an independent rounding on crafted
 * inputs (ties, carries into the exponent, range edges) without a GPU.
 *
 *  target 0: fp64 -> bf16 (general routine: zeros, subnormals, overflow)
 *  target 1: fp64 -> fp16 (general routine)
 *  target 2: fp64 -> bf16, the bit-pattern routine the structured rotation
 *            uses for results in the bf16 normal range (other inputs go to
 *            the general routine)
 *  x_host, out_host: host arrays of n elements.
 * Returns 0, OSCAR_ERR_NULL or OSCAR_ERR_ARG (oscar_kv.h).
 */
#ifndef OSCAR_CHECK_H
#define OSCAR_CHECK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int oscar_round_f64_host(int32_t target, const double* x_host, uint16_t* out_host, int64_t n);

#ifdef __cplusplus
}
#endif

#endif /* OSCAR_CHECK_H */
