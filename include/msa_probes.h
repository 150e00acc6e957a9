/*
 * msa_probes.h — measurement kernels of libmsa.so (not part of the attention
 * path).
 *
 * They give the practical peaks that the path's kernels are compared with,
 * beside the MI355X datasheet figures (HBM 8.0 TB/s, dense bf16 MFMA
 * 2.5 PFLOP/s):
 *   msa_probe_read_stream - one pass over a device buffer with non-temporal
 *                           16-byte loads (the HBM read roof of a kernel that
 *                           only streams, as the decode index kernel does);
 *   msa_probe_mfma_bf16   - a loop of independent v_mfma_f32_32x32x16_bf16
 *                           chains (the bf16 matrix-core issue roof, as used
 *                           by the prefill index and attention kernels);
 *   msa_probe_latency_chain - one lane following a chain of dependent loads
 *                           (the latency of one memory round trip, from the
 *                           level of the memory hierarchy the table fits, and
 *                           the cost of a launch: the bound of a kernel made
 *                           of short dependent steps, such as the decode
 *                           attention launch).
 * The caller times them (events on `stream`); the work per call is stated
 * below.  Same conventions as msa.h: device pointers owned by the caller,
 * host validation first (MSA_ERR_INVALID_ARGUMENT with msa_last_error()),
 * MSA_ERR_HIP for a failed launch, nothing allocated or synchronised.
 */
#ifndef MSA_PROBES_H
#define MSA_PROBES_H

#include <stddef.h>
#include <stdint.h>

#include "msa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16, >= 16) from device memory `src` once,
 * with `workgroups` one-wave workgroups (1 .. 1048576): workgroup
 * w streams the 16 KiB chunks w, w + workgroups, ... with sixteen 1 KiB wave
 * loads in flight (the pattern of the decode index kernel, which streams one
 * 16 KiB page of index keys per wave), then the bytes past the last whole
 * chunk.  The data are folded into a value that is written to sink[0]
 * (device, 4 bytes) only if it equals an improbable constant, so no write
 * traffic arises. */
msa_status msa_probe_read_stream(const void *src, size_t bytes, int32_t workgroups,
                                 uint32_t *sink, void *stream);

/* `workgroups` (1 .. 65536) workgroups of 4 waves; every wave issues
 * 4 * iters (iters 1 .. 2^24) v_mfma_f32_32x32x16_bf16 instructions in four
 * independent accumulator chains: 32768 * 4 * iters * 4 * workgroups flops.
 * sink[0] (device, 4 bytes) is written only if a result equals an
 * improbable constant. */
msa_status msa_probe_mfma_bf16(int32_t iters, int32_t workgroups, float *sink, void *stream);

/* One workgroup; one lane loads p = next[p] `steps` times (0 .. 2^24) with
 * vector-memory loads, starting at p = start (0 <= start < n), each load's
 * address depending on the value before; an entry outside [0, n) restarts
 * the chain at 0, so no load leaves next[0 .. n).  The last index reached is written to sink[0]
 * (device, 4 bytes).  With a random single-cycle table, the call takes
 * about steps round trips to wherever the table lives (L2, the Infinity
 * Cache or HBM, by its size) plus one launch. */
msa_status msa_probe_latency_chain(const int32_t *next, int32_t n, int32_t steps, int32_t start,
                                   int32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PROBES_H */
