/* Streaming-read probe (libmoe_hbm.so): measures the HBM read bandwidth a
 * plain kernel reaches, the practical ceiling beside the data-sheet peak for
 * the routed-expert GEMMs, whose time is the time to stream the MXFP4 weights
 * of every touched expert.  Measurement only: the MoE layer never calls it.
 */
#ifndef HBM_PROBE_H
#define HBM_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of device memory at `src` once (16-byte loads, each of
 * `workgroups` workgroups of 256 threads over its own contiguous share of the
 * buffer; non-temporal loads if `nontemporal` is non-zero) and stores one XOR
 * fold per wave into
 * `sink` (device, hbm_probe_sink_words(workgroups) uint32 words; its values
 * mean nothing).  src: device pointer, 16-byte aligned, bytes a multiple of 16;
 * the caller owns both buffers.  Asynchronous on `stream`.
 * Returns 0, -1 for an invalid argument (nothing launched), -4 if the launch
 * failed. */
int hbm_read_probe(const void* src, size_t bytes, int nontemporal, uint32_t* sink, int workgroups,
                   hipStream_t stream);

/* Words of `sink` that hbm_read_probe writes for `workgroups` workgroups. */
int hbm_probe_sink_words(int workgroups);

#ifdef __cplusplus
}
#endif

#endif /* HBM_PROBE_H */
