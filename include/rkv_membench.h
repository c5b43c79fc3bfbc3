/*
 * rkv_membench.h -- streaming kernels that measure the HBM bandwidth one
 * MI355X sustains, the denominator the R-KV step's bandwidth-bound kernels
 * are compared with beside the 8 TB/s specification (measurement only: the
 * step itself never calls these).
 *
 * Both kernels walk a buffer with 16-byte accesses, each workgroup a
 * contiguous stretch, every lane keeping several loads in flight.  Buffers
 * should be larger than the 256 MB last-level cache so that the traffic
 * reaches HBM.
 *
 * Conventions: device pointers, caller-owned, 16-byte aligned; bytes a
 * multiple of 16; work enqueued on `stream` (a hipStream_t, NULL = null
 * stream), asynchronous.  Return 0 on success, -1 for a bad argument, or the
 * HIP error code of the launch.
 */
#ifndef RKV_MEMBENCH_H_
#define RKV_MEMBENCH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` of src once; a word derived from every byte read goes to
 * sink[0] only when it equals a value no input produces, so the loads cannot
 * be dropped (sink: device, 4 bytes).  workgroups: 0 = 8 per compute unit. */
int rkv_membench_read(const void *src, size_t bytes, uint32_t *sink, int32_t workgroups,
                      void *stream);

/* Copies `bytes` from src to dst (distinct buffers): each byte read once and
 * written once.  workgroups: 0 = 8 per compute unit. */
int rkv_membench_copy(void *dst, const void *src, size_t bytes, int32_t workgroups, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RKV_MEMBENCH_H_ */
