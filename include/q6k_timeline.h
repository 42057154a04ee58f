/*
 * q6k_timeline.h -- the three extra calls of libq6k_timeline.so, a second build of q6k.hip with
 * Q6K_TIMELINE defined.  That library exports every call of q6k.h and q4k.h unchanged (same
 * kernels and launches), and in addition each GEMM workgroup of q6k_gemm, q6k_gemm_noalloc and
 * q4k_gemm writes one record into a device array, which these calls clear and read.  It is a
 * measurement build (where each workgroup ran, when, and at what shader clock, behind the work
 * split's and the fabric traffic's analysis); libq6k.so holds none of it.
 *
 * Record b (eight uint64) belongs to workgroup b of the latest launch that reached it:
 *   [0] start, [1] end          -- s_memrealtime ticks (a constant 100 MHz clock), read by the
 *                                  workgroup's first thread as it begins and after its stores
 *   [2] start, [3] end          -- s_memtime shader-clock cycles over the same span
 *   [4] XCD index << 32 | HW_ID -- the HW_ID hardware register (CU, shader array and engine)
 *   [5] bx | by << 32           -- the 64-token x 128-row output tile
 *   [6] s0 | s1 << 32           -- its super-blocks [s0, s1) of k
 *   [7] 1 for a split-k piece (stored into the workspace), 0 for a whole tile
 * Workgroups beyond q6k_timeline_capacity() write nothing.  Conventions are those of q6k.h.
 */
#ifndef Q6K_TIMELINE_H
#define Q6K_TIMELINE_H

#include <stddef.h>
#include <stdint.h>

#include "q6k.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Number of workgroup records the device array holds. */
int64_t q6k_timeline_capacity(void);

/* Zeroes every record (so that a record with start 0 was not written), asynchronously on
 * `stream`, with hipMemsetAsync: not for use under graph capture.  Q6K_EHIP if the runtime
 * refuses. */
q6k_status q6k_timeline_clear(void* stream);

/* Copies records 0 .. min(max_wgs, capacity) - 1 into host memory `records` (8 uint64 each), a
 * blocking copy: synchronize the stream of the recorded launch first.  Q6K_EINVAL for a null
 * pointer or negative count, Q6K_EHIP if the runtime refuses. */
q6k_status q6k_timeline_read(uint64_t* records, int64_t max_wgs);

#ifdef __cplusplus
}
#endif

#endif
