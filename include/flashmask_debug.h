/* Workgroup timeline of the attention kernels: present only in libflashmask_stamps.so, the
 * debug build of the library compiled with FM_WG_STAMPS (python -m
 * mask_aware_flashattention_amd.build --stamps).  It is a measurement aid, not part of the
 * computation: the kernels and their results are those of libflashmask.so.
 *
 * Each call copies the device array of one attention kernel to host memory: 8 unsigned 64-bit
 * words per workgroup, indexed by the workgroup's launch index (blockIdx.x < 65536), written by
 * the last launch of that kernel: {start, first tile's barrier passed, tile walk done, end,
 * HW_ID | XCC_ID << 32, tiles walked}; times are the GPU's real-time counter (s_memrealtime,
 * 100 MHz ticks); words 6 and 7 are unused; slots past the last launch's grid keep older values.
 *   host:  host memory of at least `bytes` bytes (owned by the caller)
 *   bytes: bytes to copy, at most 65536 * 8 * 8
 * Returns 0, or -1 for a null pointer, a size beyond the array or a failed copy.  Synchronous
 * (hipMemcpyFromSymbol): call it after the kernel has finished. */
#ifndef FLASHMASK_DEBUG_H
#define FLASHMASK_DEBUG_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int flashmask_debug_stamps_fwd(void* host, size_t bytes);  /* forward kernel */
int flashmask_debug_stamps_dq(void* host, size_t bytes);   /* backward: dQ kernel */
int flashmask_debug_stamps_dkdv(void* host, size_t bytes); /* backward: dK/dV kernel */

#ifdef __cplusplus
}
#endif

#endif /* FLASHMASK_DEBUG_H */
