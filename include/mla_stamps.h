/*
 * libmla_stamps — a diagnostic build of libmla (the same sources compiled with -DMLA_PHASE_STAMPS).
 * It exports every call of mla.h, and its two attention kernels (the 128-head kernel behind
 * mla_decode_attn for many rows or long histories, and the head-split kernel for a few rows with
 * short histories) also record where each workgroup's time goes. Not part of the attention path:
 * the benchmark's --phase-stamps mode uses it to break a call's time into the kernel's phases
 * (chunk plan, query staging, first tiles, the tile loop, the output stores), which is how far a
 * call is from its tile loop alone; the pages describe the decode as bound by reading the cache
 * ("从零理解 MLA", sections "缓存开销" and "实际配置"), and these are the costs around that stream.
 *
 * Per workgroup (linear index blockIdx.x + blockIdx.y * gridDim.x, up to 8192 workgroups), 16
 * uint64 slots written by thread 0 of the workgroup's last launch: 0 entry, 1 chunk known, 2 queries
 * in registers (128-head kernel), 3 first tiles issued (head-split kernel: queries and first tiles
 * landed), 4 tile loop done, 5 exit with every store completed, all on the shader clock counter
 * (s_memtime); 8 entry and 9 exit on the 100 MHz counter (s_memrealtime); 10 tiles of the chunk,
 * 11 query row, 12 chunk index, 13 kernel (1 the 128-head kernel, 2 the head-split kernel). A
 * workgroup with no chunk, or one that took the exact fallback, leaves slot 5 as it was.
 *
 * Errors: MLA_OK (0), MLA_ERR_INVALID_ARG (1) for a null or short destination, MLA_ERR_HIP (4).
 * The calls synchronise with the device (they copy through the legacy default stream).
 */
#ifndef MLA_STAMPS_H
#define MLA_STAMPS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Size in bytes of the stamp array (8192 workgroups x 16 slots x 8 bytes). */
size_t mla_phase_stamps_bytes(void);

/* Zero every slot, so that a following launch's workgroups are told apart from earlier ones. */
int mla_phase_stamps_clear(void);

/* Copy the whole stamp array into host memory `host_dst` of at least mla_phase_stamps_bytes(). */
int mla_phase_stamps_read(void* host_dst, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* MLA_STAMPS_H */
