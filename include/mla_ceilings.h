/*
 * libmla_ceilings — microbenchmarks that measure the two practical ceilings of the latent attention
 * on MI355X (gfx950): bf16 MFMA issue and HBM streaming. Not part of the attention path; the
 * benchmark calls them to state how close the kernels run to what the chip sustains.
 *
 * The pages name no hardware; the decode path they describe is bound by moving the cache
 * ("从零理解 MLA", sections "缓存开销" and "实际配置": every generated token reads the whole cache),
 * and its absorbed form trades that traffic for more multiply-adds. These calls measure both sides.
 *
 * Ownership and errors: all pointers are device memory owned by the caller; each call only
 * enqueues one kernel on `stream` (a hipStream_t; NULL = the legacy default stream) and returns
 * 0 on success, 1 for an invalid argument, 2 for an unsupported variant, 4 for a HIP launch error.
 * Nothing is allocated.
 */
#ifndef MLA_CEILINGS_H
#define MLA_CEILINGS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mla_ceiling_mfma — chip-wide v_mfma_f32_32x32x16_bf16 issue.
 *  waves_per_simd  1 or 2 (workgroups of 4 or 8 waves, one workgroup per CU)
 *  n_acc           independent accumulators per wave: 1, 4 or 8 at one wave per SIMD, 4 or 8 at two;
 *                  or, at one wave per SIMD, one dependent chain written in asm: 100 accumulating in
 *                  VGPRs, 101 in AGPRs, 102 / 103 the same with one ds_read_b128 operand per MFMA,
 *                  104 LDS-fed with one wait per four MFMAs, 105 one VALU op between MFMAs, 106 each
 *                  MFMA's operand from two ds_read_b64_tr_b16, 107 / 108 LDS-fed over two / four
 *                  independent accumulators taken in turn (an iteration issues 8 MFMAs, 12 for 104);
 *                  with waves_per_simd 2, chains 101, 103, 105 and 106 in two 4-wave workgroups per CU
 *  n_workgroups    workgroups launched (256 = one per CU)
 *  iters           loop iterations; each issues 4 * n_acc MFMAs of 32x32x16 (32768 flops each)
 *  operands        uint32 [n_workgroups * 4 * waves_per_simd * 64 * 8]: per lane the two bf16x8 operands
 *  stamps          uint64 [n_workgroups * 4 * waves_per_simd * 4], written: per wave the shader clock
 *                  counter and the 100 MHz counter before and after its loop
 *  sink            float [n_workgroups * 4 * waves_per_simd * 64], written (keeps the results alive)
 */
int mla_ceiling_mfma(int waves_per_simd, int n_acc, int n_workgroups, int iters, const void* operands,
                     unsigned long long* stamps, float* sink, void* stream);

/*
 * mla_ceiling_stream — read-only streaming of n_workgroups * bytes_per_workgroup bytes of `src`,
 * workgroup g reading the contiguous span starting at g * bytes_per_workgroup.
 *  mode 0  16-byte non-temporal vector loads, `depth` (4, 8 or 16) loads in flight per lane;
 *          bytes_per_workgroup a multiple of 16; stamps unused (may be NULL)
 *  mode 1  the attention kernel's tile ring: 36864-byte tiles (32 cached rows of 1152 bytes) moved
 *          by 16-byte global->LDS loads into four LDS buffers with `depth` (1, 2 or 3) tiles in
 *          flight, one workgroup barrier per tile; bytes_per_workgroup a multiple of 36864;
 *          stamps uint64 [n_workgroups * 4] written (clock and 100 MHz counters, start and end)
 *  sink    uint32 [n_workgroups]; written only in the practically impossible case that the XOR of
 *          the data equals a fixed constant (keeps the loads alive)
 */
int mla_ceiling_stream(int mode, int depth, int n_workgroups, const void* src, size_t bytes_per_workgroup,
                       unsigned int* sink, unsigned long long* stamps, void* stream);

/*
 * mla_ceiling_lds — LDS read throughput per CU, workgroups of 4 waves (256 workgroups: one per CU;
 * 512 or 1024: two or four per CU).
 *  mode 0  ds_read_b128 (16 bytes per lane), 1: ds_read_b64_tr_b16 (8 bytes per lane, transposed);
 *          each wave issues 8 conflict-free reads per block and waits for them, `iters` blocks
 *  stamps  uint64 [n_workgroups * 4 * 4] written (per wave: clock and 100 MHz counters, start and end)
 *  sink    uint32 [n_workgroups], written only if the folded data equals a fixed constant
 */
int mla_ceiling_lds(int mode, int n_workgroups, int iters, unsigned int* sink, unsigned long long* stamps,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_CEILINGS_H */
