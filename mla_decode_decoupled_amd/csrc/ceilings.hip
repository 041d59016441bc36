// Ceiling microbenchmarks for MI355X (gfx950): what the chip sustains for the two resources the
// latent attention is bound by, measured with the same instructions the attention kernels use.
//   * mfma:   chip-wide v_mfma_f32_32x32x16_bf16 issue with 1 or 2 waves per SIMD, NACC independent
//             accumulators per wave, operands from registers (random bf16 values: the operand data
//             changes the power draw and with it the clock). Every wave records the shader clock
//             counter (s_memtime) and the constant 100 MHz counter (s_memrealtime) around its loop,
//             so the host can tell the issue interval in cycles from the clock the chip ran at.
//   * stream: read-only HBM streaming, (a) 16-byte vector loads into registers with U loads in
//             flight per lane, (b) the attention kernel's tile ring: 32-key tiles of 1152-byte rows
//             (36 KB) moved by 16-byte global->LDS loads into four LDS buffers, `lookahead` tiles in
//             flight, one workgroup barrier per tile, one workgroup per CU.
// Built into libmla_ceilings.so, separate from the attention library.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mla_ceilings.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void stamp(unsigned long long* stamps, int slot, unsigned long long t,
                                      unsigned long long r) {
  stamps[2 * slot] = t;
  stamps[2 * slot + 1] = r;
}

// One workgroup per CU (the host reserves enough LDS to keep a second one out); 64 * WAVES threads.
template <int WAVES, int NACC>
__global__ void __launch_bounds__(64 * WAVES) mfma_peak(int iters, const uint32_t* __restrict__ operands,
                                                         unsigned long long* __restrict__ stamps,
                                                         float* __restrict__ sink) {
  extern __shared__ unsigned char reserve[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gw = blockIdx.x * WAVES + wave;
  uint32_t ua[4], ub[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ua[i] = operands[(gw * 64 + lane) * 8 + i];
    ub[i] = operands[(gw * 64 + lane) * 8 + 4 + i];
  }
  const bf16x8 a = __builtin_bit_cast(bf16x8, ua), b = __builtin_bit_cast(bf16x8, ub);
  f32x16 acc[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k) acc[k] = f32x16{};
  if (threadIdx.x == 0) reserve[0] = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int k = 0; k < NACC; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < NACC; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    stamp(stamps, 2 * gw, t0, r0);
    stamp(stamps, 2 * gw + 1, t1, r1);
  }
  sink[gw * 64 + lane] = s;
}

// (a) vector-load streaming: workgroup g reads the contiguous span [g * per_wg, (g + 1) * per_wg)
// of 16-byte words, U loads in flight per lane, non-temporal.
template <int U>
__global__ void __launch_bounds__(256) stream_vec(const u32x4* __restrict__ src, size_t per_wg,
                                                  unsigned int* __restrict__ sink) {
  const u32x4* p = src + (size_t)blockIdx.x * per_wg;
  u32x4 x = {0, 0, 0, 0};
  for (size_t i = threadIdx.x; i < per_wg; i += 256 * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + (size_t)u * 256;
      v[u] = j < per_wg ? __builtin_nontemporal_load(p + j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u];
  }
  const unsigned int r = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (r == 0x9e3779b9u) sink[blockIdx.x] = r;   // practically never: keeps the loads alive
}

// (b) the attention kernel's tile ring: workgroup g streams tiles g * tiles .. (g + 1) * tiles - 1
// (36 KB each) into four LDS buffers with nine 1 KB global->LDS loads per wave and tile, keeping
// LA tiles in flight; per tile it waits for the oldest, passes one barrier and reads one dword
// back, as the attention loop's barrier-per-tile does. The loads are issued from inline asm and the
// barrier waits only for LDS traffic, as in the attention kernels: the compiler would otherwise
// wait for every global->LDS load in flight at each barrier.
constexpr int TILE_BYTES = 32 * 1152;
constexpr int NBUF = 4;

__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int LA>
__global__ void __launch_bounds__(256) stream_lds(const unsigned char* __restrict__ src, int tiles,
                                                  unsigned int* __restrict__ sink,
                                                  unsigned long long* __restrict__ stamps) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned char* base = src + (size_t)blockIdx.x * tiles * TILE_BYTES + (w * 9 * 64 + lane) * 16;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  auto issue = [&](int t) {
    const unsigned char* g = base + (size_t)t * TILE_BYTES;
    const uint32_t d = __builtin_amdgcn_readfirstlane(lds0 + (t % NBUF) * TILE_BYTES + w * 9 * 1024);
#pragma unroll
    for (int it = 0; it < 9; ++it) dma16(g + it * 1024, d + it * 1024);
  };
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int t = 0; t < LA && t < tiles; ++t) issue(t);
  unsigned int x = 0;
  for (int t = 0; t < tiles; ++t) {
    // the tile t landed: at most (tiles issued after it) x 9 loads of this wave outstanding
    const int after = (t + LA - 1 < tiles ? LA - 1 : tiles - 1 - t);
    if (after >= 2)
      __builtin_amdgcn_s_waitcnt((18 & 15) | ((18 >> 4) << 14) | (7 << 4) | (15 << 8));
    else if (after == 1)
      __builtin_amdgcn_s_waitcnt(9 | (7 << 4) | (15 << 8));
    else
      __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    lds_barrier();   // every wave's share of tile t is in
    x ^= *reinterpret_cast<const unsigned int*>(lds + (t % NBUF) * TILE_BYTES + threadIdx.x * 16);
    lds_barrier();   // every wave read buffer t % NBUF before it is refilled
    if (t + LA < tiles) issue(t + LA);
  }
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    stamp(stamps, 2 * blockIdx.x, t0, r0);
    stamp(stamps, 2 * blockIdx.x + 1, t1, r1);
  }
  if (x == 0x9e3779b9u) sink[blockIdx.x] = x;
}

// (c) LDS read throughput of the two read forms the attention kernels use, workgroups of 4 waves
// (one to four per CU, by the grid size): ds_read_b128 (16 bytes per lane, the score operands) and ds_read_b64_tr_b16 (8 bytes
// per lane, transposed, the value operands). Each wave issues 8 reads per block (every lane a
// distinct 16-byte slot of a 1 KB row, rows 1 KB apart: no bank conflicts), waits for them, folds
// the data into one register, and repeats; `iters` blocks per wave.
template <int MODE>
__global__ void __launch_bounds__(256) lds_read(int iters, unsigned int* __restrict__ sink,
                                                unsigned long long* __restrict__ stamps) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // fill this wave's 8 KB so that the reads see defined data
  for (int i = lane; i < 8 * 1024 / 4; i += 64)
    reinterpret_cast<unsigned int*>(lds + w * 8192)[i] = (unsigned int)(i * 2654435761u);
  __syncthreads();
  const uint32_t a = (uint32_t)(uintptr_t)(lds + w * 8192 + lane * 16);
  unsigned int x = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    u32x4 v0, v1, v2, v3, v4, v5, v6, v7;
    if (MODE == 0) {
      asm volatile(
          "ds_read_b128 %0, %8 offset:0\n\tds_read_b128 %1, %8 offset:1024\n\t"
          "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
          "ds_read_b128 %4, %8 offset:4096\n\tds_read_b128 %5, %8 offset:5120\n\t"
          "ds_read_b128 %6, %8 offset:6144\n\tds_read_b128 %7, %8 offset:7168\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6), "=&v"(v7)
          : "v"(a)
          : "memory");
      x ^= v0[0] ^ v1[1] ^ v2[2] ^ v3[3] ^ v4[0] ^ v5[1] ^ v6[2] ^ v7[3];
    } else {
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      u32x2 h0, h1, h2, h3, h4, h5, h6, h7;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8 offset:0\n\tds_read_b64_tr_b16 %1, %8 offset:1024\n\t"
          "ds_read_b64_tr_b16 %2, %8 offset:2048\n\tds_read_b64_tr_b16 %3, %8 offset:3072\n\t"
          "ds_read_b64_tr_b16 %4, %8 offset:4096\n\tds_read_b64_tr_b16 %5, %8 offset:5120\n\t"
          "ds_read_b64_tr_b16 %6, %8 offset:6144\n\tds_read_b64_tr_b16 %7, %8 offset:7168\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(h0), "=&v"(h1), "=&v"(h2), "=&v"(h3), "=&v"(h4), "=&v"(h5), "=&v"(h6), "=&v"(h7)
          : "v"(a - (uint32_t)(lane * 8))   // 8 bytes per lane: lanes cover a 512-byte span of the row
          : "memory");
      x ^= h0[0] ^ h1[1] ^ h2[0] ^ h3[1] ^ h4[0] ^ h5[1] ^ h6[0] ^ h7[1];
      (void)v0; (void)v1; (void)v2; (void)v3; (void)v4; (void)v5; (void)v6; (void)v7;
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    const int gw = blockIdx.x * 4 + w;
    stamp(stamps, 2 * gw, t0, r0);
    stamp(stamps, 2 * gw + 1, t1, r1);
  }
  if (x == 0x9e3779b9u) sink[blockIdx.x] = x;
}

// (d) one wave per SIMD, one dependent chain of v_mfma_f32_32x32x16_bf16, in inline asm so that the
// accumulator's register file is fixed: VARIANT 0 accumulates in VGPRs, 1 in AGPRs; 2 and 3 do the
// same with one ds_read_b128 (a fresh 16-byte operand per lane, conflict-free) issued before each
// MFMA and waited for four MFMAs later, the way the attention kernel feeds its score chain.
template <int VARIANT>
__global__ void __launch_bounds__(256) mfma_chain(int iters, const uint32_t* __restrict__ operands,
                                                  unsigned long long* __restrict__ stamps, float* __restrict__ sink) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gw = blockIdx.x * 4 + wave;
  for (int i = threadIdx.x; i < 16384 / 4; i += 256) reinterpret_cast<uint32_t*>(lds)[i] = operands[i & 511];
  __syncthreads();
  uint32_t ua[4], ub[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ua[i] = operands[(gw * 64 + lane) * 8 + i];
    ub[i] = operands[(gw * 64 + lane) * 8 + 4 + i];
  }
  const bf16x8 a = __builtin_bit_cast(bf16x8, ua), b = __builtin_bit_cast(bf16x8, ub);
  const uint32_t la = (uint32_t)(uintptr_t)(lds + wave * 4096 + lane * 16);
  f32x16 acc = f32x16{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    if (VARIANT == 0) {
      asm volatile(
          "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
          : "+v"(acc) : "v"(a), "v"(b));
    } else if (VARIANT == 1) {
      asm volatile(
          "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
          "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
          : "+a"(acc) : "v"(a), "v"(b));
    } else {
      // ring of four operand slots: the read for MFMA k + 4 goes out right after MFMA k issues
      typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
      u32x4v r0v, r1v, r2v, r3v;
#define MLA_CHAIN_BODY(ACC)                                                                                  \
      asm volatile(                                                                                         \
          "ds_read_b128 %1, %7 offset:0\n\tds_read_b128 %2, %7 offset:1024\n\t"                             \
          "ds_read_b128 %3, %7 offset:2048\n\tds_read_b128 %4, %7 offset:3072\n\t"                          \
          "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %6, %0\n\tds_read_b128 %1, %7 offset:0\n\t" \
          "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 %0, %2, %6, %0\n\tds_read_b128 %2, %7 offset:1024\n\t" \
          "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 %0, %3, %6, %0\n\tds_read_b128 %3, %7 offset:2048\n\t" \
          "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 %0, %4, %6, %0\n\tds_read_b128 %4, %7 offset:3072\n\t" \
          "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %6, %0\n\t"                              \
          "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %0, %2, %6, %0\n\t"                              \
          "s_waitcnt lgkmcnt(1)\n\tv_mfma_f32_32x32x16_bf16 %0, %3, %6, %0\n\t"                              \
          "s_waitcnt lgkmcnt(0)\n\tv_mfma_f32_32x32x16_bf16 %0, %4, %6, %0"                                    \
          : ACC(acc), "=&v"(r0v), "=&v"(r1v), "=&v"(r2v), "=&v"(r3v), "=&v"(r3v)                              \
          : "v"(b), "v"(la)                                                                                   \
          : "memory")
      if (VARIANT == 2) {
        MLA_CHAIN_BODY("+v");
      } else if (VARIANT == 3) {
        MLA_CHAIN_BODY("+a");
      } else if (VARIANT == 4) {
        // eight slots, the waits batched: one s_waitcnt per four MFMAs
        u32x4v r4v, r5v, r6v, r7v;
        asm volatile(
            "ds_read_b128 %1, %9 offset:0\n\tds_read_b128 %2, %9 offset:1024\n\t"
            "ds_read_b128 %3, %9 offset:2048\n\tds_read_b128 %4, %9 offset:3072\n\t"
            "ds_read_b128 %5, %9 offset:0\n\tds_read_b128 %6, %9 offset:1024\n\t"
            "ds_read_b128 %7, %9 offset:2048\n\tds_read_b128 %8, %9 offset:3072\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %1, %10, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %2, %10, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %3, %10, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %4, %10, %0\n\t"
            "ds_read_b128 %1, %9 offset:0\n\tds_read_b128 %2, %9 offset:1024\n\t"
            "ds_read_b128 %3, %9 offset:2048\n\tds_read_b128 %4, %9 offset:3072\n\t"
            "s_waitcnt lgkmcnt(4)\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %5, %10, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %6, %10, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %7, %10, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %8, %10, %0\n\t"
            "s_waitcnt lgkmcnt(0)\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %1, %10, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %2, %10, %0\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %3, %10, %0\n\tv_mfma_f32_32x32x16_bf16 %0, %4, %10, %0"
            : "+a"(acc), "=&v"(r0v), "=&v"(r1v), "=&v"(r2v), "=&v"(r3v), "=&v"(r4v), "=&v"(r5v), "=&v"(r6v), "=&v"(r7v)
            : "v"(la), "v"(b)
            : "memory");
      } else if (VARIANT == 5) {
        // no LDS: one independent VALU op between consecutive MFMAs
        float t0 = 0.0f;
        asm volatile(
            "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\tv_add_f32 %1, 1.0, %1\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\tv_add_f32 %1, 1.0, %1\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\tv_add_f32 %1, 1.0, %1\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\tv_add_f32 %1, 1.0, %1\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\tv_add_f32 %1, 1.0, %1\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\tv_add_f32 %1, 1.0, %1\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\tv_add_f32 %1, 1.0, %1\n\t"
            "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\tv_add_f32 %1, 1.0, %1"
            : "+a"(acc), "+v"(t0) : "v"(a), "v"(b));
        if (t0 == 12345.0f) acc[0] += 1.0f;
      } else if (VARIANT == 7 || VARIANT == 8) {
        // two (7) or four (8) independent accumulators taken in turn, one ds_read_b128 per MFMA
        // (the second accumulator lives in v[56:71] / a[16:31], named in the asm)
        if (VARIANT == 7) {
          asm volatile(
              "ds_read_b128 v[40:43], %1 offset:0\n\tds_read_b128 v[44:47], %1 offset:1024\n\t"
              "ds_read_b128 v[48:51], %1 offset:2048\n\tds_read_b128 v[52:55], %1 offset:3072\n\t"
              "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 %0, v[40:43], %2, %0\n\tds_read_b128 v[40:43], %1 offset:0\n\t"
              "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 a[16:31], v[44:47], %2, a[16:31]\n\tds_read_b128 v[44:47], %1 offset:1024\n\t"
              "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 %0, v[48:51], %2, %0\n\tds_read_b128 v[48:51], %1 offset:2048\n\t"
              "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 a[16:31], v[52:55], %2, a[16:31]\n\tds_read_b128 v[52:55], %1 offset:3072\n\t"
              "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 %0, v[40:43], %2, %0\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 a[16:31], v[44:47], %2, a[16:31]\n\t"
              "s_waitcnt lgkmcnt(1)\n\tv_mfma_f32_32x32x16_bf16 %0, v[48:51], %2, %0\n\t"
              "s_waitcnt lgkmcnt(0)\n\tv_mfma_f32_32x32x16_bf16 a[16:31], v[52:55], %2, a[16:31]"
              : "+a"(acc) : "v"(la), "v"(b)
              : "memory", "v40", "v41", "v42", "v43", "v44", "v45", "v46", "v47", "v48", "v49", "v50", "v51", "v52",
                "v53", "v54", "v55", "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27",
                "a28", "a29", "a30", "a31");
        } else {
          asm volatile(
              "ds_read_b128 v[40:43], %1 offset:0\n\tds_read_b128 v[44:47], %1 offset:1024\n\t"
              "ds_read_b128 v[48:51], %1 offset:2048\n\tds_read_b128 v[52:55], %1 offset:3072\n\t"
              "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 %0, v[40:43], %2, %0\n\tds_read_b128 v[40:43], %1 offset:0\n\t"
              "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 a[16:31], v[44:47], %2, a[16:31]\n\tds_read_b128 v[44:47], %1 offset:1024\n\t"
              "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 a[32:47], v[48:51], %2, a[32:47]\n\tds_read_b128 v[48:51], %1 offset:2048\n\t"
              "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 a[48:63], v[52:55], %2, a[48:63]\n\tds_read_b128 v[52:55], %1 offset:3072\n\t"
              "s_waitcnt lgkmcnt(3)\n\tv_mfma_f32_32x32x16_bf16 %0, v[40:43], %2, %0\n\t"
              "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 a[16:31], v[44:47], %2, a[16:31]\n\t"
              "s_waitcnt lgkmcnt(1)\n\tv_mfma_f32_32x32x16_bf16 a[32:47], v[48:51], %2, a[32:47]\n\t"
              "s_waitcnt lgkmcnt(0)\n\tv_mfma_f32_32x32x16_bf16 a[48:63], v[52:55], %2, a[48:63]"
              : "+a"(acc) : "v"(la), "v"(b)
              : "memory", "v40", "v41", "v42", "v43", "v44", "v45", "v46", "v47", "v48", "v49", "v50", "v51", "v52",
                "v53", "v54", "v55", "a16", "a17", "a18", "a19", "a20", "a21", "a22", "a23", "a24", "a25", "a26", "a27",
                "a28", "a29", "a30", "a31", "a32", "a33", "a34", "a35", "a36", "a37", "a38", "a39", "a40", "a41", "a42",
                "a43", "a44", "a45", "a46", "a47", "a48", "a49", "a50", "a51", "a52", "a53", "a54", "a55", "a56", "a57",
                "a58", "a59", "a60", "a61", "a62", "a63");
        }
      } else {
        // P.V feeding: two ds_read_b64_tr_b16 (one A operand) per MFMA, ring of four operands in
        // v[40:55] (named in the asm, declared clobbered)
        asm volatile(
            "ds_read_b64_tr_b16 v[40:41], %1 offset:0\n\tds_read_b64_tr_b16 v[42:43], %1 offset:512\n\t"
            "ds_read_b64_tr_b16 v[44:45], %1 offset:1024\n\tds_read_b64_tr_b16 v[46:47], %1 offset:1536\n\t"
            "ds_read_b64_tr_b16 v[48:49], %1 offset:2048\n\tds_read_b64_tr_b16 v[50:51], %1 offset:2560\n\t"
            "ds_read_b64_tr_b16 v[52:53], %1 offset:3072\n\tds_read_b64_tr_b16 v[54:55], %1 offset:3584\n\t"
            "s_waitcnt lgkmcnt(6)\n\tv_mfma_f32_32x32x16_bf16 %0, v[40:43], %2, %0\n\t"
            "ds_read_b64_tr_b16 v[40:41], %1 offset:0\n\tds_read_b64_tr_b16 v[42:43], %1 offset:512\n\t"
            "s_waitcnt lgkmcnt(6)\n\tv_mfma_f32_32x32x16_bf16 %0, v[44:47], %2, %0\n\t"
            "ds_read_b64_tr_b16 v[44:45], %1 offset:1024\n\tds_read_b64_tr_b16 v[46:47], %1 offset:1536\n\t"
            "s_waitcnt lgkmcnt(6)\n\tv_mfma_f32_32x32x16_bf16 %0, v[48:51], %2, %0\n\t"
            "ds_read_b64_tr_b16 v[48:49], %1 offset:2048\n\tds_read_b64_tr_b16 v[50:51], %1 offset:2560\n\t"
            "s_waitcnt lgkmcnt(6)\n\tv_mfma_f32_32x32x16_bf16 %0, v[52:55], %2, %0\n\t"
            "ds_read_b64_tr_b16 v[52:53], %1 offset:3072\n\tds_read_b64_tr_b16 v[54:55], %1 offset:3584\n\t"
            "s_waitcnt lgkmcnt(6)\n\tv_mfma_f32_32x32x16_bf16 %0, v[40:43], %2, %0\n\t"
            "s_waitcnt lgkmcnt(4)\n\tv_mfma_f32_32x32x16_bf16 %0, v[44:47], %2, %0\n\t"
            "s_waitcnt lgkmcnt(2)\n\tv_mfma_f32_32x32x16_bf16 %0, v[48:51], %2, %0\n\t"
            "s_waitcnt lgkmcnt(0)\n\tv_mfma_f32_32x32x16_bf16 %0, v[52:55], %2, %0"
            : "+a"(acc)
            : "v"(la - (uint32_t)(lane * 8)), "v"(b)
            : "memory", "v40", "v41", "v42", "v43", "v44", "v45", "v46", "v47", "v48", "v49", "v50", "v51", "v52",
              "v53", "v54", "v55");
      }
#undef MLA_CHAIN_BODY
      (void)a;
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += acc[e];
  if (lane == 0) {
    stamp(stamps, 2 * gw, t0, r0);
    stamp(stamps, 2 * gw + 1, t1, r1);
  }
  sink[gw * 64 + lane] = s;
}

template <int WAVES, int NACC>
hipError_t launch_mfma(int n_wg, int iters, const uint32_t* ops, unsigned long long* stamps, float* sink,
                       hipStream_t st) {
  constexpr int kReserve = 96 * 1024;   // more than half of the 160 KB: one workgroup per CU
  hipError_t e = hipFuncSetAttribute((const void*)mfma_peak<WAVES, NACC>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kReserve);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mfma_peak<WAVES, NACC>), dim3(n_wg), dim3(64 * WAVES), kReserve, st, iters, ops, stamps, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int mla_ceiling_mfma(int waves_per_simd, int n_acc, int n_workgroups, int iters, const void* operands,
                     unsigned long long* stamps, float* sink, void* stream) {
  if (n_workgroups < 1 || iters < 1 || !operands || !stamps || !sink) return 1;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  const uint32_t* ops = (const uint32_t*)operands;
  if (waves_per_simd == 1 && n_acc == 4) e = launch_mfma<4, 4>(n_workgroups, iters, ops, stamps, sink, st);
  else if (waves_per_simd == 1 && n_acc == 8) e = launch_mfma<4, 8>(n_workgroups, iters, ops, stamps, sink, st);
  else if (waves_per_simd == 1 && n_acc == 1) e = launch_mfma<4, 1>(n_workgroups, iters, ops, stamps, sink, st);
  else if (waves_per_simd == 2 && n_acc == 4) e = launch_mfma<8, 4>(n_workgroups, iters, ops, stamps, sink, st);
  else if (waves_per_simd == 2 && n_acc == 8) e = launch_mfma<8, 8>(n_workgroups, iters, ops, stamps, sink, st);
  else if (waves_per_simd == 2 && n_acc >= 100 && n_acc <= 108) {
    // the same single-wave chains with two workgroups of 4 waves per CU (two waves per SIMD): the
    // host passes twice as many workgroups
    constexpr int kLds = 20 * 1024;
    const void* fns[9] = {(const void*)mfma_chain<0>, (const void*)mfma_chain<1>, (const void*)mfma_chain<2>,
                          (const void*)mfma_chain<3>, (const void*)mfma_chain<4>, (const void*)mfma_chain<5>,
                          (const void*)mfma_chain<6>, (const void*)mfma_chain<7>, (const void*)mfma_chain<8>};
    e = hipFuncSetAttribute(fns[n_acc - 100], hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e == hipSuccess) {
      switch (n_acc) {
        case 101: hipLaunchKernelGGL(mfma_chain<1>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        case 103: hipLaunchKernelGGL(mfma_chain<3>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        case 105: hipLaunchKernelGGL(mfma_chain<5>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        case 106: hipLaunchKernelGGL(mfma_chain<6>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        default: return 2;
      }
      e = hipGetLastError();
    }
  } else if (waves_per_simd == 1 && n_acc >= 100 && n_acc <= 108) {
    // single-chain variants (see mfma_chain): 100 VGPR accumulator, 101 AGPR, 102/103 the same fed by LDS,
    // 104 LDS-fed with batched waits, 105 one VALU op per MFMA, 106 fed by transposed reads, 107 / 108
    // LDS-fed over two / four independent accumulators
    constexpr int kLds = 96 * 1024;
    const void* fns[9] = {(const void*)mfma_chain<0>, (const void*)mfma_chain<1>, (const void*)mfma_chain<2>,
                          (const void*)mfma_chain<3>, (const void*)mfma_chain<4>, (const void*)mfma_chain<5>,
                          (const void*)mfma_chain<6>, (const void*)mfma_chain<7>, (const void*)mfma_chain<8>};
    e = hipFuncSetAttribute(fns[n_acc - 100], hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e == hipSuccess) {
      switch (n_acc) {
        case 100: hipLaunchKernelGGL(mfma_chain<0>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        case 101: hipLaunchKernelGGL(mfma_chain<1>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        case 102: hipLaunchKernelGGL(mfma_chain<2>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        case 103: hipLaunchKernelGGL(mfma_chain<3>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        case 104: hipLaunchKernelGGL(mfma_chain<4>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        case 105: hipLaunchKernelGGL(mfma_chain<5>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        case 107: hipLaunchKernelGGL(mfma_chain<7>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        case 108: hipLaunchKernelGGL(mfma_chain<8>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
        default: hipLaunchKernelGGL(mfma_chain<6>, dim3(n_workgroups), dim3(256), kLds, st, iters, ops, stamps, sink); break;
      }
      e = hipGetLastError();
    }
  } else return 2;
  return e == hipSuccess ? 0 : 4;
}

int mla_ceiling_lds(int mode, int n_workgroups, int iters, unsigned int* sink, unsigned long long* stamps,
                    void* stream) {
  if (n_workgroups < 1 || iters < 1 || !sink || !stamps) return 1;
  if (mode != 0 && mode != 1) return 2;
  hipStream_t st = (hipStream_t)stream;
  constexpr int kReserve = 40 * 1024;   // 32 KB used; up to four workgroups per CU
  const void* fn = mode == 0 ? (const void*)lds_read<0> : (const void*)lds_read<1>;
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kReserve) != hipSuccess) return 4;
  if (mode == 0)
    hipLaunchKernelGGL(lds_read<0>, dim3(n_workgroups), dim3(256), kReserve, st, iters, sink, stamps);
  else
    hipLaunchKernelGGL(lds_read<1>, dim3(n_workgroups), dim3(256), kReserve, st, iters, sink, stamps);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int mla_ceiling_stream(int mode, int depth, int n_workgroups, const void* src, size_t bytes_per_workgroup,
                       unsigned int* sink, unsigned long long* stamps, void* stream) {
  if (n_workgroups < 1 || !src || !sink || bytes_per_workgroup == 0) return 1;
  hipStream_t st = (hipStream_t)stream;
  if (mode == 0) {
    if (bytes_per_workgroup % 16 != 0) return 1;
    const size_t per = bytes_per_workgroup / 16;
    switch (depth) {
      case 4: hipLaunchKernelGGL(stream_vec<4>, dim3(n_workgroups), dim3(256), 0, st, (const u32x4*)src, per, sink); break;
      case 8: hipLaunchKernelGGL(stream_vec<8>, dim3(n_workgroups), dim3(256), 0, st, (const u32x4*)src, per, sink); break;
      case 16: hipLaunchKernelGGL(stream_vec<16>, dim3(n_workgroups), dim3(256), 0, st, (const u32x4*)src, per, sink); break;
      default: return 2;
    }
    return hipGetLastError() == hipSuccess ? 0 : 4;
  }
  if (mode == 1) {
    if (!stamps || bytes_per_workgroup % TILE_BYTES != 0) return 1;
    const int tiles = (int)(bytes_per_workgroup / TILE_BYTES);
    const int lds = NBUF * TILE_BYTES;
    hipError_t e = hipSuccess;
    switch (depth) {
      case 1:
        e = hipFuncSetAttribute((const void*)stream_lds<1>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e == hipSuccess)
          hipLaunchKernelGGL(stream_lds<1>, dim3(n_workgroups), dim3(256), lds, st, (const unsigned char*)src, tiles, sink, stamps);
        break;
      case 2:
        e = hipFuncSetAttribute((const void*)stream_lds<2>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e == hipSuccess)
          hipLaunchKernelGGL(stream_lds<2>, dim3(n_workgroups), dim3(256), lds, st, (const unsigned char*)src, tiles, sink, stamps);
        break;
      case 3:
        e = hipFuncSetAttribute((const void*)stream_lds<3>, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e == hipSuccess)
          hipLaunchKernelGGL(stream_lds<3>, dim3(n_workgroups), dim3(256), lds, st, (const unsigned char*)src, tiles, sink, stamps);
        break;
      default: return 2;
    }
    if (e != hipSuccess) return 4;
    return hipGetLastError() == hipSuccess ? 0 : 4;
  }
  return 2;
}

}  // extern "C"
