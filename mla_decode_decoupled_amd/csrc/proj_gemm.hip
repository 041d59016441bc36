// Query absorption and latent output projection as per-head MFMA GEMMs, for many query rows
// at once (batched decode, chunked prefill) at the DeepSeek-V2/V3 shape (128 heads,
// d_nope = d_v = 128, d_latent = 512, d_rope = 64, bf16 weights).
//
//   absorb: q~[r, i, :] = q_nope[r, i, :] W_UK[i]      ([R x 128] x [128 x 512] per head)
//   out:    o[r, i, :]  = z[r, i, :] W_UV[i]^T         ([R x 512] x [512 x 128] per head)
// ("从零理解 MLA", section "矩阵吸收": the content query is carried into the latent space through
// W_UK, and the latent attention output comes back through W_UV.)
//
// A workgroup owns one head and 64 query rows; the weight slab of that head is read once per
// workgroup, so weights are re-read only R / 64 times. Both contractions run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation. The absorbed query is rounded to bf16 once, as
// q_packed is stored. z is float32: it enters the MFMA as two bf16 parts (hi = bf16(z),
// lo = bf16(z - hi)), whose products with the bf16 weight are exact, so o keeps float32-level
// accuracy before its final rounding.
//
// Every operand reaches LDS through direct 1 KB global->LDS loads of whole row segments (an
// MFMA fragment loaded straight from global memory would touch 32 rows per instruction); rows
// are XOR-swizzled by 16-byte piece so that the 16 rows read together by a fragment load fall on
// distinct bank groups.
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace gemm {

constexpr int H = 128;
constexpr int DN = 128;   // d_nope = d_v
constexpr int DC = 512;
constexpr int DR = 64;
constexpr int ROW = DC + DR;
constexpr int BM = 64;    // query rows per workgroup

typedef __bf16 bf16x8e __attribute__((ext_vector_type(8)));
typedef short i16x4e __attribute__((ext_vector_type(4)));
typedef float f32x16e __attribute__((ext_vector_type(16)));

// one 16-byte-per-lane direct global->LDS load: lane l writes LDS bytes lds_base + 16 l
__device__ __forceinline__ void dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ f32x16e mfma(bf16x8e a, bf16x8e b, f32x16e c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)MLA_LDS(const char, p); }

// ---------------------------------------------------------------- absorb
// grid (4 column quarters, ceil(R / 64), H), 256 threads: one workgroup per (head i, 64 rows,
// quarter of the 512 latent columns), so the 4 quarters of a row tile run side by side and share
// its q_nope rows through L2. LDS: W_UK[i][:, quarter] (128 rows a x 256 B; 16-byte piece c of
// row a sits at slot c ^ 4 (a & 3), so the 4 rows x 4 pieces of a transpose read hit distinct
// banks), the 64 q_nope rows (256 B each, pieces XOR-swizzled by row & 15), the RoPE frequencies;
// the output tile reuses the weight area. Quarter q also rotates a quarter of each row's position
// query.
constexpr int WQ_ROW = 128 * 2;                 // 256 B: one quarter of a W_UK row
constexpr int A_OFF = DN * WQ_ROW;              // 32768
constexpr int THETA_OFF = A_OFF + BM * DN * 2;  // 49152
constexpr int ABSORB_LDS = THETA_OFF + (DR / 2) * 8;
constexpr int OUT_STRIDE = 128 * 2 + 16;        // staged output rows (bf16, one quarter)
static_assert(BM * OUT_STRIDE <= A_OFF, "output tile must fit the weight area");

// B operand (16 k x 32 n) of the swizzled quarter slab W[k][n] (rows of 256 B), k-step s, column
// block nb, via two transpose reads: lane l = 16q + L (g = l / 32) gets W[16s + 8g + e][32nb + l % 32]
// for e = 0..7; source lane L of each 16-lane group points at row 16s + 8g + 4h + L/4, columns
// 32nb + 16(q & 1) + 4(L & 3) .. +3 (in 16-byte piece (that column) / 8, swizzled), halves h = 0, 1.
__device__ __forceinline__ bf16x8e wq_fragment(const unsigned char* slab, int s, int nb, int lane) {
  const int g = lane >> 5, q = lane >> 4, L = lane & 15;
  const int col = 32 * nb + 16 * (q & 1) + 4 * (L & 3);
  i16x4e hv[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 16 * s + 8 * g + 4 * h + (L >> 2);
    const int piece = (col >> 3) ^ (4 * (row & 3));
    hv[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4e*)MLA_LDS(
        unsigned char, slab + row * WQ_ROW + 16 * piece + 2 * (col & 7)));
  }
  return __builtin_bit_cast(bf16x8e, hv);
}

__global__ void __launch_bounds__(256) absorb_q_gemm(const bf16* __restrict__ q_nope, const bf16* __restrict__ q_rope,
                                                     const int32_t* __restrict__ q_pos, const bf16* __restrict__ w_uk,
                                                     bf16* __restrict__ q_packed, int n_rows, double base) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int quarter = blockIdx.x, r0 = blockIdx.y * BM, i = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int nr = min(BM, n_rows - r0);
  double* theta = reinterpret_cast<double*>(smem + THETA_OFF);

  // W_UK[i][:, quarter]: four 256 B rows per instruction (wave w: instructions w, w + 4, ..);
  // lane l fills row 4k + l/16, slot l%16 with piece (l%16) ^ 4 (row & 3)
  {
    const uint32_t lds0 = lds_addr(smem);
#pragma unroll
    for (int k = w; k < DN / 4; k += 4) {
      const int row = 4 * k + (lane >> 4), slot = lane & 15;
      const bf16* src = w_uk + ((size_t)i * DN + row) * DC + 128 * quarter + 8 * (slot ^ (4 * (row & 3)));
      dma16(src, __builtin_amdgcn_readfirstlane(lds0 + k * 1024));
    }
  }
  // q_nope rows: four 256 B rows per instruction; lane l fills row 4q + l/16, slot l%16 with
  // piece (l%16) ^ (row & 15). Rows past the end repeat the last row (never stored).
  {
    const uint32_t lds0 = lds_addr(smem + A_OFF);
#pragma unroll
    for (int q = w; q < BM / 4; q += 4) {
      const int row = 4 * q + (lane >> 4), slot = lane & 15;
      const int rs = min(row, nr - 1);
      const bf16* src = q_nope + ((size_t)(r0 + rs) * H + i) * DN + 8 * (slot ^ (row & 15));
      dma16(src, __builtin_amdgcn_readfirstlane(lds0 + q * 1024));
    }
  }
  if (t < DR / 2) theta[t] = rope_theta(base, t, DR);
  __builtin_amdgcn_s_waitcnt(0);   // vmcnt 0: this wave's rows have landed
  __syncthreads();

  // position part of these rows: quarter q rotates pairs 8q .. 8q + 7 (dims 16q .. 16q + 15), one
  // thread per row; float64-reduced angle, float32 rotation, two 16-byte pieces in and out
  if (t < nr) {
    const int rr = t;
    const size_t r = (size_t)(r0 + rr);
    const int64_t pos = q_pos[r];
    const i32x4* src = reinterpret_cast<const i32x4*>(q_rope + (r * H + i) * DR + 16 * quarter);
    i32x4 x[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) x[u] = src[u];
    i32x4 y[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {   // one pair (2j, 2j+1) per 32-bit word
        const int j = 8 * quarter + 4 * u + e;
        float sn, co;
        rope_sincos(theta[j], pos, &sn, &co);
        const uint32_t wd = (uint32_t)x[u][e];
        const float x0 = __uint_as_float(wd << 16), x1 = __uint_as_float(wd & 0xFFFF0000u);
        const bf16 y0 = (bf16)(x0 * co - x1 * sn), y1 = (bf16)(x0 * sn + x1 * co);
        y[u][e] = (int)((uint32_t)__builtin_bit_cast(unsigned short, y0) |
                        ((uint32_t)__builtin_bit_cast(unsigned short, y1) << 16));
      }
    i32x4* dst = reinterpret_cast<i32x4*>(q_packed + (r * H + i) * ROW + DC + 16 * quarter);
#pragma unroll
    for (int u = 0; u < 2; ++u) dst[u] = y[u];
  }

  // wave w: quarter columns 32w .. 32w + 31 x both row blocks
  f32x16e acc[2] = {f32x16e{}, f32x16e{}};
#pragma unroll
  for (int s = 0; s < DN / 16; ++s) {
    bf16x8e a[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int m = 32 * rb + l32;
      a[rb] = *reinterpret_cast<const bf16x8e*>(smem + A_OFF + m * (DN * 2) + 16 * ((2 * s + g) ^ (m & 15)));
    }
    const bf16x8e b = wq_fragment(smem, s, w, lane);
    acc[0] = mfma(a[0], b, acc[0]);
    acc[1] = mfma(a[1], b, acc[1]);
  }
  __syncthreads();   // every wave is done with W: the area takes the output tile

  // D layout: lane holds quarter column 32w + l32 of rows 32rb + 8j + 4g + e
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 32 * rb + 8 * j + 4 * g + e, col = 32 * w + l32;
        *reinterpret_cast<bf16*>(smem + row * OUT_STRIDE + 2 * col) = (bf16)acc[rb][4 * j + e];
      }
  __syncthreads();
  // the quarter's 256 B of each row out: 64 rows x 16 pieces of 16 bytes
  for (int p = t; p < nr * 16; p += 256) {
    const int row = p >> 4, ch = p & 15;
    *reinterpret_cast<i32x4*>(q_packed + ((size_t)(r0 + row) * H + i) * ROW + 128 * quarter + ch * 8) =
        *reinterpret_cast<const i32x4*>(smem + row * OUT_STRIDE + ch * 16);
  }
}

// ---------------------------------------------------------------- output projection
// grid (ceil(R / 64), H, DN / NO), 256 threads: one row tile, one head and NO of its 128 outputs
// per workgroup. NO = 128 normally; NO = 64 when there is a single row tile, so that 64 rows still
// give 256 workgroups (with more tiles the halves would each load and split the z rows again). The
// latent dimension is taken in two halves of 256; per half LDS holds W_UV[i][the NO outputs, half
// of the latent] (NO rows of 512 B) and the 64 z rows' half (64 rows of 1 KB float32, then split in
// place into bf16 hi / lo parts), both XOR-swizzled by 16-byte piece. The NO / 32 output blocks of
// 32 are dealt to the waves first, then the two row blocks of 32: wave w computes outputs
// 32 (w % (NO / 32)) .. +31 for RBW = NO / 64 row blocks from (w / (NO / 32)) RBW on. Every output
// sums the same products in the same order whatever NO.
constexpr int KH = DC / 2;                    // latent columns per half
constexpr int WV_ROW = KH * 2;                // 512 B
constexpr int Z_ROW = KH * 4;                 // 1024 B
template <int NO> constexpr int outp_z_off() { return NO * WV_ROW; }
template <int NO> constexpr int outp_lds() { return outp_z_off<NO>() + BM * Z_ROW; }   // 128 KB or 96 KB

template <int NO>
__global__ void __launch_bounds__(256) out_proj_gemm(const float* __restrict__ z, const bf16* __restrict__ w_uv,
                                                     bf16* __restrict__ o, int n_rows) {
  static_assert(NO == 64 || NO == 128, "half or all of the outputs");
  constexpr int Z_OFF = outp_z_off<NO>();
  constexpr int WO = NO / 32;    // waves across the outputs
  constexpr int RBW = NO / 64;   // row blocks of 32 per wave
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int i = blockIdx.y, r0 = blockIdx.x * BM, v0 = blockIdx.z * NO;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int nr = min(BM, n_rows - r0);
  const uint32_t lds_w = lds_addr(smem), lds_z = lds_addr(smem + Z_OFF);

  f32x16e acc[RBW];
#pragma unroll
  for (int k = 0; k < RBW; ++k) acc[k] = f32x16e{};
  const int ob = w % WO, rb0 = (w / WO) * RBW;
  for (int kh = 0; kh < 2; ++kh) {
    if (kh > 0) __syncthreads();   // the previous half is no longer read
    // W_UV rows: two 512 B rows per instruction, lane l -> row 2q + l/32, slot (l%32) holds
    // piece (l%32) ^ (row & 15)
#pragma unroll 4
    for (int q = w; q < NO / 2; q += 4) {
      const int row = 2 * q + (lane >> 5), slot = lane & 31;
      const bf16* src = w_uv + ((size_t)i * DN + v0 + row) * DC + kh * KH + 8 * (slot ^ (row & 15));
      dma16(src, __builtin_amdgcn_readfirstlane(lds_w + q * 1024));
    }
    // z rows: one 1 KB row half per instruction, slot l holds piece l ^ (row & 15); rows past
    // the end repeat the last row (their outputs are not written)
#pragma unroll 4
    for (int row = w; row < BM; row += 4) {
      const int rs = min(row, nr - 1);
      const float* src = z + ((size_t)(r0 + rs) * H + i) * DC + kh * KH + 4 * (lane ^ (row & 15));
      dma16(src, __builtin_amdgcn_readfirstlane(lds_z + row * Z_ROW));
    }
    __builtin_amdgcn_s_waitcnt(0);   // vmcnt 0: this wave's rows have landed
    __syncthreads();
    // each 16-byte piece of 4 floats becomes [hi0..hi3 | lo0..lo3] in bf16, in place (a thread
    // reads and rewrites only its own pieces): hi = bf16(z), lo = bf16(z - hi)
    for (int pc = t; pc < BM * (Z_ROW / 16); pc += 256) {
      unsigned char* at = smem + Z_OFF + pc * 16;
      const f32x4 zv = *reinterpret_cast<const f32x4*>(at);
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const bf16 h0 = (bf16)zv[2 * e], h1 = (bf16)zv[2 * e + 1];
        const bf16 l0 = (bf16)(zv[2 * e] - (float)h0), l1 = (bf16)(zv[2 * e + 1] - (float)h1);
        hw[e] = (uint32_t)__builtin_bit_cast(unsigned short, h0) | ((uint32_t)__builtin_bit_cast(unsigned short, h1) << 16);
        lw[e] = (uint32_t)__builtin_bit_cast(unsigned short, l0) | ((uint32_t)__builtin_bit_cast(unsigned short, l1) << 16);
      }
      *reinterpret_cast<i32x4*>(at) = i32x4{(int)hw[0], (int)hw[1], (int)lw[0], (int)lw[1]};
    }
    __syncthreads();

    const int v = 32 * ob + l32;   // local W_UV row (output v0 + v)
#pragma unroll 2
    for (int s = 0; s < KH / 16; ++s) {
      // B: W_UV[i][v0 + v][16s + 8g .. +7] = logical piece 2s + g of local row v
      const bf16x8e b = *reinterpret_cast<const bf16x8e*>(smem + v * WV_ROW + 16 * ((2 * s + g) ^ (v & 15)));
#pragma unroll
      for (int k = 0; k < RBW; ++k) {
        // A: z[m][16s + 8g .. +7] = logical float pieces 2(2s + g) and 2(2s + g) + 1 of row m
        const int m = 32 * (rb0 + k) + l32;
        const int p0 = 2 * (2 * s + g);
        const unsigned char* q0 = smem + Z_OFF + m * Z_ROW + 16 * (p0 ^ (m & 15));
        const unsigned char* q1 = smem + Z_OFF + m * Z_ROW + 16 * ((p0 + 1) ^ (m & 15));
        typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
        const i32x2 h0 = *reinterpret_cast<const i32x2*>(q0), h1 = *reinterpret_cast<const i32x2*>(q1);
        const i32x2 l0 = *reinterpret_cast<const i32x2*>(q0 + 8), l1 = *reinterpret_cast<const i32x2*>(q1 + 8);
        const i32x2 hh[2] = {h0, h1}, ll[2] = {l0, l1};
        acc[k] = mfma(__builtin_bit_cast(bf16x8e, hh), b, acc[k]);
        acc[k] = mfma(__builtin_bit_cast(bf16x8e, ll), b, acc[k]);
      }
    }
  }
  // D layout: lane holds output v0 + 32 ob + l32 of rows 32 (rb0 + k) + 8j + 4g + e
#pragma unroll
  for (int k = 0; k < RBW; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 32 * (rb0 + k) + 8 * j + 4 * g + e;
        if (row < nr) o[((size_t)(r0 + row) * H + i) * DN + v0 + 32 * ob + l32] = (bf16)acc[k][4 * j + e];
      }
}

}  // namespace gemm

hipError_t launch_absorb_q_gemm(const LayerDims& L, int n_rows, const void* q_nope, const void* q_rope,
                                const int32_t* q_pos, const void* w_uk, void* q_packed, hipStream_t stream) {
  static std::atomic<uint32_t> lds_set{0};
  {
    const hipError_t e = ensure_lds_limit(lds_set, {{(const void*)gemm::absorb_q_gemm, gemm::ABSORB_LDS}});
    if (e != hipSuccess) return e;
  }
  // the quarters of a row tile, then the row tiles of one head, run together
  const dim3 grid(4, (n_rows + gemm::BM - 1) / gemm::BM, gemm::H);
  hipLaunchKernelGGL(gemm::absorb_q_gemm, grid, dim3(256), gemm::ABSORB_LDS, stream, (const bf16*)q_nope,
                     (const bf16*)q_rope, q_pos, (const bf16*)w_uk, (bf16*)q_packed, n_rows, L.rope_base);
  return hipGetLastError();
}

hipError_t launch_out_proj_gemm(const LayerDims& L, int n_rows, const float* z, const void* w_uv, void* o,
                                hipStream_t stream) {
  (void)L;
  static std::atomic<uint32_t> lds_set{0};
  {
    const hipError_t e = ensure_lds_limit(lds_set, {{(const void*)gemm::out_proj_gemm<128>, gemm::outp_lds<128>()},
                                                    {(const void*)gemm::out_proj_gemm<64>, gemm::outp_lds<64>()}});
    if (e != hipSuccess) return e;
  }
  // row tiles (and output halves) of one head run together
  const int tiles = (n_rows + gemm::BM - 1) / gemm::BM;
  if (tiles == 1)
    hipLaunchKernelGGL(gemm::out_proj_gemm<64>, dim3(1, gemm::H, 2), dim3(256), gemm::outp_lds<64>(), stream, z,
                       (const bf16*)w_uv, (bf16*)o, n_rows);
  else
    hipLaunchKernelGGL(gemm::out_proj_gemm<128>, dim3(tiles, gemm::H), dim3(256), gemm::outp_lds<128>(), stream, z,
                       (const bf16*)w_uv, (bf16*)o, n_rows);
  return hipGetLastError();
}

}  // namespace mla
