// Optional output projection u = W_O concat_i(o_i) ("Decoupled RoPE · MLA Part 2", §5 step 5 and
// the output line of the forward pass in §7; "从零理解 MLA", section "矩阵吸收", last step).
//
// The heads' outputs o [n_rows, H, d_v], as stored by mla_out_proj, are read back as one row of
// K = H * d_v values per query row (head-major: element i * d_v + v is o[r, i, v]) and multiplied
// by W_O [d_model, K] (the weight of nn.Linear(K, d_model)); fp32 accumulation, one rounding to
// the storage dtype.
//   * wo_generic: any shape and dtype; one wave per output, lanes split K.
//   * wo_gemv (bf16, K = 16384, few rows): W_O is streamed from HBM once per block of 4 query
//     rows, whose o rows sit in LDS; a wave owns 8 rows of W_O, two at a time, 16 independent
//     16-byte loads per lane in flight.
//   * wo_gemm (bf16, K = 16384, many rows): MFMA 32x32x16 tiles, 128 x 128 outputs per workgroup,
//     both operands K-contiguous (o rows and W_O rows), staged through padded LDS rows.
#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace wo {

constexpr int KW = 128 * 128;   // H * d_v of the DeepSeek-V2/V3 shape

// ---------------------------------------------------------------- generic
// grid (ceil(d_model / 4), min(n_rows, 65535)), 256 threads: wave w computes u[r, 4 blockIdx.x + w]
// for rows r = blockIdx.y, blockIdx.y + gridDim.y, ...
template <typename T>
__global__ void __launch_bounds__(256) wo_generic(const T* __restrict__ o, const T* __restrict__ w_o,
                                                  T* __restrict__ u, int n_rows, int K, int d_model) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = blockIdx.x * 4 + w;
  if (n >= d_model) return;
  const T* wrow = w_o + (size_t)n * K;
  for (int r = blockIdx.y; r < n_rows; r += gridDim.y) {
    const T* orow = o + (size_t)r * K;
    float s = 0.0f;
    for (int k = lane; k < K; k += 64) s = fmaf(to_f32(wrow[k]), to_f32(orow[k]), s);
    s = warp_sum(s);
    if (lane == 0) u[(size_t)r * d_model + n] = from_f32<T>(s);
  }
}

__device__ __forceinline__ void unpack8(const i32x4 v, float* f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t x = (uint32_t)v[e];
    f[2 * e] = __uint_as_float(x << 16);
    f[2 * e + 1] = __uint_as_float(x & 0xFFFF0000u);
  }
}

// ---------------------------------------------------------------- few rows
constexpr int kRB = 4;              // query rows per pass (their o rows: 4 x 32 KB of LDS)
constexpr int kRowsPerWave = 8;     // W_O rows per wave
constexpr int GEMV_LDS = kRB * KW * 2;

// grid (ceil(d_model / 32), ceil(n_rows / kRB)), 256 threads, GEMV_LDS dynamic LDS
__global__ void __launch_bounds__(256) wo_gemv(const bf16* __restrict__ o, const bf16* __restrict__ w_o,
                                               bf16* __restrict__ u, int n_rows, int d_model) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int r0 = blockIdx.y * kRB, nr = min(kRB, n_rows - r0);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // stage the block's o rows (rows past the end as zeros)
  for (int e = threadIdx.x; e < kRB * KW / 8; e += 256) {
    const int rr = e / (KW / 8), c = e % (KW / 8);
    i32x4 v = {0, 0, 0, 0};
    if (rr < nr) v = *reinterpret_cast<const i32x4*>(o + (size_t)(r0 + rr) * KW + 8 * c);
    *reinterpret_cast<i32x4*>(smem + ((size_t)rr * KW + 8 * c) * 2) = v;
  }
  __syncthreads();
  const int nbase = blockIdx.x * 32 + w * kRowsPerWave;
#pragma unroll 1
  for (int p = 0; p < kRowsPerWave; p += 2) {
    float acc[2][kRB];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int rr = 0; rr < kRB; ++rr) acc[q][rr] = 0.0f;
    // lane covers K positions 8 lane + 512 j (j = 0..31), 8 chunks per step
#pragma unroll 1
    for (int jb = 0; jb < 32; jb += 8) {
      i32x4 wv[2][8];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int n = nbase + p + q;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          wv[q][j] = n < d_model ? __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(
                                       w_o + (size_t)n * KW + 8 * lane + 512 * (jb + j)))
                                 : i32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float wf[2][8];
        unpack8(wv[0][j], wf[0]);
        unpack8(wv[1][j], wf[1]);
#pragma unroll
        for (int rr = 0; rr < kRB; ++rr) {
          const i32x4 ov = *reinterpret_cast<const i32x4*>(smem + ((size_t)rr * KW + 8 * lane + 512 * (jb + j)) * 2);
          float of[8];
          unpack8(ov, of);
#pragma unroll
          for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][rr] = fmaf(wf[q][e], of[e], acc[q][rr]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int rr = 0; rr < kRB; ++rr) {
        const float s = warp_sum(acc[q][rr]);
        const int n = nbase + p + q;
        if (lane == 0 && rr < nr && n < d_model) u[(size_t)(r0 + rr) * d_model + n] = (bf16)s;
      }
  }
}

// ---------------------------------------------------------------- many rows
typedef __bf16 bf16x8e __attribute__((ext_vector_type(8)));
typedef float f32x16e __attribute__((ext_vector_type(16)));

constexpr int TM = 128, TN = 128, TK = 32;
constexpr int SROW = TK + 8;   // bf16 per staged row (80 bytes: 16 lanes of a 16-byte read hit 16 bank groups)
constexpr int GEMM_LDS = 2 * 2 * TM * SROW * 2;   // two buffers of the A and B tiles

// grid (ceil(d_model / 128), ceil(n_rows / 128)), 256 threads, GEMM_LDS dynamic LDS.
// Wave w computes rows 64 (w / 2) .. +63 and columns 64 (w % 2) .. +63 of the tile: 2 x 2 MFMA
// blocks of 32 x 32. Per K step of 32, every thread moves 2 x 16 bytes of A (o rows) and of B
// (W_O rows) global -> registers -> LDS; the next step's loads are in flight during the MFMAs.
__global__ void __launch_bounds__(256) wo_gemm(const bf16* __restrict__ o, const bf16* __restrict__ w_o,
                                               bf16* __restrict__ u, int n_rows, int d_model) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16* As = reinterpret_cast<bf16*>(smem);                 // [2][TM][SROW]
  bf16* Bs = As + 2 * TM * SROW;                            // [2][TN][SROW]
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  // loader: thread t moves rows t / 4 and 64 + t / 4, 16-byte piece t % 4 of each K step
  const int lr = t >> 2, lc = (t & 3) * 8;
  const bf16* ga[2];
  const bf16* gb[2];
  bool va[2], vb[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int ra = m0 + lr + 64 * h, rb = n0 + lr + 64 * h;
    va[h] = ra < n_rows;
    vb[h] = rb < d_model;
    ga[h] = o + (size_t)(va[h] ? ra : 0) * KW + lc;
    gb[h] = w_o + (size_t)(vb[h] ? rb : 0) * KW + lc;
  }
  i32x4 ra_[2], rb_[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      ra_[h] = va[h] ? *reinterpret_cast<const i32x4*>(ga[h] + k0) : i32x4{0, 0, 0, 0};
      rb_[h] = vb[h] ? *reinterpret_cast<const i32x4*>(gb[h] + k0) : i32x4{0, 0, 0, 0};   // reused by every row tile
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<i32x4*>(As + ((size_t)buf * TM + lr + 64 * h) * SROW + lc) = ra_[h];
      *reinterpret_cast<i32x4*>(Bs + ((size_t)buf * TN + lr + 64 * h) * SROW + lc) = rb_[h];
    }
  };
  f32x16e acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16e{};
  const int wm = 64 * (w >> 1), wn = 64 * (w & 1);
  gload(0);
  lstore(0);
  __syncthreads();
  constexpr int NK = KW / TK;
  for (int kt = 0; kt < NK; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < NK) gload((kt + 1) * TK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8e af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8e*>(As + ((size_t)buf * TM + wm + 32 * i + l32) * SROW + 16 * ks + 8 * g);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8e*>(Bs + ((size_t)buf * TN + wn + 32 * j + l32) * SROW + 16 * ks + 8 * g);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < NK) {
      lstore(buf ^ 1);   // the other buffer was last read before the previous barrier
      __syncthreads();
    }
  }
  // D block (i, j): lane holds column n = l32, rows 8 q + 4 g + e (register 4 q + e)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 32 * j + l32;
      if (n >= d_model) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = m0 + wm + 32 * i + 8 * q + 4 * g + e;
          if (m < n_rows) u[(size_t)m * d_model + n] = (bf16)acc[i][j][4 * q + e];
        }
    }
}

}  // namespace wo

template <typename T>
hipError_t launch_w_o_generic(int n_rows, int K, int d_model, const void* o, const void* w_o, void* u,
                              hipStream_t stream) {
  hipLaunchKernelGGL(wo::wo_generic<T>, dim3((d_model + 3) / 4, n_rows < 65535 ? n_rows : 65535), dim3(256), 0,
                     stream, (const T*)o, (const T*)w_o, (T*)u, n_rows, K, d_model);
  return hipGetLastError();
}
template hipError_t launch_w_o_generic<float>(int, int, int, const void*, const void*, void*, hipStream_t);
template hipError_t launch_w_o_generic<__bf16>(int, int, int, const void*, const void*, void*, hipStream_t);

bool w_o_fast_supported(int K) { return K == wo::KW; }

hipError_t launch_w_o_fast(int n_rows, int d_model, const void* o, const void* w_o, void* u, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)wo::wo_gemv, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       wo::GEMV_LDS);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)wo::wo_gemm, hipFuncAttributeMaxDynamicSharedMemorySize, wo::GEMM_LDS);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (n_rows < kGemmMinRows)
    hipLaunchKernelGGL(wo::wo_gemv, dim3((d_model + 31) / 32, (n_rows + wo::kRB - 1) / wo::kRB), dim3(256),
                       wo::GEMV_LDS, stream, (const bf16*)o, (const bf16*)w_o, (bf16*)u, n_rows, d_model);
  else
    hipLaunchKernelGGL(wo::wo_gemm, dim3((d_model + wo::TN - 1) / wo::TN, (n_rows + wo::TM - 1) / wo::TM),
                       dim3(256), wo::GEMM_LDS, stream, (const bf16*)o, (const bf16*)w_o, (bf16*)u, n_rows, d_model);
  return hipGetLastError();
}

}  // namespace mla
