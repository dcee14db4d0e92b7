// ternary_gemv (M = 1) and ternary_gemm_small (M <= 8) for gfx950.
//
// y_r = s_r * sum_j c_rj * x_j with the codes decoded in registers from the
// packed words (Neutrino-1 8B model page: codes decoded inside the matrix
// kernels, introduction; per-row scale, "Where the bytes live"; a drafted run
// scored in one forward pass, "speculative").
//
// Work split: a wave owns 4 consecutive rows. Lane l streams 16-byte chunks
// l, l+64, ... of each row (one wave-wide 1 KiB load per row per 4,096
// columns), keeps the matching 64 activations in registers as fp16 pairs and
// accumulates fp32 partial sums with v_dot2. The four row sums are finished
// by one transposed cross-lane reduction.
#include "pbg_device.hpp"
#include "pbg_internal.hpp"

namespace pbg {
namespace {

constexpr int kRowsPerWave = 4;
constexpr int kGemvWaves = 4;

// Sum over one 16-byte chunk (4 words, 64 codes) against 32 activation pairs.
__device__ __forceinline__ float chunk_dot(const uint4& w, const uint32_t* xp, float acc) {
  float a0 = word_dot(w.x, xp + 0, 0.0f);
  float a1 = word_dot(w.y, xp + 8, 0.0f);
  float a2 = word_dot(w.z, xp + 16, 0.0f);
  float a3 = word_dot(w.w, xp + 24, 0.0f);
  return acc + ((a0 + a1) + (a2 + a3));
}

__global__ __launch_bounds__(kGemvWaves* kWave) void ternary_gemv_kernel(const uint4* __restrict__ packed,
                                                                          const float* __restrict__ scale,
                                                                          int64_t n, int64_t k, int64_t chunks,
                                                                          const uint16_t* __restrict__ x,
                                                                          float* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * kGemvWaves + (threadIdx.x / kWave)) * kRowsPerWave;
  if (row0 >= n) return;  // whole wave leaves together
  float acc[kRowsPerWave] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t c = lane; c < chunks; c += kWave) {
    uint32_t xp[32];
    load_x_pairs<32>(x, k, 64 * c, xp);
    uint4 w[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
      w[i] = (row0 + i < n) ? packed[(row0 + i) * chunks + c] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) acc[i] = chunk_dot(w[i], xp, acc[i]);
  }
  const float r = wave_reduce4(acc[0], acc[1], acc[2], acc[3]);
  const int slot = reduce4_slot(lane);
  if (slot >= 0 && row0 + slot < n) y[row0 + slot] = r * (scale[row0 + slot] * kCodeUnitInv);
}

// Small M: lane l handles words l, l+64, ... of each row (16 codes each) so
// that M rows of 16 activations fit in registers; every decoded code pair is
// used for all M activation rows.
template <int M>
__global__ __launch_bounds__(kGemvWaves* kWave) void ternary_gemm_small_kernel(const uint32_t* __restrict__ packed,
                                                                                const float* __restrict__ scale,
                                                                                int64_t n, int64_t k, int64_t words,
                                                                                const uint16_t* __restrict__ x,
                                                                                float* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * kGemvWaves + (threadIdx.x / kWave)) * kRowsPerWave;
  if (row0 >= n) return;
  float acc[kRowsPerWave][M];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.0f;
  for (int64_t w = lane; w < words; w += kWave) {
    uint32_t xp[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m) load_x_pairs<8>(x + m * k, k, 16 * w, xp[m]);
    uint32_t wd[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) wd[i] = (row0 + i < n) ? packed[(row0 + i) * words + w] : 0u;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t cp = code_pair(wd[i], t);
#pragma unroll
        for (int m = 0; m < M; ++m) acc[i][m] = dot2(cp, xp[m][t], acc[i][m]);
      }
    }
  }
  const int slot = reduce4_slot(lane);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float r = wave_reduce4(acc[0][m], acc[1][m], acc[2][m], acc[3][m]);
    if (slot >= 0 && row0 + slot < n) y[m * n + row0 + slot] = r * (scale[row0 + slot] * kCodeUnitInv);
  }
}

template <int M>
void launch_small(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                  hipStream_t stream) {
  const int64_t rows_per_block = kGemvWaves * kRowsPerWave;
  const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL(ternary_gemm_small_kernel<M>, grid, dim3(kGemvWaves * kWave), 0, stream, packed, scale, n, k,
                     words_per_row(k), x, y);
}

}  // namespace

hipError_t launch_ternary_gemv(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                               const uint16_t* x, float* y, hipStream_t stream) {
  const int64_t rows_per_block = kGemvWaves * kRowsPerWave;
  const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL(ternary_gemv_kernel, grid, dim3(kGemvWaves * kWave), 0, stream,
                     reinterpret_cast<const uint4*>(packed), scale, n, k, words_per_row(k) / 4, x, y);
  return hipGetLastError();
}

hipError_t launch_ternary_gemm_small(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                                     const uint16_t* x, int m, float* y, hipStream_t stream) {
  switch (m) {
    case 1: launch_small<1>(packed, scale, n, k, x, y, stream); break;
    case 2: launch_small<2>(packed, scale, n, k, x, y, stream); break;
    case 3: launch_small<3>(packed, scale, n, k, x, y, stream); break;
    case 4: launch_small<4>(packed, scale, n, k, x, y, stream); break;
    case 5: launch_small<5>(packed, scale, n, k, x, y, stream); break;
    case 6: launch_small<6>(packed, scale, n, k, x, y, stream); break;
    case 7: launch_small<7>(packed, scale, n, k, x, y, stream); break;
    case 8: launch_small<8>(packed, scale, n, k, x, y, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pbg
