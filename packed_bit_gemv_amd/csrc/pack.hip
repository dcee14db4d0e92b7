// pack_ternary: int8 codes -> 2-bit words, row sums and code counts.
// Load-time step; the per-row scale and row sum are the row metadata of the
// Neutrino-1 8B model page ("Where the bytes live"), the counts its code
// occupancy ("Inside the coded lane").
#include "pbg_device.hpp"
#include "pbg_internal.hpp"

namespace pbg {
namespace {

constexpr int kPackWaves = 4;         // waves per workgroup
constexpr int kPackMaxBlocks = 4096;  // the grid stays far below the launch limits at any n

// Nonzero and sign bit of code j (0..15) in its word.
__device__ __forceinline__ uint32_t nz_bit(int j) { return 16u * (j & 1) + 14u - 2u * (j >> 1); }
__device__ __forceinline__ uint32_t sign_bit(int j) { return nz_bit(j) + 1u; }

struct Tally {
  int minus, zero, plus, invalid;
};

__device__ __forceinline__ void put_code(int c, int j, uint32_t& word, int& sum, Tally& t) {
  if (c == 1) {
    word |= 1u << nz_bit(j);
    sum += 1;
    t.plus += 1;
  } else if (c == -1) {
    word |= (1u << nz_bit(j)) | (1u << sign_bit(j));
    sum -= 1;
    t.minus += 1;
  } else if (c == 0) {
    t.zero += 1;
  } else {
    t.invalid += 1;
  }
}

__global__ void zero_stats_kernel(int64_t* stats) {
  if (threadIdx.x < 4) stats[threadIdx.x] = 0;
}

// One wave per row at a time (rows wave, wave + all waves, ...); lane l packs
// words l, l + 64, ... of the row. The row sum is reduced across the wave;
// the code counts are kept per lane over all rows of the wave, reduced per
// workgroup and added to the totals with one 64-bit atomic each (integers:
// the order of additions does not matter).
__global__ __launch_bounds__(kPackWaves* kWave) void pack_kernel(const int8_t* __restrict__ codes, int64_t n,
                                                                 int64_t k, int64_t words,
                                                                 uint32_t* __restrict__ packed,
                                                                 int32_t* __restrict__ row_sum,
                                                                 int64_t* __restrict__ stats) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const bool vec = (k % 16 == 0) && ((reinterpret_cast<uintptr_t>(codes) & 15u) == 0);
  Tally t = {0, 0, 0, 0};
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kPackWaves;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kPackWaves + wave; row < n; row += stride) {
    const int8_t* src = codes + row * k;
    int sum = 0;
    for (int64_t w = lane; w < words; w += kWave) {
      uint32_t word = 0;
      const int64_t c0 = 16 * w;
      if (c0 < k) {
        if (vec) {
          const uint4 v = *reinterpret_cast<const uint4*>(src + c0);
          const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 16; ++j) put_code(static_cast<int8_t>(q[j >> 2] >> (8 * (j & 3))), j, word, sum, t);
        } else {
          for (int j = 0; j < 16 && c0 + j < k; ++j) put_code(src[c0 + j], j, word, sum, t);
        }
      }
      packed[row * words + w] = word;
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) row_sum[row] = sum;
  }
  __shared__ int red[4][kPackWaves];
  int vals[4] = {t.minus, t.zero, t.plus, t.invalid};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int v = vals[i];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) red[i][wave] = v;
  }
  __syncthreads();
  if (threadIdx.x < 4) {
    int64_t tot = 0;
    for (int wv = 0; wv < kPackWaves; ++wv) tot += red[threadIdx.x][wv];
    if (tot) atomicAdd(reinterpret_cast<unsigned long long*>(stats + threadIdx.x), static_cast<unsigned long long>(tot));
  }
}

}  // namespace

hipError_t launch_pack(const int8_t* codes, int64_t n, int64_t k, uint32_t* packed, int32_t* row_sum,
                       int64_t* stats, hipStream_t stream) {
  const int64_t words = words_per_row(k);
  hipLaunchKernelGGL(zero_stats_kernel, dim3(1), dim3(64), 0, stream, stats);
  const int64_t blocks = (n + kPackWaves - 1) / kPackWaves;
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(blocks < kPackMaxBlocks ? blocks : kPackMaxBlocks)),
                     dim3(kPackWaves * kWave), 0, stream, codes, n, k, words, packed, row_sum, stats);
  return hipGetLastError();
}

}  // namespace pbg
