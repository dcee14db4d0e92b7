// pack_ternary: int8 codes -> 2-bit words, row sums and code counts.
// Load-time step; the per-row scale and row sum are the row metadata of the
// Neutrino-1 8B model page ("Where the bytes live"), the counts its code
// occupancy ("Inside the coded lane").
#include "pbg_device.hpp"
#include "pbg_internal.hpp"

namespace pbg {
namespace {

// At most 256 workgroups of 16 waves: each workgroup ends with one 64-bit
// atomic per nonzero code count, and atomics on the four counts (one cache
// line) serialise at the memory side, so the grid is kept small; 16 waves per
// CU still keep 64 KiB of codes in flight.
constexpr int kPackWaves = 16;        // waves per workgroup
constexpr int kPackMaxBlocks = 256;
constexpr int kPackBatch = 4;         // words per lane whose loads are in flight together

// Nonzero bit of code j (0..15) in its word; the sign bit is the next one up.
__device__ __forceinline__ uint32_t nz_bit(int j) { return 16u * (j & 1) + 14u - 2u * (j >> 1); }

struct Tally {
  int minus, zero, plus, invalid;
};

// Field of one code byte: a valid code (0x00, 0x01 or 0xFF as a byte) is its
// own 2-bit two's complement, b & 3; anything else packs as 0 and is counted.
__device__ __forceinline__ void put_code(uint32_t b, int j, uint32_t& word, int& bad) {
  const bool ok = ((b + 1u) & 0xFFu) <= 2u;
  bad += ok ? 0 : 1;
  word |= (ok ? (b & 3u) : 0u) << nz_bit(j);
}

// The fields of code bytes 4q .. 4q + 3 (bytes 0..3 of u) at their places in
// the word, four bytes at a time:
//  - t = b + 1 (mod 256) per byte, without carries between bytes; a valid code
//    gives t <= 2;
//  - bit 7 of a byte of `inv` is set when t >= 3, an invalid code;
//  - f holds b & 3 of every valid byte and 0 for the invalid ones;
//  - a byte permute puts codes 4q + 2 and 4q (the low half's two fields) 8 bits
//    apart in the low half and codes 4q + 3 and 4q + 1 in the high half, and a
//    shift by 6 closes each gap, leaving the fields of pair 2q + 1 below those
//    of pair 2q; the final shift moves pair 2q to bits 14 - 4q (low half) and
//    30 - 4q (high half).
__device__ __forceinline__ uint32_t pack4(uint32_t u, int q, int& bad) {
  const uint32_t t = ((u & 0x7F7F7F7Fu) + 0x01010101u) ^ (u & 0x80808080u);
  const uint32_t inv = (((t & 0x7F7F7F7Fu) + 0x7D7D7D7Du) | t) & 0x80808080u;
  bad += __popc(inv);
  const uint32_t f = u & 0x03030303u & ~((inv >> 6) | (inv >> 7));
  const uint32_t g = __builtin_amdgcn_perm(f, f, 0x01030002u);  // bytes (2, 0, 3, 1) of f
  const uint32_t h = (g | (g >> 6)) & 0x000F000Fu;
  return h << (12 - 4 * q);
}

// Packs the 16 code bytes of v into one word.
__device__ __forceinline__ uint32_t pack16(const uint4& v, int& bad) {
  return pack4(v.x, 0, bad) | pack4(v.y, 1, bad) | pack4(v.z, 2, bad) | pack4(v.w, 3, bad);
}

// Counts of a packed word holding `codes` codes, `bad` of them invalid (and
// packed as 0): its nonzero bits mark +1 and -1, its sign bits -1.
__device__ __forceinline__ void tally(uint32_t word, int codes, int bad, int& sum, Tally& t) {
  const int nz = __popc(word & 0x55555555u);
  const int minus = __popc(word & 0xAAAAAAAAu);
  t.plus += nz - minus;
  t.minus += minus;
  t.zero += codes - bad - nz;
  t.invalid += bad;
  sum += nz - 2 * minus;
}

__global__ void zero_stats_kernel(int64_t* stats) {
  if (threadIdx.x < 4) stats[threadIdx.x] = 0;
}

// One wave per row at a time (rows wave, wave + all waves, ...); lane l packs
// words l, l + 64, ... of the row, with the loads of kPackBatch words in
// flight together when the row is whole 16-byte chunks. The row sum is
// reduced across the wave; the code counts are kept per lane over all rows of
// the wave, reduced per workgroup and added to the totals with one 64-bit
// atomic each (integers: the order of additions does not matter).
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
    uint32_t* dst = packed + row * words;
    int sum = 0;
    if (vec) {
      const int64_t full = k / 16;  // words that hold codes; the rest is padding
      for (int64_t w0 = 0; w0 < words; w0 += kWave * kPackBatch) {
        uint4 v[kPackBatch];
#pragma unroll
        for (int u = 0; u < kPackBatch; ++u) {
          const int64_t w = w0 + lane + u * kWave;
          v[u] = w < full ? *reinterpret_cast<const uint4*>(src + 16 * w) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kPackBatch; ++u) {
          const int64_t w = w0 + lane + u * kWave;
          if (w < words) {
            int bad = 0;
            const uint32_t word = pack16(v[u], bad);
            if (w < full) tally(word, 16, bad, sum, t);
            dst[w] = word;
          }
        }
      }
    } else {
      for (int64_t w = lane; w < words; w += kWave) {
        const int64_t c0 = 16 * w;
        const int codes_here = c0 < k ? static_cast<int>(k - c0 < 16 ? k - c0 : 16) : 0;
        uint32_t word = 0;
        int bad = 0;
        for (int j = 0; j < codes_here; ++j) put_code(static_cast<uint8_t>(src[c0 + j]), j, word, bad);
        tally(word, codes_here, bad, sum, t);
        dst[w] = word;
      }
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
