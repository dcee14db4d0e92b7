// int8_head_gemv: Y[i][v] = s_v * sum_j w_vj * X[i][j] for the untied int8
// output head with a per-row scale (Neutrino-1 8B model page, "Where the
// bytes live"), for 1..8 activation rows.
//
// Each lane streams 16-byte chunks (16 weights) of 4 rows. A weight byte b is
// turned into the fp16 value b exactly: the byte, biased to b + 128, becomes
// the low mantissa byte of fp16 0x64xx = 1024 + (b + 128), and one packed fp16
// subtraction of 1152 leaves b. v_dot2 then accumulates w * x in fp32.
#include <atomic>

#include "packed_bit_gemv.h"
#include "pbg_device.hpp"
#include "pbg_internal.hpp"

namespace pbg {
namespace {

constexpr int kHeadRows = 4;
constexpr int kHeadWaves = 4;

// Greedy-argmax keys of one activation row are spread over kArgmaxBins bins
// on separate 128-byte lines (workgroup b uses bin b % kArgmaxBins): device
// atomics on one address serialise at the memory side (about 10 ns each), so
// ten thousand workgroups on one key would take as long as the head itself.
// The bins are zero between calls: the caller zeroes the workspace once and
// the finishing kernel clears every bin it has read.
constexpr int kArgmaxBins = 256;
constexpr int kArgmaxStride = 16;  // keys between bins (128 bytes)
static_assert(kArgmaxBins * kArgmaxStride == PBG_ARGMAX_KEYS_PER_ROW, "workspace layout");

__device__ __forceinline__ unsigned long long* argmax_bin(unsigned long long* keys, int row) {
  return keys + (static_cast<int64_t>(row) * kArgmaxBins + blockIdx.x % kArgmaxBins) * kArgmaxStride;
}

// Four int8 weights (one dword) -> two fp16 pairs (w0, w1), (w2, w3).
__device__ __forceinline__ void int8x4_to_half2x2(uint32_t v, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = v ^ 0x80808080u;  // b + 128 as an unsigned byte
  const half2_t bias = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
  // v_perm_b32: selector bytes 0..3 pick bytes of u, 4 picks a 0x64 byte.
  const half2_t l = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) - bias;
  const half2_t h = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) - bias;
  lo = __builtin_bit_cast(uint32_t, l);
  hi = __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint4 load_w_chunk(const int8_t* __restrict__ row, int64_t k, int64_t c0, bool vec) {
  if (vec) return *reinterpret_cast<const uint4*>(row + c0);
  uint32_t q[4] = {0u, 0u, 0u, 0u};
  for (int j = 0; j < 16; ++j)
    if (c0 + j < k) q[j >> 2] |= static_cast<uint32_t>(static_cast<uint8_t>(row[c0 + j])) << (8 * (j & 3));
  return make_uint4(q[0], q[1], q[2], q[3]);
}

template <int M, bool AM>
__global__ __launch_bounds__(kHeadWaves* kWave) void int8_head_kernel(const int8_t* __restrict__ w,
                                                                       const float* __restrict__ scale, int64_t n,
                                                                       int64_t k, const uint16_t* __restrict__ x,
                                                                       float* __restrict__ y,
                                                                       unsigned long long* __restrict__ keys) {
  __shared__ unsigned long long wg_key[AM ? M : 1];
  if constexpr (AM) {
    if (threadIdx.x < M) wg_key[threadIdx.x] = 0ull;
    __syncthreads();
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * kHeadWaves + (threadIdx.x / kWave)) * kHeadRows;
  const int64_t chunks = (k + 15) / 16;
  const bool vec = (k % 16 == 0);
  float acc[kHeadRows][M];
#pragma unroll
  for (int i = 0; i < kHeadRows; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.0f;
  if (row0 < n) {  // wave-uniform
    for (int64_t c = lane; c < chunks; c += kWave) {
      uint32_t xp[M][8];
#pragma unroll
      for (int m = 0; m < M; ++m) load_x_pairs<8>(x + m * k, k, 16 * c, xp[m]);
      uint4 wv[kHeadRows];
#pragma unroll
      for (int i = 0; i < kHeadRows; ++i)
        wv[i] = (row0 + i < n) ? load_w_chunk(w + (row0 + i) * k, k, 16 * c, vec) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int i = 0; i < kHeadRows; ++i) {
        uint32_t hp[8];
        int8x4_to_half2x2(wv[i].x, hp[0], hp[1]);
        int8x4_to_half2x2(wv[i].y, hp[2], hp[3]);
        int8x4_to_half2x2(wv[i].z, hp[4], hp[5]);
        int8x4_to_half2x2(wv[i].w, hp[6], hp[7]);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float a = acc[i][m];
#pragma unroll
          for (int p = 0; p < 8; ++p) a = dot2(hp[p], xp[m][p], a);
          acc[i][m] = a;
        }
      }
    }
  }
  const int slot = reduce4_slot(lane);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float r = wave_reduce4(acc[0][m], acc[1][m], acc[2][m], acc[3][m]);
    if (slot >= 0 && row0 + slot < n) {
      const float v = r * scale[row0 + slot];
      if constexpr (AM) atomicMax(&wg_key[m], argmax_key(v, row0 + slot));
      else y[m * n + row0 + slot] = v;
    }
  }
  if constexpr (AM) {
    __syncthreads();
    if (threadIdx.x < M) atomicMax(argmax_bin(keys, threadIdx.x), wg_key[threadIdx.x]);
  }
}

template <int M, bool AM>
void launch_head_m(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                   unsigned long long* keys, hipStream_t stream) {
  const int64_t rows_per_block = kHeadWaves * kHeadRows;
  const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL((int8_head_kernel<M, AM>), grid, dim3(kHeadWaves * kWave), 0, stream, w, scale, n, k, x, y, keys);
}

// Fast path (k % 16 == 0, w and x 16-byte aligned). A workgroup holds G row
// groups x SW K-slices of 1,024 columns; wave (g, s) owns R rows and lane l
// the 16 weights s*1024 + 16*l .. +15 of each of them (slices past SW loop).
// The lane's 16 activations of every row of X stay in registers; all R row
// loads are issued (non-temporal, rows past n clamped) before the first
// conversion, and the row scales are prefetched. Partial sums are reduced
// four at a time across the wave, then added over the SW slices in order in
// LDS.
template <int M, int SW, int G, int R, bool AM>
__global__ __launch_bounds__(SW* G* kWave) void int8_head_fast_kernel(const int8_t* __restrict__ w,
                                                                       const float* __restrict__ scale, int64_t n,
                                                                       int64_t k, const uint16_t* __restrict__ x,
                                                                       float* __restrict__ y,
                                                                       unsigned long long* __restrict__ keys) {
  __shared__ unsigned long long wg_key[AM ? M : 1];
  if constexpr (AM) {
    if (threadIdx.x < M) wg_key[threadIdx.x] = 0ull;
    __syncthreads();
  }
  constexpr int kVals = R * M;  // partial sums per lane: (row i, activation row m) at i * M + m
  constexpr int kRed = (kVals + 3) / 4;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = wave / SW, s = wave % SW;
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * G + g) * R;
  const int64_t chunks = k / 16, groups = k / 8;
  const int64_t slices = (chunks + kWave - 1) / kWave;
  const uint4* wq = reinterpret_cast<const uint4*>(w);
  const uint4* xg = reinterpret_cast<const uint4*>(x);
  const int slot = reduce4_slot(lane);

  // scales of the outputs this lane writes at the end
  float sc[kRed];
#pragma unroll
  for (int q = 0; q < kRed; ++q) {
    const int idx = 4 * q + (slot < 0 ? 0 : slot);
    const int64_t r = row0 + (idx < kVals ? idx / M : 0);
    sc[q] = scale[r < n ? r : n - 1];
  }
  float acc[4 * kRed];
#pragma unroll
  for (int i = 0; i < 4 * kRed; ++i) acc[i] = 0.0f;

  for (int64_t sl = s; sl < slices; sl += SW) {  // wave-uniform
    const int64_t c = sl * kWave + lane;
    const bool in = c < chunks;
    const int64_t cc = in ? c : chunks - 1;
    uint4 xv[M][2];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      xv[m][0] = xg[m * groups + 2 * cc];
      xv[m][1] = xg[m * groups + 2 * cc + 1];
    }
    uint4 wv[R];
#pragma unroll
    for (int i = 0; i < R; ++i) wv[i] = load_nt(wq + (row0 + i < n ? row0 + i : n - 1) * chunks + cc);
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t keep = in ? 0xFFFFFFFFu : 0u;  // activations past k read as zero
    uint32_t xp[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      xp[m][0] = xv[m][0].x & keep;
      xp[m][1] = xv[m][0].y & keep;
      xp[m][2] = xv[m][0].z & keep;
      xp[m][3] = xv[m][0].w & keep;
      xp[m][4] = xv[m][1].x & keep;
      xp[m][5] = xv[m][1].y & keep;
      xp[m][6] = xv[m][1].z & keep;
      xp[m][7] = xv[m][1].w & keep;
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      uint32_t hp[8];
      int8x4_to_half2x2(wv[i].x, hp[0], hp[1]);
      int8x4_to_half2x2(wv[i].y, hp[2], hp[3]);
      int8x4_to_half2x2(wv[i].z, hp[4], hp[5]);
      int8x4_to_half2x2(wv[i].w, hp[6], hp[7]);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
        for (int p = 0; p < 8; p += 2) {
          a0 = dot2(hp[p], xp[m][p], a0);
          a1 = dot2(hp[p + 1], xp[m][p + 1], a1);
        }
        acc[i * M + m] += a0 + a1;
      }
    }
  }
  float red[kRed];
#pragma unroll
  for (int q = 0; q < kRed; ++q) red[q] = wave_reduce4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  if constexpr (SW == 1) {
    if (slot >= 0) {
#pragma unroll
      for (int q = 0; q < kRed; ++q) {
        const int idx = 4 * q + slot;
        const int64_t r = row0 + idx / M;
        if (idx < kVals && r < n) {
          const float v = red[q] * sc[q];
          if constexpr (AM) atomicMax(&wg_key[idx % M], argmax_key(v, r));
          else y[static_cast<int64_t>(idx % M) * n + r] = v;
        }
      }
    }
  } else {
    __shared__ float part[G][SW][4 * kRed];
    if (slot >= 0) {
#pragma unroll
      for (int q = 0; q < kRed; ++q) part[g][s][4 * q + slot] = red[q];
    }
    __syncthreads();
    if (s == 0 && slot >= 0) {
#pragma unroll
      for (int q = 0; q < kRed; ++q) {
        const int idx = 4 * q + slot;
        const int64_t r = row0 + idx / M;
        if (idx < kVals && r < n) {
          float sum = part[g][0][idx];
#pragma unroll
          for (int t = 1; t < SW; ++t) sum += part[g][t][idx];
          const float v = sum * sc[q];
          if constexpr (AM) atomicMax(&wg_key[idx % M], argmax_key(v, r));
          else y[static_cast<int64_t>(idx % M) * n + r] = v;
        }
      }
    }
  }
  if constexpr (AM) {
    __syncthreads();
    if (threadIdx.x < M) atomicMax(argmax_bin(keys, threadIdx.x), wg_key[threadIdx.x]);
  }
}

template <int M, int SW, int G, int R, bool AM>
void launch_head_fast(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                      unsigned long long* keys, hipStream_t stream) {
  const int64_t rows_per_block = static_cast<int64_t>(G) * R;
  const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL((int8_head_fast_kernel<M, SW, G, R, AM>), grid, dim3(SW * G * kWave), 0, stream, w, scale, n, k,
                     x, y, keys);
}

// 2 <= M <= 8 on the matrix cores for k the persistent kernel below does not
// take (k % 16 == 0, w and x 16-byte aligned).
// v_mfma_f32_16x16x32_f16 takes a 16-row tile of weights converted to fp16
// (A) and the M activation rows as B columns (zero past M). A lane with row
// i = lane % 16 and K-group g = lane / 16 loads 16 weights per 64-column unit
// u: columns 64u + 16g .. +15; MFMA step v (0, 1) uses columns 64u + 16g + 8v
// .. +7, and the B lane (g, j) holds x_j at the same columns. SK waves split
// the units of T tiles; the next unit's loads go out before the current one
// is converted; partial tiles meet in LDS and are added in wave order.
template <int SK, int T, int UPW, bool AM>
__global__ __launch_bounds__(SK* kWave) void int8_head_mfma_kernel(const int8_t* __restrict__ w,
                                                                    const float* __restrict__ scale, int64_t n,
                                                                    int64_t k, const uint16_t* __restrict__ x, int m,
                                                                    float* __restrict__ y,
                                                                    unsigned long long* __restrict__ keys) {
  __shared__ unsigned long long wg_key[AM ? 8 : 1];
  if constexpr (AM) {
    if (threadIdx.x < 8) wg_key[threadIdx.x] = 0ull;  // ordered before use by the barrier below
  }
  typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
  typedef float float4_t __attribute__((ext_vector_type(4)));
  constexpr int kRows = 16 * T;
  __shared__ float part[SK][kRows][8];
  const int lane = threadIdx.x & (kWave - 1);
  const int s = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int li = lane & 15, lg = lane >> 4;
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * kRows;
  const int64_t chunks = k / 16, groups = k / 8;
  const uint4* wq = reinterpret_cast<const uint4*>(w);
  const uint4* xg = reinterpret_cast<const uint4*>(x);

  // Outputs (row, column) o = threadIdx.x + e * SK * 64 of the tile block,
  // row o / 8 and column o % 8; their scales are fetched now.
  constexpr int kOut = (kRows * 8 + SK * kWave - 1) / (SK * kWave);
  float sc[kOut];
#pragma unroll
  for (int e = 0; e < kOut; ++e) {
    const int o = threadIdx.x + e * SK * kWave;
    const int64_t r = row_base + (o < kRows * 8 ? o >> 3 : kRows - 1);
    sc[e] = scale[r < n ? r : n - 1];
  }

  auto load_unit = [&](int q, uint4 (&xb)[2], uint4 (&wv)[T]) {
    const int64_t u = s + static_cast<int64_t>(SK) * q;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int64_t gi = 8 * u + 2 * lg + v;
      const bool ok = li < m && gi < groups;
      xb[v] = xg[ok ? static_cast<int64_t>(li) * groups + gi : 0];
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t r = row_base + 16 * t + li;
      const int64_t c = 4 * u + lg;
      wv[t] = load_nt(wq + (r < n ? r : n - 1) * chunks + (c < chunks ? c : chunks - 1));
    }
  };

  float4_t d[T];
#pragma unroll
  for (int t = 0; t < T; ++t) d[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  uint4 xb[2][2], wv[2][T];
  load_unit(0, xb[0], wv[0]);
#pragma unroll
  for (int q = 0; q < UPW; ++q) {
    if (q + 1 < UPW) load_unit(q + 1, xb[(q + 1) & 1], wv[(q + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t u = s + static_cast<int64_t>(SK) * q;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      uint4 bx = xb[q & 1][v];
      const int64_t gi = 8 * u + 2 * lg + v;
      const uint32_t keep = (li < m && gi < groups) ? 0xFFFFFFFFu : 0u;
      bx.x &= keep;
      bx.y &= keep;
      bx.z &= keep;
      bx.w &= keep;
      const half8_t b = __builtin_bit_cast(half8_t, bx);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t w0 = v == 0 ? wv[q & 1][t].x : wv[q & 1][t].z;
        const uint32_t w1 = v == 0 ? wv[q & 1][t].y : wv[q & 1][t].w;
        uint4 ap;
        int8x4_to_half2x2(w0, ap.x, ap.y);
        int8x4_to_half2x2(w1, ap.z, ap.w);
        d[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ap), b, d[t], 0, 0, 0);
      }
    }
  }
  if (li < 8) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[s][16 * t + 4 * lg + r][li] = d[t][r];
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kOut; ++e) {
    const int o = threadIdx.x + e * SK * kWave;
    const int orow = o >> 3, ocol = o & 7;
    const int64_t r = row_base + orow;
    if (o < kRows * 8 && ocol < m && r < n) {
      float sum = part[0][orow][ocol];
#pragma unroll
      for (int w2 = 1; w2 < SK; ++w2) sum += part[w2][orow][ocol];
      const float v = sum * sc[e];
      if constexpr (AM) atomicMax(&wg_key[ocol], argmax_key(v, r));
      else y[static_cast<int64_t>(ocol) * n + r] = v;
    }
  }
  if constexpr (AM) {
    __syncthreads();
    if (threadIdx.x < m) atomicMax(argmax_bin(keys, threadIdx.x), wg_key[threadIdx.x]);
  }
}

template <int SK, int T, int UPW, bool AM>
void launch_head_mfma(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, int m, float* y,
                      unsigned long long* keys, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((n + 16 * T - 1) / (16 * T)));
  hipLaunchKernelGGL((int8_head_mfma_kernel<SK, T, UPW, AM>), grid, dim3(SK * kWave), 0, stream, w, scale, n, k, x, m,
                     y, keys);
}


// 2 <= M <= 8 with k % 1024 == 0 and k <= 4096 (w and x 16-byte aligned).
// Persistent: workgroup b converts row blocks b, b + grid, ... of kPTiles
// 16-row tiles, and x is copied into LDS once per workgroup, by direct
// global-to-LDS loads, in the order the MFMA B operand reads it: group q
// (columns 8q .. 8q + 7) of row j sits at ((2 (q / 8) + q % 2) * 4 +
// (q % 8) / 2) * M + j. Wave (tg, kq) owns tile tg and the contiguous K
// quarter kq of every row block, kPBatch 64-column units per batch, with the
// next batch (of this or the next row block) in flight while one is
// converted. The kPQuarters partial tiles meet in LDS, in a buffer that
// alternates between row blocks so that one barrier per block suffices.
constexpr int kPTiles = 2;     // 16-row tiles per row block
constexpr int kPQuarters = 4;  // K parts per tile
constexpr int kPBatch = 4;     // 64-column units per batch
constexpr int kPMaxK = 4096;
constexpr int kPWaves = kPTiles * kPQuarters;
constexpr int kPKStep = 64 * kPQuarters * kPBatch;  // k must be a multiple

__device__ __forceinline__ void load_lds16(const uint4* g, uint4* lds_base) {
  __builtin_amdgcn_global_load_lds(g, lds_base, 16, 0, 0);  // lane l writes lds_base[l]
}

template <int M, bool AM>
__global__ __launch_bounds__(kPWaves* kWave) void int8_head_persist_kernel(const int8_t* __restrict__ w,
                                                                           const float* __restrict__ scale, int64_t n,
                                                                           int64_t k, const uint16_t* __restrict__ x,
                                                                           float* __restrict__ y,
                                                                           unsigned long long* __restrict__ keys) {
  typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
  typedef float float4_t __attribute__((ext_vector_type(4)));
  constexpr int kThreads = kPWaves * kWave;
  constexpr int kRows = kPTiles * 16;
  static_assert(kRows * M <= kThreads, "one output per thread per row block");
  __shared__ uint4 xs[M * (kPMaxK / 8)];
  __shared__ float part[2][kPTiles][kPQuarters][16][M];
  __shared__ unsigned long long wg_key[AM ? M : 1];
  if constexpr (AM) {
    if (threadIdx.x < M) wg_key[threadIdx.x] = 0ull;  // ordered before use by the barrier below
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int tg = wave / kPQuarters, kq = wave % kPQuarters;
  const int li = lane & 15, lg = lane >> 4;
  const int groups = static_cast<int>(k / 8);
  const int64_t chunks = k / 16;
  const int upw = static_cast<int>(k / (64 * kPQuarters));  // units per wave and row block
  const int nb = upw / kPBatch;                              // batches per row block
  const int64_t nrb = (n + kRows - 1) / kRows;
  const int my_rb = static_cast<int>((nrb - blockIdx.x + gridDim.x - 1) / gridDim.x);
  const int total = my_rb * nb;
  const uint4* wq = reinterpret_cast<const uint4*>(w);
  const uint4* xg = reinterpret_cast<const uint4*>(x);
  const int o = threadIdx.x;  // output (row o / M, column o % M) of each row block
  auto out_row = [&](int i) { return (blockIdx.x + static_cast<int64_t>(i) * gridDim.x) * kRows + o / M; };

  auto load_batch = [&](int g, uint4 (&wv)[kPBatch]) {
    const int64_t r = (blockIdx.x + static_cast<int64_t>(g / nb) * gridDim.x) * kRows + tg * 16 + li;
    const uint4* row = wq + (r < n ? r : n - 1) * chunks;
    const int u0 = kq * upw + (g % nb) * kPBatch;
#pragma unroll
    for (int c = 0; c < kPBatch; ++c) wv[c] = row[4 * (u0 + c) + lg];
  };
  uint4 wv[2][kPBatch];
  if (total > 0) load_batch(0, wv[0]);
  if (total > 1) load_batch(1, wv[1]);
  const int64_t r0 = out_row(0);
  float sc = scale[r0 < n ? r0 : n - 1];  // scale of the next row block's output
  const int slots = M * groups;
  for (int base = wave * kWave; base < slots; base += kThreads) {
    const int s = base + lane;
    const int j = s % M, t2 = s / M, g = t2 & 3, st = t2 >> 2;
    if (s < slots) load_lds16(xg + static_cast<int64_t>(j) * groups + 8 * (st >> 1) + 2 * g + (st & 1), &xs[base]);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  float4_t d = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto convert = [&](int g, const uint4 (&wb)[kPBatch]) {
    const int u0 = kq * upw + (g % nb) * kPBatch;
#pragma unroll
    for (int c = 0; c < kPBatch; ++c) {
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        uint4 bx = make_uint4(0u, 0u, 0u, 0u);
        if (li < M) bx = xs[((2 * (u0 + c) + v) * 4 + lg) * M + li];
        uint4 ap;
        int8x4_to_half2x2(v == 0 ? wb[c].x : wb[c].z, ap.x, ap.y);
        int8x4_to_half2x2(v == 0 ? wb[c].y : wb[c].w, ap.z, ap.w);
        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ap), __builtin_bit_cast(half8_t, bx), d,
                                                   0, 0, 0);
      }
    }
  };
  auto finish = [&](int g) {  // after the last batch of row block g / nb
    const int i = g / nb, p = i & 1;
    if (li < M) {
#pragma unroll
      for (int r = 0; r < 4; ++r) part[p][tg][kq][4 * lg + r][li] = d[r];  // rows 4 lg + r of column li
    }
    d = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    __syncthreads();
    const int64_t r = out_row(i);
    if (o < kRows * M && r < n) {
      const int lr = o / M, ocol = o % M;
      float sum = part[p][lr / 16][0][lr % 16][ocol];
#pragma unroll
      for (int q = 1; q < kPQuarters; ++q) sum += part[p][lr / 16][q][lr % 16][ocol];
      const float v = sum * sc;
      if constexpr (AM) atomicMax(&wg_key[ocol], argmax_key(v, r));
      else y[static_cast<int64_t>(ocol) * n + r] = v;
    }
    const int64_t rn = out_row(i + 1);
    sc = scale[rn < n ? rn : n - 1];
  };
  for (int g = 0; g < total; g += 2) {  // total is even or the last pass has one batch
    convert(g, wv[0]);
    if (g + 2 < total) load_batch(g + 2, wv[0]);
    if (g % nb == nb - 1) finish(g);
    if (g + 1 < total) {
      convert(g + 1, wv[1]);
      if (g + 3 < total) load_batch(g + 3, wv[1]);
      if ((g + 1) % nb == nb - 1) finish(g + 1);
    }
  }
  if constexpr (AM) {
    __syncthreads();
    if (threadIdx.x < M) atomicMax(argmax_bin(keys, threadIdx.x), wg_key[threadIdx.x]);
  }
}

// 3 <= M <= 4 with k % 1024 == 0, k <= 4096 and n >= 8 (w and x 16-byte
// aligned), on the VALU. Persistent: a workgroup holds one wave per 1,024-column K-slice;
// each wave keeps its slice of the M activation rows in registers for the
// whole launch and walks row groups b, b + grid, ... of kXRows rows, with the
// next group's loads (and the scale of the value each thread finishes) in
// flight while the current group is converted, multiplied and reduced. The
// slices meet in LDS in slice order, in a buffer that alternates between
// groups, so one barrier per group suffices. With x read once per wave rather
// than once per group, the M dot2 per weight pair and the conversion stay
// within the issue budget of the 622 MB stream up to M = 4; at M = 3 and 4 this
// measured 99.8-100.7 and 102.3-103.5 us against 107.8-109.6 us for the
// persistent matrix-core kernel below, and slower from M = 5.
constexpr int kXRows = 8;
constexpr int kXSlice = 1024;

template <int M, int SW, bool AM>
__global__ __launch_bounds__(SW* kWave) void int8_head_xreg_kernel(const int8_t* __restrict__ w,
                                                                    const float* __restrict__ scale, int64_t n,
                                                                    const uint16_t* __restrict__ x,
                                                                    float* __restrict__ y,
                                                                    unsigned long long* __restrict__ keys) {
  constexpr int kVals = kXRows * M;  // (row i, activation row m) at i * M + m
  constexpr int kRed = (kVals + 3) / 4;
  static_assert(kVals % 4 == 0 && kVals <= kWave, "the first wave finishes every value");
  __shared__ float part[2][SW][4 * kRed];
  __shared__ unsigned long long wg_key[AM ? M : 1];
  if constexpr (AM) {
    if (threadIdx.x < M) wg_key[threadIdx.x] = 0ull;  // ordered before use by the first group's barrier
  }
  const int lane = threadIdx.x & (kWave - 1);
  const int s = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int slot = reduce4_slot(lane);
  constexpr int64_t chunks = SW * kXSlice / 16, groups = SW * kXSlice / 8;  // k = SW * kXSlice
  const int64_t c = static_cast<int64_t>(s) * kWave + lane;  // this lane's 16 weights of every row
  const uint4* wq = reinterpret_cast<const uint4*>(w);
  const uint4* xg = reinterpret_cast<const uint4*>(x);
  uint32_t xp[M][8];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint4 a = xg[m * groups + 2 * c], b = xg[m * groups + 2 * c + 1];
    xp[m][0] = a.x;
    xp[m][1] = a.y;
    xp[m][2] = a.z;
    xp[m][3] = a.w;
    xp[m][4] = b.x;
    xp[m][5] = b.y;
    xp[m][6] = b.z;
    xp[m][7] = b.w;
  }
  const int64_t ng = (n + kXRows - 1) / kXRows;
  const int64_t stride = gridDim.x;
  const int ti = (threadIdx.x < kVals ? threadIdx.x : 0) / M;  // row of the value this thread finishes
  // Group g covers rows g * kXRows .. + kXRows - 1; the last group is read as
  // the final kXRows rows of the head (n >= kXRows), so no row needs a clamp,
  // and it stores only the rows not stored by the group before it.
  auto first_row = [&](int64_t g) {
    const int64_t r0 = g * kXRows;
    return r0 < n - kXRows ? r0 : n - kXRows;
  };
  auto load = [&](int64_t g, uint4 (&wv)[kXRows], float& scl) {
    const int64_t rs = first_row(g < ng ? g : ng - 1);
    const uint4* base = wq + rs * chunks + c;
#pragma unroll
    for (int i = 0; i < kXRows; ++i) wv[i] = load_nt(base + i * chunks);
    scl = scale[rs + ti];
  };
  auto step = [&](int64_t g, const uint4 (&wv)[kXRows], int buf, float scl) {
    float acc[kVals];
#pragma unroll
    for (int i = 0; i < kXRows; ++i) {
      uint32_t hp[8];
      int8x4_to_half2x2(wv[i].x, hp[0], hp[1]);
      int8x4_to_half2x2(wv[i].y, hp[2], hp[3]);
      int8x4_to_half2x2(wv[i].z, hp[4], hp[5]);
      int8x4_to_half2x2(wv[i].w, hp[6], hp[7]);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        // the first dot2 of the chain takes an inline zero (no zeroing move)
        float a;
        asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(a) : "v"(hp[0]), "v"(xp[m][0]));
#pragma unroll
        for (int p = 1; p < 8; ++p) a = dot2(hp[p], xp[m][p], a);
        acc[i * M + m] = a;
      }
    }
#pragma unroll
    for (int q = 0; q < kRed; ++q) {
      const float red = wave_reduce4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
      if (slot >= 0) part[buf][s][4 * q + slot] = red;
    }
    __syncthreads();
    if (threadIdx.x < kVals) {
      const int64_t r = first_row(g) + ti;
      if (r >= g * kXRows) {
        float sum = part[buf][0][threadIdx.x];
#pragma unroll
        for (int t = 1; t < SW; ++t) sum += part[buf][t][threadIdx.x];
        const float v = sum * scl;
        const int m = threadIdx.x % M;
        if constexpr (AM) atomicMax(&wg_key[m], argmax_key(v, r));
        else y[static_cast<int64_t>(m) * n + r] = v;
      }
    }
  };
  uint4 wa[kXRows], wb[kXRows];
  float sa, sb;
  int64_t g = blockIdx.x;
  load(g, wa, sa);
  for (; g < ng; g += 2 * stride) {  // workgroup-uniform
    load(g + stride, wb, sb);
    __builtin_amdgcn_sched_barrier(0);
    step(g, wa, 0, sa);
    if (g + stride >= ng) break;
    load(g + 2 * stride, wa, sa);
    __builtin_amdgcn_sched_barrier(0);
    step(g + stride, wb, 1, sb);
  }
  if constexpr (AM) {
    __syncthreads();
    if (threadIdx.x < M) atomicMax(argmax_bin(keys, threadIdx.x), wg_key[threadIdx.x]);
  }
}

// Compute units of the current device (queried once per device).
int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <int M, bool AM>
void launch_head_persist(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                         unsigned long long* keys, hipStream_t stream) {
  // resident workgroups per CU: LDS (160 KB on gfx950) for larger M, else 3 (the best of 2..4 in sweeps)
  constexpr int kLds = 16 * M * (kPMaxK / 8) + 4 * 2 * kPTiles * kPQuarters * 16 * M;
  constexpr int kPerCu = (160 * 1024) / kLds < 3 ? (160 * 1024) / kLds : 3;
  const int64_t nrb = (n + kPTiles * 16 - 1) / (kPTiles * 16);
  const int64_t cap = static_cast<int64_t>(kPerCu) * compute_units();
  const dim3 grid(static_cast<unsigned>(nrb < cap ? nrb : cap));
  hipLaunchKernelGGL((int8_head_persist_kernel<M, AM>), grid, dim3(kPWaves * kWave), 0, stream, w, scale, n, k, x,
                     y, keys);
}

template <int M, bool AM>
void launch_head_xreg(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                      unsigned long long* keys, hipStream_t stream) {
  // three workgroups per CU: 3-4 waves per SIMD at 120-140 VGPRs
  const int64_t ng = (n + kXRows - 1) / kXRows;
  const int64_t cap = 3 * static_cast<int64_t>(compute_units());
  const dim3 grid(static_cast<unsigned>(ng < cap ? ng : cap));
  switch (k / kXSlice) {  // the K-slices, one wave each, as a constant for the address arithmetic
    case 1: hipLaunchKernelGGL((int8_head_xreg_kernel<M, 1, AM>), grid, dim3(kWave), 0, stream, w, scale, n, x, y, keys); break;
    case 2: hipLaunchKernelGGL((int8_head_xreg_kernel<M, 2, AM>), grid, dim3(2 * kWave), 0, stream, w, scale, n, x, y, keys); break;
    case 3: hipLaunchKernelGGL((int8_head_xreg_kernel<M, 3, AM>), grid, dim3(3 * kWave), 0, stream, w, scale, n, x, y, keys); break;
    default: hipLaunchKernelGGL((int8_head_xreg_kernel<M, 4, AM>), grid, dim3(4 * kWave), 0, stream, w, scale, n, x, y, keys); break;
  }
}

template <int M, bool AM>
void launch_head_any(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                     unsigned long long* keys, hipStream_t stream) {
  const bool aligned = k % 16 == 0 && (reinterpret_cast<uintptr_t>(w) & 15u) == 0 &&
                       (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
  const int64_t units = (k / 16 + 3) / 4;  // 64-column units
  if (aligned && M == 1) {
    // two groups of 4 rows per 8-wave workgroup: 85.6-86.3 us at steady
    // clocks against 92.1-93.0 for two groups of 8 rows and 86.9-90.2 for one
    // group of 4 to 12 (graph-timed, bit-identical). Timed within ~30 ms of an
    // idle gap, while power management holds the VALU-heavier launches back,
    // the 4-row groups measured slower than the 8-row ones.
    launch_head_fast<1, 4, 2, 4, AM>(w, scale, n, k, x, y, keys, stream);
  } else if (aligned && M == 2) {
    // two activation rows still fit the VALU path. One group of 8 rows per
    // 4-wave workgroup streams the 151,936 x 4,096 head at the rate of a
    // plain read: 89.6-92.9 us at steady clocks, against 96.7-98.6 us for
    // groups of 4 rows and 106.8 us for the persistent matrix-core kernel.
    // Workgroups that re-read x for every group of rows lose from M = 3
    // (best 111.8 against 108.4 us at M = 3); the kernel above, which keeps
    // x in registers, takes M = 3 and 4.
    launch_head_fast<2, 4, 1, 8, AM>(w, scale, n, k, x, y, keys, stream);
  } else if (aligned && (M == 3 || M == 4) && k % kXSlice == 0 && k <= 4 * kXSlice && n >= kXRows) {
    if constexpr (M == 3 || M == 4) launch_head_xreg<M, AM>(w, scale, n, k, x, y, keys, stream);
  } else if (aligned && k % kPKStep == 0 && k <= kPMaxK) {
    launch_head_persist<M, AM>(w, scale, n, k, x, y, keys, stream);
  } else if (aligned && M >= 3 && units <= 8 * 16) {
    // Other k: 8 waves split the units of 4 tiles (64 rows); at M = 2 the
    // wave-per-4-rows kernel is faster there (measured).
    if (units <= 8) launch_head_mfma<8, 4, 1, AM>(w, scale, n, k, x, M, y, keys, stream);
    else if (units <= 16) launch_head_mfma<8, 4, 2, AM>(w, scale, n, k, x, M, y, keys, stream);
    else if (units <= 32) launch_head_mfma<8, 4, 4, AM>(w, scale, n, k, x, M, y, keys, stream);
    else if (units <= 64) launch_head_mfma<8, 4, 8, AM>(w, scale, n, k, x, M, y, keys, stream);
    else launch_head_mfma<8, 4, 16, AM>(w, scale, n, k, x, M, y, keys, stream);
  } else {
    launch_head_m<M, AM>(w, scale, n, k, x, y, keys, stream);
  }
}

// One wave per activation row: the row's bins are read (four per lane), the
// maximum is reduced across the wave, and the bins are set back to zero so
// that the workspace is ready for the next call without a clearing launch.
__global__ __launch_bounds__(8 * kWave) void argmax_finish_kernel(unsigned long long* __restrict__ keys, int m,
                                                                  int32_t* __restrict__ token,
                                                                  float* __restrict__ logit) {
  static_assert(kArgmaxBins % kWave == 0, "whole bins per lane");
  const int row = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (row >= m) return;  // whole waves leave together
  unsigned long long key = 0ull;
#pragma unroll
  for (int b = lane; b < kArgmaxBins; b += kWave) {
    unsigned long long* p = keys + (static_cast<int64_t>(row) * kArgmaxBins + b) * kArgmaxStride;
    const unsigned long long v = *p;
    key = v > key ? v : key;
    *p = 0ull;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off /= 2) {
    const unsigned long long o = __shfl_xor(key, off, kWave);
    key = o > key ? o : key;
  }
  if (lane == 0) {
    token[row] = argmax_key_row(key);
    if (logit) logit[row] = argmax_key_logit(key);
  }
}

template <bool AM>
hipError_t dispatch_head(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, int m, float* y,
                         unsigned long long* keys, hipStream_t stream) {
  switch (m) {
    case 1: launch_head_any<1, AM>(w, scale, n, k, x, y, keys, stream); break;
    case 2: launch_head_any<2, AM>(w, scale, n, k, x, y, keys, stream); break;
    case 3: launch_head_any<3, AM>(w, scale, n, k, x, y, keys, stream); break;
    case 4: launch_head_any<4, AM>(w, scale, n, k, x, y, keys, stream); break;
    case 5: launch_head_any<5, AM>(w, scale, n, k, x, y, keys, stream); break;
    case 6: launch_head_any<6, AM>(w, scale, n, k, x, y, keys, stream); break;
    case 7: launch_head_any<7, AM>(w, scale, n, k, x, y, keys, stream); break;
    case 8: launch_head_any<8, AM>(w, scale, n, k, x, y, keys, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_int8_head(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, int m,
                            float* y, hipStream_t stream) {
  return dispatch_head<false>(w, scale, n, k, x, m, y, nullptr, stream);
}

hipError_t launch_int8_head_argmax(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, int m,
                                   unsigned long long* keys, int32_t* token, float* logit, hipStream_t stream) {
  const hipError_t e = dispatch_head<true>(w, scale, n, k, x, m, nullptr, keys, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(argmax_finish_kernel, dim3(1), dim3(8 * kWave), 0, stream, keys, m, token, logit);
  return hipGetLastError();
}

// Bins of int8_head_argmax_noalloc: the keys workspace of PBG_MAX_M rows in
// device memory the library owns (256 KiB on every GPU it runs on, held until
// the process ends). Code-object storage starts zeroed, and every call's
// finishing kernel sets the bins it read back to zero, so the array is zero
// whenever no call is in flight. Calls that overlap in time on one GPU share
// it and race.
static __device__ __align__(256) unsigned long long scratch[PBG_MAX_M * PBG_ARGMAX_KEYS_PER_ROW];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device. In host code the array's name only stands in for the symbol, so
// kernels are handed this address, never the name.
hipError_t scratch_address(unsigned long long** out) {
  static std::atomic<unsigned long long*> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  unsigned long long* p = cache[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    p = static_cast<unsigned long long*>(addr);
    cache[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

hipError_t launch_int8_head_argmax_noalloc(const int8_t* w, const float* scale, int64_t n, int64_t k,
                                           const uint16_t* x, int m, int32_t* token, float* logit,
                                           hipStream_t stream) {
  if (m < 1 || m > PBG_MAX_M) return hipErrorInvalidValue;
  unsigned long long* keys = nullptr;
  const hipError_t e = scratch_address(&keys);
  if (e != hipSuccess) return e;
  return launch_int8_head_argmax(w, scale, n, k, x, m, keys, token, logit, stream);
}

}  // namespace pbg
