// int8_head_gemv: Y[i][v] = s_v * sum_j w_vj * X[i][j] for the untied int8
// output head with a per-row scale (Neutrino-1 8B model page, "Where the
// bytes live"), for 1..8 activation rows.
//
// Each lane streams 16-byte chunks (16 weights) of 4 rows. A weight byte b is
// turned into the fp16 value b exactly: the byte, biased to b + 128, becomes
// the low mantissa byte of fp16 0x64xx = 1024 + (b + 128), and one packed fp16
// subtraction of 1152 leaves b. v_dot2 then accumulates w * x in fp32.
#include "pbg_device.hpp"
#include "pbg_internal.hpp"

namespace pbg {
namespace {

constexpr int kRowsPerWave = 4;
constexpr int kHeadWaves = 4;

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

template <int M>
__global__ __launch_bounds__(kHeadWaves* kWave) void int8_head_kernel(const int8_t* __restrict__ w,
                                                                       const float* __restrict__ scale, int64_t n,
                                                                       int64_t k, const uint16_t* __restrict__ x,
                                                                       float* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * kHeadWaves + (threadIdx.x / kWave)) * kRowsPerWave;
  if (row0 >= n) return;
  const int64_t chunks = (k + 15) / 16;
  const bool vec = (k % 16 == 0);
  float acc[kRowsPerWave][M];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.0f;
  for (int64_t c = lane; c < chunks; c += kWave) {
    uint32_t xp[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m) load_x_pairs<8>(x + m * k, k, 16 * c, xp[m]);
    uint4 wv[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
      wv[i] = (row0 + i < n) ? load_w_chunk(w + (row0 + i) * k, k, 16 * c, vec) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
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
  const int slot = reduce4_slot(lane);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float r = wave_reduce4(acc[0][m], acc[1][m], acc[2][m], acc[3][m]);
    if (slot >= 0 && row0 + slot < n) y[m * n + row0 + slot] = r * scale[row0 + slot];
  }
}

template <int M>
void launch_head_m(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                   hipStream_t stream) {
  const int64_t rows_per_block = kHeadWaves * kRowsPerWave;
  const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL(int8_head_kernel<M>, grid, dim3(kHeadWaves * kWave), 0, stream, w, scale, n, k, x, y);
}

// Fast path (k % 16 == 0, w and x 16-byte aligned). A workgroup holds G row
// groups x SW K-slices of 1,024 columns; wave (g, s) owns R rows and lane l
// the 16 weights s*1024 + 16*l .. +15 of each of them (slices past SW loop).
// The lane's 16 activations of every row of X stay in registers; all R row
// loads are issued (non-temporal, rows past n clamped) before the first
// conversion, and the row scales are prefetched. Partial sums are reduced
// four at a time across the wave, then added over the SW slices in order in
// LDS.
template <int M, int SW, int G, int R>
__global__ __launch_bounds__(SW* G* kWave) void int8_head_fast_kernel(const int8_t* __restrict__ w,
                                                                       const float* __restrict__ scale, int64_t n,
                                                                       int64_t k, const uint16_t* __restrict__ x,
                                                                       float* __restrict__ y) {
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
        if (idx < kVals && r < n) y[static_cast<int64_t>(idx % M) * n + r] = red[q] * sc[q];
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
          y[static_cast<int64_t>(idx % M) * n + r] = sum * sc[q];
        }
      }
    }
  }
}

template <int M, int SW, int G, int R>
void launch_head_fast(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                      hipStream_t stream) {
  const int64_t rows_per_block = static_cast<int64_t>(G) * R;
  const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL((int8_head_fast_kernel<M, SW, G, R>), grid, dim3(SW * G * kWave), 0, stream, w, scale, n, k, x,
                     y);
}

template <int M>
void launch_head_any(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                     hipStream_t stream) {
  // The register-resident fast path wins at M = 1 (measured); with more rows
  // its per-lane accumulators crowd out waves, and the wave-per-4-rows kernel
  // is faster.
  const bool fast = M == 1 && k % 16 == 0 && (reinterpret_cast<uintptr_t>(w) & 15u) == 0 &&
                    (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
  if (!fast) {
    launch_head_m<M>(w, scale, n, k, x, y, stream);
    return;
  }
  constexpr int kR = M <= 2 ? 8 : 4;
  launch_head_fast<M, 4, 2, kR>(w, scale, n, k, x, y, stream);
}

}  // namespace

hipError_t launch_int8_head(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, int m,
                            float* y, hipStream_t stream) {
  switch (m) {
    case 1: launch_head_any<1>(w, scale, n, k, x, y, stream); break;
    case 2: launch_head_any<2>(w, scale, n, k, x, y, stream); break;
    case 3: launch_head_any<3>(w, scale, n, k, x, y, stream); break;
    case 4: launch_head_any<4>(w, scale, n, k, x, y, stream); break;
    case 5: launch_head_any<5>(w, scale, n, k, x, y, stream); break;
    case 6: launch_head_any<6>(w, scale, n, k, x, y, stream); break;
    case 7: launch_head_any<7>(w, scale, n, k, x, y, stream); break;
    case 8: launch_head_any<8>(w, scale, n, k, x, y, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pbg
