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

}  // namespace

hipError_t launch_int8_head(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, int m,
                            float* y, hipStream_t stream) {
  switch (m) {
    case 1: launch_head_m<1>(w, scale, n, k, x, y, stream); break;
    case 2: launch_head_m<2>(w, scale, n, k, x, y, stream); break;
    case 3: launch_head_m<3>(w, scale, n, k, x, y, stream); break;
    case 4: launch_head_m<4>(w, scale, n, k, x, y, stream); break;
    case 5: launch_head_m<5>(w, scale, n, k, x, y, stream); break;
    case 6: launch_head_m<6>(w, scale, n, k, x, y, stream); break;
    case 7: launch_head_m<7>(w, scale, n, k, x, y, stream); break;
    case 8: launch_head_m<8>(w, scale, n, k, x, y, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pbg
