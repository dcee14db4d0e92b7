// The 3-bit (five-level) variant: pack_ternary3, ternary3_gemv (M = 1) and
// ternary3_gemm_small (M <= 8) for gfx950.
//
// Codes c in {-2, -1, 0, +1, +2}, y_r = s_r * sum_j c_rj * x_j (Neutrino-1 8B
// model page: the coded lane is exactly 3 bits per weight, "Where the bytes
// live"; its codes split into zero, plus and minus, "Inside the coded lane").
// A row of K codes, padded to 128 * ceil(K / 128), is its sign/nonzero plane
// in the 2-bit layout followed by a magnitude plane (bit 16h + 8i + t of a
// 32-code word for code 16i + 2t + h), as include/packed_bit_gemv.h states.
//
// The decode helpers are in pbg_device3.hpp.
#include "pbg_device.hpp"
#include "pbg_device3.hpp"
#include "pbg_internal.hpp"

namespace pbg {
namespace {

// ---------------------------------------------------------------------------
// pack_ternary3
// ---------------------------------------------------------------------------
constexpr int kPack3Waves = 8;
constexpr int kPack3MaxBlocks = 512;

struct Tally3 {
  int m2, m1, z, p1, p2;  // codes -2, -1, 0, +1, +2
  int invalid;
};

// One code byte b: its (sign, nonzero) field in bits 1..0, its magnitude
// flag, its value; an invalid byte (outside -2..+2) packs as 0 and counts.
// `real` is false for padding past k (a zero code that is not counted).
__device__ __forceinline__ void code3(uint32_t b, bool real, uint32_t& field, uint32_t& mag, int& value, Tally3& tl) {
  const uint32_t t = (b + 2u) & 0xFFu;  // 0..4 for a valid code
  const bool ok = t <= 4u;
  const int v = ok && real ? static_cast<int>(t) - 2 : 0;
  field = v == 0 ? 0u : (v < 0 ? 3u : 1u);
  mag = (v == 2 || v == -2) ? 1u : 0u;
  value = v;
  if (real) {
    tl.m2 += t == 0u;
    tl.m1 += t == 1u;
    tl.z += t == 2u;
    tl.p1 += t == 3u;
    tl.p2 += t == 4u;
    tl.invalid += !ok;
  }
}

// Packs codes 32g .. 32g + 31 of a row (`here` of them inside k, from src)
// into sign/nonzero words s0, s1 and magnitude word mw; adds them to the row
// sum.
__device__ __forceinline__ void pack_group3(const int8_t* __restrict__ src, int here, bool vec, uint32_t& s0,
                                            uint32_t& s1, uint32_t& mw, int& sum, Tally3& tl) {
  uint32_t bytes[8];
  if (vec) {
    const uint4 a = reinterpret_cast<const uint4*>(src)[0];
    const uint4 b = reinterpret_cast<const uint4*>(src)[1];
    bytes[0] = a.x, bytes[1] = a.y, bytes[2] = a.z, bytes[3] = a.w;
    bytes[4] = b.x, bytes[5] = b.y, bytes[6] = b.z, bytes[7] = b.w;
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      uint32_t v = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * q + e < here) v |= static_cast<uint32_t>(static_cast<uint8_t>(src[4 * q + e])) << (8 * e);
      bytes[q] = v;
    }
  }
  s0 = s1 = mw = 0u;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    uint32_t field, mag;
    int v;
    code3((bytes[j >> 2] >> (8 * (j & 3))) & 0xFFu, j < here, field, mag, v, tl);
    const int i = j >> 4, jj = j & 15, t = jj >> 1, h = jj & 1;
    const uint32_t fbits = field << (16 * h + 14 - 2 * t);
    if (i == 0) s0 |= fbits;
    else s1 |= fbits;
    mw |= mag << (16 * h + 8 * i + t);
    sum += v;
  }
}

__global__ void zero_stats3_kernel(int64_t* stats) {
  if (threadIdx.x < 6) stats[threadIdx.x] = 0;
}

// One wave per row at a time; lane l packs the 32-code groups l, l + 64, ...
// The counts are kept per lane, reduced per workgroup and added with one
// 64-bit integer atomic each (integers: the order does not matter).
__global__ __launch_bounds__(kPack3Waves* kWave) void pack3_kernel(const int8_t* __restrict__ codes, int64_t n,
                                                                   int64_t k, int64_t groups,
                                                                   uint32_t* __restrict__ packed,
                                                                   int32_t* __restrict__ row_sum,
                                                                   int64_t* __restrict__ stats) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const bool aligned = (k % 16 == 0) && ((reinterpret_cast<uintptr_t>(codes) & 15u) == 0);
  const int64_t words = 3 * groups;  // 2 sign/nonzero words and 1 magnitude word per group
  Tally3 tl = {0, 0, 0, 0, 0, 0};
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kPack3Waves;
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * kPack3Waves + wave; row < n; row += stride) {
    const int8_t* src = codes + row * k;
    uint32_t* dst = packed + row * words;
    int sum = 0;
    for (int64_t g = lane; g < groups; g += kWave) {
      const int64_t c0 = 32 * g;
      const int here = c0 < k ? static_cast<int>(k - c0 < 32 ? k - c0 : 32) : 0;
      uint32_t s0, s1, mw;
      pack_group3(src + (here > 0 ? c0 : 0), here, aligned && here == 32, s0, s1, mw, sum, tl);
      dst[2 * g] = s0;
      dst[2 * g + 1] = s1;
      dst[2 * groups + g] = mw;
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    if (lane == 0) row_sum[row] = sum;
  }
  __shared__ int red[6][kPack3Waves];
  int vals[6] = {tl.m2, tl.m1, tl.z, tl.p1, tl.p2, tl.invalid};
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    int v = vals[i];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) red[i][wave] = v;
  }
  __syncthreads();
  if (threadIdx.x < 6) {
    int64_t tot = 0;
    for (int w = 0; w < kPack3Waves; ++w) tot += red[threadIdx.x][w];
    if (tot) atomicAdd(reinterpret_cast<unsigned long long*>(stats + threadIdx.x), static_cast<unsigned long long>(tot));
  }
}

// ---------------------------------------------------------------------------
// ternary3_gemv (M = 1)
// ---------------------------------------------------------------------------
// Fast path: k % 8 == 0, x 16-byte aligned, CPL = ceil(chunks / 64) <= 4.
// The 2-bit kernel's work split and order of events (ternary.hip): a wave
// owns R consecutive rows over the whole K; lane l takes sign/nonzero chunks
// l + 64 j (16 bytes, 64 codes) and the matching 8 bytes of the magnitude
// plane; the activations go through LDS chunk-major; all row loads are in
// flight before the first decode; one transposed reduction ends the rows.
template <int CPL, int G, int R>
__global__ __launch_bounds__(G* kWave) void ternary3_gemv_kernel(const uint32_t* __restrict__ packed,
                                                                 const float* __restrict__ scale, int64_t n,
                                                                 int64_t k, int64_t chunks,
                                                                 const uint16_t* x,  // not restrict: keeps its
                                                                 float* __restrict__ y) {  // loads above the barrier
  static_assert(R >= 1 && R <= 4, "one reduction finishes the rows");
  constexpr int kThreads = G * kWave;
  constexpr int kGroups = CPL * kWave * 8;  // 16-byte activation groups of the CPL chunks of every lane
  constexpr int kXPer = (kGroups + kThreads - 1) / kThreads;
  __shared__ uint4 xs[kGroups];             // group q of chunk 64 j + l at (8 j + q) * 64 + l
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * G + wave) * R;
  const int64_t groups = k / 8;
  const int64_t row_words = 6 * chunks;  // 4 sign/nonzero and 2 magnitude words per chunk
  const uint4* xg = reinterpret_cast<const uint4*>(x);

  uint4 xv[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int gi = threadIdx.x + i * kThreads;
    xv[i] = xg[gi < groups ? gi : 0];
  }
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");  // activation loads queue ahead of the weight loads
  __builtin_amdgcn_sched_barrier(0);

  uint4 w[R][CPL];
  uint2 mg[R][CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int64_t c = lane + static_cast<int64_t>(kWave) * j;
    const int64_t cc = c < chunks ? c : chunks - 1;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t* row = packed + (row0 + i < n ? row0 + i : n - 1) * row_words;
      w[i][j] = load_nt(reinterpret_cast<const uint4*>(row) + cc);
      mg[i][j] = load_nt2(reinterpret_cast<const uint2*>(row + 4 * chunks) + cc);
    }
  }
  const int slot = reduce4_slot(lane);
  const int64_t rs = row0 + (slot < 0 ? 0 : slot);
  const float sc = scale[rs < n ? rs : n - 1];
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int gi = threadIdx.x + i * kThreads;
    if (gi < kGroups) {
      const int c = gi >> 3, q = gi & 7;
      xs[((c >> 6) * 8 + q) * kWave + (c & (kWave - 1))] = masked(xv[i], gi < groups);
    }
  }
  __syncthreads();
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    uint32_t xp[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 v = xs[(j * 8 + q) * kWave + lane];
      xp[4 * q + 0] = v.x;
      xp[4 * q + 1] = v.y;
      xp[4 * q + 2] = v.z;
      xp[4 * q + 3] = v.w;
    }
#pragma unroll
    for (int i = 0; i < R; ++i) acc[i] = chunk3_dot(w[i][j], mg[i][j], xp, acc[i]);
  }
  const float red = wave_reduce4(acc[0], acc[1], acc[2], acc[3]);
  if (slot >= 0 && slot < R && row0 + slot < n) y[row0 + slot] = red * (sc * kCodeUnitInv);
}

// Any k and 2-byte-aligned x, 1 <= M <= 8 rows: a wave owns 4 rows and lane l
// the sign/nonzero words l, l + 64, ... of each (16 codes) with their
// magnitude bits; activations are loaded with element guards. Used when the
// fast paths' layout conditions do not hold.
template <int M>
__global__ __launch_bounds__(4 * kWave) void ternary3_generic_kernel(const uint32_t* __restrict__ packed,
                                                                     const float* __restrict__ scale, int64_t n,
                                                                     int64_t k, int64_t chunks,
                                                                     const uint16_t* __restrict__ x,
                                                                     float* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x / kWave)) * 4;
  if (row0 >= n) return;  // whole wave leaves together
  const int64_t row_words = 6 * chunks, words = 4 * chunks;
  float acc[4][M];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.0f;
  for (int64_t wi = lane; wi < words; wi += kWave) {
    uint32_t xp[M][8];
#pragma unroll
    for (int m = 0; m < M; ++m) load_x_pairs<8>(x + m * k, k, 16 * wi, xp[m]);
    const int half = static_cast<int>(wi & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t* row = packed + (row0 + i < n ? row0 + i : n - 1) * row_words;
      const uint32_t w = row0 + i < n ? row[wi] : 0u;
      const uint32_t mw = row0 + i < n ? row[words + (wi >> 1)] : 0u;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint32_t op = code_pair(w, t) | mag_pair(mw, half, t);
#pragma unroll
        for (int m = 0; m < M; ++m) acc[i][m] = dot2(op, xp[m][t], acc[i][m]);
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

// 2 <= M <= 8 on the matrix cores (k % 8 == 0, x 16-byte aligned): the 2-bit
// small-M kernel of ternary.hip (ternary_gemm_mfma_kernel: 16-row tiles of
// decoded codes as the A operand of v_mfma_f32_16x16x32_f16, activations as
// B columns, whole-line x loads transposed through a per-wave LDS slice, SK
// waves splitting the 256-column units of T tiles) with the magnitude bits
// OR-ed into every A operand. Lane (i, g) loads, per unit, sign/nonzero chunk
// 4u + g of its row (16 bytes) and that chunk's two magnitude words.
// SPLIT2: K is also split across workgroups into at most two slices of SK *
// UPW units (blockIdx.y, as in the 2-bit kernel's SPLIT = 2): each adds s *
// its partial to y, which holds +0 on entry, with an fp32 atomic add; two
// addends onto +0 give the same bits in either order.
template <int SK, int T, int UPW, int MP, bool SPLIT2>
__global__ __launch_bounds__(SK* kWave) void ternary3_gemm_mfma_kernel(const uint32_t* __restrict__ packed,
                                                                        const float* __restrict__ scale, int64_t n,
                                                                        int64_t k, int64_t chunks,
                                                                        const uint16_t* __restrict__ x, int m,
                                                                        float* __restrict__ y) {
  constexpr int kRows = 16 * T;
  __shared__ float part[SK][kRows][8];
  const int lane = threadIdx.x & (kWave - 1);
  const int s = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int li = lane & 15, lg = lane >> 4;
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * kRows;
  const int64_t groups = k / 8;
  const int64_t row_words = 6 * chunks;
  const int64_t u0 = SPLIT2 ? static_cast<int64_t>(blockIdx.y) * SK * UPW : 0;  // first unit of the slice
  const uint4* xg = reinterpret_cast<const uint4*>(x);

  constexpr int kOut = (kRows * 8 + SK * kWave - 1) / (SK * kWave);
  float sc[kOut];
#pragma unroll
  for (int e = 0; e < kOut; ++e) {
    const int o = threadIdx.x + e * SK * kWave;
    const int64_t r = row_base + (o < kRows * 8 ? o >> 3 : kRows - 1);
    sc[e] = scale[r < n ? r : n - 1];
  }

  constexpr int kXLoads = MP / 2;
  constexpr int kSlots = 33;  // 16-byte slots per row and unit, one of padding
  __shared__ uint4 xs[SK][2][MP * kSlots];
  const int xrow = li >> 3, xg8 = li & 7;
  auto load_x = [&](int q, uint4 (&xr)[kXLoads]) {
    const int64_t u = u0 + s + static_cast<int64_t>(SK) * q;
#pragma unroll
    for (int a = 0; a < kXLoads; ++a) {
      const int row = 2 * a + xrow;
      const int64_t gi = 32 * u + 8 * lg + xg8;
      xr[a] = xg[row < m && gi < groups ? static_cast<int64_t>(row) * groups + gi : 0];
    }
  };
  auto stage_x = [&](int q, const uint4 (&xr)[kXLoads]) {
    const int64_t gi = 32 * (u0 + s + static_cast<int64_t>(SK) * q) + 8 * lg + xg8;
#pragma unroll
    for (int a = 0; a < kXLoads; ++a)
      xs[s][q & 1][(2 * a + xrow) * kSlots + 8 * lg + xg8] = masked(xr[a], gi < groups);
  };
  auto load_w = [&](int q, uint4 (&wv)[T], uint2 (&mv)[T]) {
    const int64_t c = 4 * (u0 + s + static_cast<int64_t>(SK) * q) + lg;
    const int64_t cc = c < chunks ? c : chunks - 1;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t r = row_base + 16 * t + li;
      const uint32_t* row = packed + (r < n ? r : n - 1) * row_words;
      wv[t] = load_nt(reinterpret_cast<const uint4*>(row) + cc);
      mv[t] = load_nt2(reinterpret_cast<const uint2*>(row + 4 * chunks) + cc);
    }
  };

  mfma_float4_t d[T];
#pragma unroll
  for (int t = 0; t < T; ++t) d[t] = mfma_float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  uint4 xr[kXLoads], wv[2][T];
  uint2 mv[2][T];
  load_x(0, xr);
  load_w(0, wv[0], mv[0]);
  stage_x(0, xr);
  if (UPW > 1) {
    load_x(1, xr);
    load_w(1, wv[1], mv[1]);
  }
  const int brow = (li % MP) * kSlots + 8 * lg;
#pragma unroll
  for (int q = 0; q < UPW; ++q) {
    __builtin_amdgcn_sched_barrier(0);
    mfma3_unit_half<0, T>(wv[q & 1], mv[q & 1], &xs[s][q & 1][brow], d);
    mfma3_unit_half<1, T>(wv[q & 1], mv[q & 1], &xs[s][q & 1][brow], d);
    if (q + 1 < UPW) {
      stage_x(q + 1, xr);
      if (q + 2 < UPW) {
        load_x(q + 2, xr);
        load_w(q + 2, wv[q & 1], mv[q & 1]);
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
      for (int w = 1; w < SK; ++w) sum += part[w][orow][ocol];
      if constexpr (SPLIT2)
        __hip_atomic_fetch_add(y + static_cast<int64_t>(ocol) * n + r, sum * (sc[e] * kCodeUnitInv),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        y[static_cast<int64_t>(ocol) * n + r] = sum * (sc[e] * kCodeUnitInv);
    }
  }
}

template <int SK, int T, int UPW, int MP>
void launch_mfma3_mp(const uint32_t* packed, const float* scale, int64_t n, int64_t k, int64_t chunks,
                     const uint16_t* x, int m, float* y, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((n + 16 * T - 1) / (16 * T)));
  hipLaunchKernelGGL((ternary3_gemm_mfma_kernel<SK, T, UPW, MP, false>), grid, dim3(SK * kWave), 0, stream, packed,
                     scale, n, k, chunks, x, m, y);
}

// Two K-slices added onto a zeroed y.
template <int SK, int T, int UPW, int MP>
void launch_mfma3_split2_mp(const uint32_t* packed, const float* scale, int64_t n, int64_t k, int64_t chunks,
                            const uint16_t* x, int m, float* y, hipStream_t stream) {
  const int64_t units = (chunks + 3) / 4;
  const unsigned slices = static_cast<unsigned>((units + SK * UPW - 1) / (SK * UPW));
  hipLaunchKernelGGL((ternary3_gemm_mfma_kernel<SK, T, UPW, MP, true>),
                     dim3(static_cast<unsigned>((n + 16 * T - 1) / (16 * T)), slices), dim3(SK * kWave), 0, stream,
                     packed, scale, n, k, chunks, x, m, y);
}

template <int SK, int T, int UPW>
void launch_mfma3_cfg(const uint32_t* packed, const float* scale, int64_t n, int64_t k, int64_t chunks,
                      const uint16_t* x, int m, float* y, hipStream_t stream) {
  if (m <= 2) launch_mfma3_mp<SK, T, UPW, 2>(packed, scale, n, k, chunks, x, m, y, stream);
  else if (m <= 4) launch_mfma3_mp<SK, T, UPW, 4>(packed, scale, n, k, chunks, x, m, y, stream);
  else launch_mfma3_mp<SK, T, UPW, 8>(packed, scale, n, k, chunks, x, m, y, stream);
}

template <int CPL, int G, int R>
void launch_gemv3_cfg(const uint32_t* packed, const float* scale, int64_t n, int64_t k, int64_t chunks,
                      const uint16_t* x, float* y, hipStream_t stream) {
  const int64_t rows_per_block = static_cast<int64_t>(G) * R;
  const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL((ternary3_gemv_kernel<CPL, G, R>), grid, dim3(G * kWave), 0, stream, packed, scale, n, k, chunks,
                     x, y);
}

template <int M>
void launch_generic3(const uint32_t* packed, const float* scale, int64_t n, int64_t k, int64_t chunks,
                     const uint16_t* x, float* y, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((n + 15) / 16));
  hipLaunchKernelGGL((ternary3_generic_kernel<M>), grid, dim3(4 * kWave), 0, stream, packed, scale, n, k, chunks, x,
                     y);
}

}  // namespace

hipError_t launch_pack3(const int8_t* codes, int64_t n, int64_t k, uint32_t* packed, int32_t* row_sum,
                        int64_t* stats, hipStream_t stream) {
  const int64_t groups = words_per_row3(k) / 3;
  hipLaunchKernelGGL(zero_stats3_kernel, dim3(1), dim3(64), 0, stream, stats);
  const int64_t blocks = (n + kPack3Waves - 1) / kPack3Waves;
  hipLaunchKernelGGL(pack3_kernel, dim3(static_cast<unsigned>(blocks < kPack3MaxBlocks ? blocks : kPack3MaxBlocks)),
                     dim3(kPack3Waves * kWave), 0, stream, codes, n, k, groups, packed, row_sum, stats);
  return hipGetLastError();
}

hipError_t launch_ternary3_gemv(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                                float* y, hipStream_t stream) {
  const int64_t chunks = words_per_row3(k) / 6;  // 16-byte sign/nonzero chunks per row
  const int64_t cpl = (chunks + kWave - 1) / kWave;
  if (k % 8 != 0 || (reinterpret_cast<uintptr_t>(x) & 15u) != 0 || cpl > 4) {
    launch_generic3<1>(packed, scale, n, k, chunks, x, y, stream);
    return hipGetLastError();
  }
  const bool big = n >= 2048;
  switch (cpl) {
    case 1:
      if (n >= 8192) launch_gemv3_cfg<1, 4, 3>(packed, scale, n, k, chunks, x, y, stream);
      else if (big) launch_gemv3_cfg<1, 4, 2>(packed, scale, n, k, chunks, x, y, stream);
      else launch_gemv3_cfg<1, 4, 1>(packed, scale, n, k, chunks, x, y, stream);
      break;
    case 2:
      if (big) launch_gemv3_cfg<2, 4, 2>(packed, scale, n, k, chunks, x, y, stream);
      else launch_gemv3_cfg<2, 4, 1>(packed, scale, n, k, chunks, x, y, stream);
      break;
    case 3:
      if (big) launch_gemv3_cfg<3, 8, 1>(packed, scale, n, k, chunks, x, y, stream);
      else launch_gemv3_cfg<3, 4, 1>(packed, scale, n, k, chunks, x, y, stream);
      break;
    default:
      if (big) launch_gemv3_cfg<4, 8, 1>(packed, scale, n, k, chunks, x, y, stream);
      else launch_gemv3_cfg<4, 4, 1>(packed, scale, n, k, chunks, x, y, stream);
      break;
  }
  return hipGetLastError();
}

bool ternary3_split2_applies(int64_t n, int64_t k, int m, const uint16_t* x) {
  const int64_t units = (words_per_row3(k) / 6 + 3) / 4;  // 256-column units
  return k % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15u) == 0 && m >= 2 && m <= 8 && units > 16 &&
         units <= 48 && n > 0;
}

hipError_t launch_ternary3_gemm_split2(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                                       const uint16_t* x, int m, float* y, hipStream_t stream) {
  if (!ternary3_split2_applies(n, k, m, x)) return hipErrorInvalidValue;
  const int64_t chunks = words_per_row3(k) / 6;
  // the 2-bit block's shape: 32-row blocks, 8 waves of 3 units, slices of 24 units
  if (m <= 2) launch_mfma3_split2_mp<8, 2, 3, 2>(packed, scale, n, k, chunks, x, m, y, stream);
  else if (m <= 4) launch_mfma3_split2_mp<8, 2, 3, 4>(packed, scale, n, k, chunks, x, m, y, stream);
  else launch_mfma3_split2_mp<8, 2, 3, 8>(packed, scale, n, k, chunks, x, m, y, stream);
  return hipGetLastError();
}

hipError_t launch_ternary3_gemm_small(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                                      const uint16_t* x, int m, float* y, hipStream_t stream) {
  if (m == 1) return launch_ternary3_gemv(packed, scale, n, k, x, y, stream);
  const int64_t chunks = words_per_row3(k) / 6;
  const int64_t units = (chunks + 3) / 4;  // 256-column units
  if (k % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15u) == 0 && units <= 64) {
    // The 2-bit small-M launch shapes (ternary.hip), by rows and units.
    if (units <= 16) {
      // N >= 8,192 from a graph-timed sweep of ten shapes at 12,288 x 4,096
      // (pools of 36 matrices, both orders): one tile of 4 waves at m = 2
      // (7.40 against 7.70 us for three tiles), three tiles of 8 waves from m
      // = 3 (7.83 / 8.15 against 7.94 / 8.33 us at m = 4 / 8); the other
      // shapes of this table were the fastest or within 0.05 us of it
      if (n >= 8192 && m == 2) launch_mfma3_cfg<4, 1, 4>(packed, scale, n, k, chunks, x, m, y, stream);
      else if (n >= 8192) launch_mfma3_cfg<8, 3, 2>(packed, scale, n, k, chunks, x, m, y, stream);
      else if (n >= 5120) launch_mfma3_cfg<4, 2, 4>(packed, scale, n, k, chunks, x, m, y, stream);
      else launch_mfma3_cfg<8, 1, 2>(packed, scale, n, k, chunks, x, m, y, stream);
    } else if (units <= 32) {
      launch_mfma3_cfg<8, 1, 4>(packed, scale, n, k, chunks, x, m, y, stream);
    } else if (units <= 48) {
      launch_mfma3_cfg<12, 1, 4>(packed, scale, n, k, chunks, x, m, y, stream);
    } else {
      launch_mfma3_cfg<8, 1, 8>(packed, scale, n, k, chunks, x, m, y, stream);
    }
    return hipGetLastError();
  }
  switch (m) {
    case 2: launch_generic3<2>(packed, scale, n, k, chunks, x, y, stream); break;
    case 3: launch_generic3<3>(packed, scale, n, k, chunks, x, y, stream); break;
    case 4: launch_generic3<4>(packed, scale, n, k, chunks, x, y, stream); break;
    case 5: launch_generic3<5>(packed, scale, n, k, chunks, x, y, stream); break;
    case 6: launch_generic3<6>(packed, scale, n, k, chunks, x, y, stream); break;
    case 7: launch_generic3<7>(packed, scale, n, k, chunks, x, y, stream); break;
    case 8: launch_generic3<8>(packed, scale, n, k, chunks, x, y, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pbg
