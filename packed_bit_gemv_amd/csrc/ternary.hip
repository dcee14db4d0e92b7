// ternary_gemv (M = 1) and ternary_gemm_small (M <= 8) for gfx950.
//
// y_r = s_r * sum_j c_rj * x_j with the codes decoded in registers from the
// packed words (Neutrino-1 8B model page: the kernels expand the codes
// themselves, introduction; per-row scale, "Where the bytes live"; a drafted run
// scored in one forward pass, "speculative").
//
// Work split (M = 1): a wave owns R consecutive rows (R <= 4) over the whole
// K. Lane l streams the 16-byte chunks (64 codes) l, l + 64, ... of each row,
// reads the matching activations from LDS as fp16 pairs and accumulates fp32
// partial sums with v_dot2; every row load of the wave is in flight before the
// first decode. The rows are finished by one transposed cross-lane reduction.
#include "pbg_device.hpp"
#include "pbg_internal.hpp"

namespace pbg {
namespace {

constexpr int kRowsPerWave = 4;  // small-M kernel
constexpr int kGemvWaves = 4;

// M = 1, fast path: k % 8 == 0, x 16-byte aligned and CPL = ceil(k / 4,096)
// <= 4 chunks per lane. A workgroup holds G waves; wave g owns R consecutive
// rows and lane l the chunks l + 64 j (j < CPL) of each of them.
//  1. Every thread loads its share of the activations, then a barrier: all
//     activation loads are queued in the vector memory pipe before any weight
//     load, so they return first.
//  2. Each wave issues all R * CPL row loads (rows past n and chunks past the
//     row clamped) and the row scale, unconditionally, so the compiler can
//     retire them in order.
//  3. The activations go through LDS, chunk-major and conflict-free; for each
//     j the lane reads its 32 fp16 pairs once and decodes that chunk of all R
//     rows, so every activation is read from LDS once per wave.
//  4. One transposed reduction over the wave finishes the R rows.
// Splitting K across the waves of a workgroup instead (and adding the slices
// in LDS) measured 9-25 % slower for CPL = 2..4 on MI355X, and across
// workgroups (ternary_gemm_splitk's scheme) no faster at one activation row:
// the combine's atomic round trip ends the launch later than the shorter
// activation staging saves.
template <int CPL, int G, int R>
__global__ __launch_bounds__(G* kWave) void ternary_gemv_kernel(const uint4* __restrict__ packed,
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
  const uint4* xg = reinterpret_cast<const uint4*>(x);

  // 1. activations first
  uint4 xv[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int gi = threadIdx.x + i * kThreads;
    xv[i] = xg[gi < groups ? gi : 0];
  }
  // Order, not wait: the activation loads stay in flight across the barrier.
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // 2. rows and scale
  uint4 w[R][CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int64_t c = lane + static_cast<int64_t>(kWave) * j;
    const int64_t cc = c < chunks ? c : chunks - 1;
#pragma unroll
    for (int i = 0; i < R; ++i) w[i][j] = load_nt(packed + (row0 + i < n ? row0 + i : n - 1) * chunks + cc);
  }
  const int slot = reduce4_slot(lane);
  const int64_t rs = row0 + (slot < 0 ? 0 : slot);
  const float sc = scale[rs < n ? rs : n - 1];
  __builtin_amdgcn_sched_barrier(0);

  // 3. activations through LDS (zero past k), decoded chunk by chunk
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
    for (int i = 0; i < R; ++i) acc[i] = chunk_dot(w[i][j], xp, acc[i]);
  }

  // 4. reduction and epilogue
  const float red = wave_reduce4(acc[0], acc[1], acc[2], acc[3]);
  if (slot >= 0 && slot < R && row0 + slot < n) y[row0 + slot] = red * (sc * kCodeUnitInv);
}

// 2 <= M <= 3, fast path (same conditions as the M = 1 fast path, K <= 12,288):
// the M = 1 kernel with M activation rows. All M rows go through LDS; for
// each chunk the lane reads the 32 fp16 pairs of every row once, decodes
// each operand once and feeds it to M dot2s, so the decode is shared and the
// weights are read once for all M rows. The R * M sums are reduced four at a
// time. Past M = 3 the activation pairs no longer fit in registers and the
// matrix-core kernel below takes over.
template <int CPL, int G, int R, int M>
__global__ __launch_bounds__(G* kWave) void ternary_gemm_rows_kernel(const uint4* __restrict__ packed,
                                                                     const float* __restrict__ scale, int64_t n,
                                                                     int64_t k, int64_t chunks, const uint16_t* x,
                                                                     float* __restrict__ y) {
  constexpr int kThreads = G * kWave;
  constexpr int kGroups = CPL * kWave * 8;  // 16-byte activation groups per activation row
  constexpr int kXPer = (M * kGroups + kThreads - 1) / kThreads;
  constexpr int kVals = R * M;              // sum (row i, activation row m) at i * M + m
  constexpr int kRed = (kVals + 3) / 4;
  __shared__ uint4 xs[M][kGroups];          // group q of chunk 64 j + l at (8 j + q) * 64 + l
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * G + wave) * R;
  const int64_t groups = k / 8;
  const uint4* xg = reinterpret_cast<const uint4*>(x);

  uint4 xv[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int gi = threadIdx.x + i * kThreads;
    const int m = gi / kGroups, g = gi % kGroups;
    xv[i] = xg[m < M && g < groups ? m * groups + g : 0];
  }
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");  // activation loads queue ahead of the weight loads
  __builtin_amdgcn_sched_barrier(0);

  uint4 w[R][CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int64_t c = lane + static_cast<int64_t>(kWave) * j;
    const int64_t cc = c < chunks ? c : chunks - 1;
#pragma unroll
    for (int i = 0; i < R; ++i) w[i][j] = load_nt(packed + (row0 + i < n ? row0 + i : n - 1) * chunks + cc);
  }
  const int slot = reduce4_slot(lane);
  float sc[kRed];
#pragma unroll
  for (int q = 0; q < kRed; ++q) {
    const int idx = 4 * q + (slot < 0 ? 0 : slot);
    const int64_t r = row0 + (idx < kVals ? idx / M : 0);
    sc[q] = scale[r < n ? r : n - 1];
  }
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int gi = threadIdx.x + i * kThreads;
    const int m = gi / kGroups, g = gi % kGroups;
    if (m < M) {
      const int c = g >> 3, q = g & 7;
      xs[m][((c >> 6) * 8 + q) * kWave + (c & (kWave - 1))] = masked(xv[i], g < groups);
    }
  }
  __syncthreads();
  float acc[4 * kRed];
#pragma unroll
  for (int i = 0; i < 4 * kRed; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    uint32_t xp[M][32];
#pragma unroll
    for (int m = 0; m < M; ++m)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint4 v = xs[m][(j * 8 + q) * kWave + lane];
        xp[m][4 * q + 0] = v.x;
        xp[m][4 * q + 1] = v.y;
        xp[m][4 * q + 2] = v.z;
        xp[m][4 * q + 3] = v.w;
      }
#pragma unroll
    for (int i = 0; i < R; ++i) chunk_dot_m<M>(w[i][j], xp, &acc[i * M]);
  }
  float red[kRed];
#pragma unroll
  for (int q = 0; q < kRed; ++q) red[q] = wave_reduce4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  if (slot >= 0) {
#pragma unroll
    for (int q = 0; q < kRed; ++q) {
      const int idx = 4 * q + slot;
      const int64_t r = row0 + idx / M;
      if (idx < kVals && r < n) y[static_cast<int64_t>(idx % M) * n + r] = red[q] * (sc[q] * kCodeUnitInv);
    }
  }
}

// M = 1, any k and any 2-byte-aligned x: a wave owns 4 rows, loads are
// guarded element by element. Used only when the fast path's layout
// conditions do not hold.
__global__ __launch_bounds__(4 * kWave) void ternary_gemv_generic_kernel(const uint4* __restrict__ packed,
                                                                         const float* __restrict__ scale,
                                                                         int64_t n, int64_t k, int64_t chunks,
                                                                         const uint16_t* __restrict__ x,
                                                                         float* __restrict__ y) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x / kWave)) * 4;
  if (row0 >= n) return;  // whole wave leaves together
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t c = lane; c < chunks; c += kWave) {
    uint32_t xp[32];
    load_x_pairs<32>(x, k, 64 * c, xp);
    uint4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (row0 + i < n) ? packed[(row0 + i) * chunks + c] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = chunk_dot(w[i], xp, acc[i]);
  }
  const float r = wave_reduce4(acc[0], acc[1], acc[2], acc[3]);
  const int slot = reduce4_slot(lane);
  if (slot >= 0 && row0 + slot < n) y[row0 + slot] = r * (scale[row0 + slot] * kCodeUnitInv);
}

template <int CPL, int G, int R>
void launch_gemv_cfg(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                     hipStream_t stream) {
  const int64_t rows_per_block = static_cast<int64_t>(G) * R;
  const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL((ternary_gemv_kernel<CPL, G, R>), grid, dim3(G * kWave), 0, stream,
                     reinterpret_cast<const uint4*>(packed), scale, n, k, words_per_row(k) / 4, x, y);
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

// Small M on the matrix cores (2 <= M <= 8, k % 8 == 0, x 16-byte aligned).
// v_mfma_f32_16x16x32_f16 multiplies a 16-row tile of decoded codes (A,
// 16 x 32) by 16 activation columns (B, 32 x 16, of which columns j < M are
// used), so the cost per code does not grow with M. A lane with row i = lane
// % 16 and K-group g = lane / 16 loads 16 bytes (64 codes) of its row per
// 256-column unit u: codes 256u + 64g .. +63. MFMA step v (0..7) of the unit
// takes codes 256u + 64g + 8v .. +7 of that lane (word v/2, half v%2, decoded
// as 4 operand pairs), and the B lane (g, j) holds x_j at the same 8 columns,
// so A and B agree on every column whatever order the unit uses inside a
// K-group. The accumulator lane (g, j) holds rows 4g..4g+3 of column j.
// Only columns j < M <= MP of B matter (MP = 2, 4 or 8). x is loaded a whole
// 128-byte line at a time: load a of a unit gives lane-group g the line of
// groups 8g..8g+7 for rows 2a and 2a + 1, so MP / 2 loads cover the unit. A
// per-wave LDS slice (MP rows of 32 16-byte slots plus one of padding, two
// buffers) turns that into the B layout: step v reads slot 8g + v of row
// j mod MP, conflict-free. Columns j >= M are discarded in the epilogue.
// A workgroup holds SK waves that split the units of T tiles; their partial
// tiles meet in LDS and are added in wave order.
// SPLIT (0 = whole K per workgroup): K is also split across workgroups;
// blockIdx.y is the slice of SK * UPW units (starting at unit blockIdx.y * SK
// * UPW). SPLIT = 1: the slices of a row block meet through `sp` (SplitK).
// SPLIT = 2: at most two slices, each adds s * its partial to y with an fp32
// atomic add; y holds +0 on entry, and +0 + a + b gives the same bits in
// either order, so the result does not depend on which slice ends first.
template <int SK, int T, int UPW, int MP, int SPLIT>
__global__ __launch_bounds__(SK* kWave) void ternary_gemm_mfma_kernel(const uint4* __restrict__ packed,
                                                                       const float* __restrict__ scale,
                                                                       int64_t n, int64_t k, int64_t chunks,
                                                                       const uint16_t* __restrict__ x, int m,
                                                                       float* __restrict__ y, SplitK sp) {
  constexpr int kRows = 16 * T;
  __shared__ float part[SK][kRows][8];
  const int lane = threadIdx.x & (kWave - 1);
  const int s = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int li = lane & 15, lg = lane >> 4;
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * kRows;
  const int64_t groups = k / 8;  // 8-column activation groups
  const int64_t u0 = SPLIT != 0 ? static_cast<int64_t>(blockIdx.y) * SK * UPW : 0;  // first unit of the slice
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

  // x of one 256-column unit: MP / 2 line-wise loads, staged through this
  // wave's LDS slice. Rows past m read x[0..7] (their columns are discarded)
  // and groups past k are zeroed when staged.
  constexpr int kXLoads = MP / 2;
  constexpr int kSlots = 33;  // 16-byte slots per row and unit, one of padding
  __shared__ uint4 xs[SK][2][MP * kSlots];
  const int xrow = li >> 3, xg8 = li & 7;
  auto load_x = [&](int q, uint4 (&xr)[kXLoads]) {
    const int64_t u = u0 + s + static_cast<int64_t>(SK) * q;
#pragma unroll
    for (int a = 0; a < kXLoads; ++a) {
      const int row = 2 * a + xrow;
      const int64_t gi = 32 * u + 8 * lg + xg8;  // 8-column group within a row of x
      xr[a] = xg[row < m && gi < groups ? static_cast<int64_t>(row) * groups + gi : 0];
    }
  };
  auto stage_x = [&](int q, const uint4 (&xr)[kXLoads]) {
    const int64_t gi = 32 * (u0 + s + static_cast<int64_t>(SK) * q) + 8 * lg + xg8;
#pragma unroll
    for (int a = 0; a < kXLoads; ++a)
      xs[s][q & 1][(2 * a + xrow) * kSlots + 8 * lg + xg8] = masked(xr[a], gi < groups);
  };
  // one 16-byte chunk of A per tile
  auto load_w = [&](int q, uint4 (&wv)[T]) {
    const int64_t c = 4 * (u0 + s + static_cast<int64_t>(SK) * q) + lg;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t r = row_base + 16 * t + li;
      wv[t] = load_nt(packed + (r < n ? r : n - 1) * chunks + (c < chunks ? c : chunks - 1));
    }
  };

  mfma_float4_t d[T];
#pragma unroll
  for (int t = 0; t < T; ++t) d[t] = mfma_float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // unit q + 1's loads are in flight while unit q is decoded; its x is
  // staged after unit q's last MFMA
  uint4 xr[kXLoads], wv[2][T];
  load_x(0, xr);
  load_w(0, wv[0]);
  stage_x(0, xr);
  if (UPW > 1) {
    load_x(1, xr);
    load_w(1, wv[1]);
  }
  const int brow = (li % MP) * kSlots + 8 * lg;  // B slots of this lane (lanes j >= MP repeat a row)
#pragma unroll
  for (int q = 0; q < UPW; ++q) {
    __builtin_amdgcn_sched_barrier(0);
    mfma_unit_half<0, T>(wv[q & 1], &xs[s][q & 1][brow], d);
    mfma_unit_half<1, T>(wv[q & 1], &xs[s][q & 1][brow], d);
    if (q + 1 < UPW) {
      stage_x(q + 1, xr);
      if (q + 2 < UPW) {
        load_x(q + 2, xr);
        load_w(q + 2, wv[q & 1]);
      }
    }
  }
  // partial tiles to LDS: lane (g, j) holds rows 4g..4g+3 of column j
  if (li < 8) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[s][16 * t + 4 * lg + r][li] = d[t][r];
  }
  __syncthreads();
  float sum[kOut];
#pragma unroll
  for (int e = 0; e < kOut; ++e) {
    const int o = threadIdx.x + e * SK * kWave;
    const int orow = o >> 3, ocol = o & 7;
    const int64_t r = row_base + orow;
    sum[e] = 0.0f;
    if (o < kRows * 8 && ocol < m && r < n) {
      sum[e] = part[0][orow][ocol];
#pragma unroll
      for (int w = 1; w < SK; ++w) sum[e] += part[w][orow][ocol];
      if constexpr (SPLIT == 0) y[static_cast<int64_t>(ocol) * n + r] = sum[e] * (sc[e] * kCodeUnitInv);
      if constexpr (SPLIT == 2)
        __hip_atomic_fetch_add(y + static_cast<int64_t>(ocol) * n + r, sum[e] * (sc[e] * kCodeUnitInv),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if constexpr (SPLIT == 1) {
    unsigned long long* acc = sp.acc + static_cast<int64_t>(blockIdx.x) * (kRows * 8);
#pragma unroll
    for (int e = 0; e < kOut; ++e) {
      const int o = threadIdx.x + e * SK * kWave;
      const int64_t r = row_base + (o >> 3);
      float total;
      if (o < kRows * 8 && (o & 7) < m && r < n && splitk_add(acc + o, sum[e], sp.S, total))
        y[static_cast<int64_t>(o & 7) * n + r] = total * (sc[e] * kCodeUnitInv);
    }
  }
}

template <int CPL, int G, int R, int M>
void launch_rows_cfg(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                     hipStream_t stream) {
  const int64_t rows_per_block = static_cast<int64_t>(G) * R;
  const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL((ternary_gemm_rows_kernel<CPL, G, R, M>), grid, dim3(G * kWave), 0, stream,
                     reinterpret_cast<const uint4*>(packed), scale, n, k, words_per_row(k) / 4, x, y);
}

template <int SK, int T, int UPW, int MP>
void launch_mfma_mp(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x, int m,
                    float* y, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((n + 16 * T - 1) / (16 * T)));
  hipLaunchKernelGGL((ternary_gemm_mfma_kernel<SK, T, UPW, MP, 0>), grid, dim3(SK * kWave), 0, stream,
                     reinterpret_cast<const uint4*>(packed), scale, n, k, words_per_row(k) / 4, x, m, y,
                     SplitK{nullptr, 1});
}

// MP = m rounded up to 2, 4 or 8: the activation rows one x slice holds.
template <int SK, int T, int UPW>
void launch_mfma_cfg(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x, int m,
                     float* y, hipStream_t stream) {
  if (m <= 2) launch_mfma_mp<SK, T, UPW, 2>(packed, scale, n, k, x, m, y, stream);
  else if (m <= 4) launch_mfma_mp<SK, T, UPW, 4>(packed, scale, n, k, x, m, y, stream);
  else launch_mfma_mp<SK, T, UPW, 8>(packed, scale, n, k, x, m, y, stream);
}

template <int M>
void launch_small(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                  hipStream_t stream) {
  const int64_t rows_per_block = kGemvWaves * kRowsPerWave;
  const dim3 grid(static_cast<unsigned>((n + rows_per_block - 1) / rows_per_block));
  hipLaunchKernelGGL(ternary_gemm_small_kernel<M>, grid, dim3(kGemvWaves * kWave), 0, stream, packed, scale, n, k,
                     words_per_row(k), x, y);
}

// Split-K launches: grid (row blocks, slices). A row block's accumulators
// follow those of the row blocks before it, 8 bytes per output.
template <int SK, int T, int UPW, int MP>
hipError_t launch_mfma_split_mp(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                                int m, float* y, void* ws, int64_t ws_bytes, hipStream_t stream) {
  const int64_t units = (words_per_row(k) / 4 + 3) / 4;
  const int64_t nrb = (n + 16 * T - 1) / (16 * T);
  const int slices = static_cast<int>((units + SK * UPW - 1) / (SK * UPW));
  if (slices > 15 || 8 * nrb * (16 * T * 8) > ws_bytes) return hipErrorInvalidValue;
  hipLaunchKernelGGL((ternary_gemm_mfma_kernel<SK, T, UPW, MP, 1>), dim3(static_cast<unsigned>(nrb), slices),
                     dim3(SK * kWave), 0, stream, reinterpret_cast<const uint4*>(packed), scale, n, k,
                     words_per_row(k) / 4, x, m, y, SplitK{static_cast<unsigned long long*>(ws), slices});
  return hipGetLastError();
}

template <int SK, int T, int UPW>
hipError_t launch_mfma_split(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                             int m, float* y, void* ws, int64_t ws_bytes, hipStream_t stream) {
  if (m <= 2) return launch_mfma_split_mp<SK, T, UPW, 2>(packed, scale, n, k, x, m, y, ws, ws_bytes, stream);
  if (m <= 4) return launch_mfma_split_mp<SK, T, UPW, 4>(packed, scale, n, k, x, m, y, ws, ws_bytes, stream);
  return launch_mfma_split_mp<SK, T, UPW, 8>(packed, scale, n, k, x, m, y, ws, ws_bytes, stream);
}

// Two K-slices added onto a zeroed y (SPLIT = 2).
template <int SK, int T, int UPW, int MP>
void launch_mfma_split2_mp(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                           int m, float* y, hipStream_t stream) {
  const int64_t units = (words_per_row(k) / 4 + 3) / 4;
  const unsigned slices = static_cast<unsigned>((units + SK * UPW - 1) / (SK * UPW));
  hipLaunchKernelGGL((ternary_gemm_mfma_kernel<SK, T, UPW, MP, 2>),
                     dim3(static_cast<unsigned>((n + 16 * T - 1) / (16 * T)), slices), dim3(SK * kWave), 0, stream,
                     reinterpret_cast<const uint4*>(packed), scale, n, k, words_per_row(k) / 4, x, m, y,
                     SplitK{nullptr, static_cast<int>(slices)});
}

}  // namespace

bool ternary_split2_applies(int64_t n, int64_t k, int m, const uint16_t* x) {
  const int64_t units = (words_per_row(k) / 4 + 3) / 4;  // 256-column units
  return k % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15u) == 0 && m >= 2 && m <= 8 && units > 16 &&
         units <= 48 && n > 0;
}

hipError_t launch_ternary_gemm_split2(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                                      const uint16_t* x, int m, float* y, hipStream_t stream) {
  if (!ternary_split2_applies(n, k, m, x)) return hipErrorInvalidValue;
  // 32-row blocks, 8 waves of 3 units: slices of 24 units (6,144 columns)
  if (m <= 2) launch_mfma_split2_mp<8, 2, 3, 2>(packed, scale, n, k, x, m, y, stream);
  else if (m <= 4) launch_mfma_split2_mp<8, 2, 3, 4>(packed, scale, n, k, x, m, y, stream);
  else launch_mfma_split2_mp<8, 2, 3, 8>(packed, scale, n, k, x, m, y, stream);
  return hipGetLastError();
}

int64_t splitk_workspace_bytes(int64_t n, int64_t /*k*/) {
  // one 8-byte accumulator per output of a row block (at most 8 activation
  // rows, row blocks of at most 64 rows)
  return 8 * 8 * (n + 64);
}

hipError_t launch_ternary_gemm_splitk(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                                      const uint16_t* x, int m, float* y, void* ws, int64_t ws_bytes,
                                      hipStream_t stream) {
  const bool fast = k % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
  const int64_t units = (words_per_row(k) / 4 + 3) / 4;  // 256-column units
  // Split where graph-timed sweeps on MI355X measured it faster than the
  // plain dispatch (pools of 36 matrices, m = 2..8, both orders; us plain /
  // split): n <= 2,048 at every m (1,024 x 12,288: 5.01 / 4.10 at m = 2,
  // 6.80 / 4.21 at m = 8; 2,048 x 12,288: 5.09 / 4.84 and 7.01 / 5.43;
  // 1,024 x 16,384: 5.79 / 4.64 and 8.34 / 6.37), and 4,096 x 12,288 from
  // m = 5 (6.66 / 6.59 at m = 5, 7.42 / 6.85 at m = 8; 5.38 / 6.02 at m = 2).
  // 4,096 x 16,384 stays unsplit (9.21 / 9.94 at m = 8). Slices of 12, 24 and
  // 24 units for n <= 1,024, <= 2,048 and beyond. One activation row, K of
  // one 4,096-column slice and everything else run unsplit.
  if (!fast || m == 1 || units <= 16 || k > kSplitMaxK)
    return launch_ternary_gemm_small(packed, scale, n, k, x, m, y, stream);
  if (n <= 1024) return launch_mfma_split<12, 1, 1>(packed, scale, n, k, x, m, y, ws, ws_bytes, stream);
  if (n <= 2048) return launch_mfma_split<12, 1, 2>(packed, scale, n, k, x, m, y, ws, ws_bytes, stream);
  if (n <= 4096 && units <= 48 && m >= 5)
    return launch_mfma_split<8, 2, 3>(packed, scale, n, k, x, m, y, ws, ws_bytes, stream);
  return launch_ternary_gemm_small(packed, scale, n, k, x, m, y, stream);
}

hipError_t launch_ternary_gemv(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                               const uint16_t* x, float* y, hipStream_t stream) {
  // One K-slice is 64 lanes x 64 codes = 4,096 columns.
  const int64_t slices = (words_per_row(k) / 4 + kWave - 1) / kWave;
  if (k % 8 != 0 || (reinterpret_cast<uintptr_t>(x) & 15u) != 0 || slices > 4) {
    const dim3 grid(static_cast<unsigned>((n + 15) / 16));
    hipLaunchKernelGGL(ternary_gemv_generic_kernel, grid, dim3(4 * kWave), 0, stream,
                       reinterpret_cast<const uint4*>(packed), scale, n, k, words_per_row(k) / 4, x, y);
    return hipGetLastError();
  }
  // Launch shapes from graph-timed sweeps on MI355X (rotating weight pools
  // larger than the Infinity Cache); weight loads are non-temporal (each byte
  // is read once per call).
  const bool big = n >= 2048;
  switch (slices) {
    case 1:
      if (n >= 8192) launch_gemv_cfg<1, 4, 3>(packed, scale, n, k, x, y, stream);
      else if (big) launch_gemv_cfg<1, 4, 2>(packed, scale, n, k, x, y, stream);
      else launch_gemv_cfg<1, 4, 1>(packed, scale, n, k, x, y, stream);
      break;
    case 2:
      if (big) launch_gemv_cfg<2, 4, 2>(packed, scale, n, k, x, y, stream);
      else launch_gemv_cfg<2, 4, 1>(packed, scale, n, k, x, y, stream);
      break;
    case 3:
      if (big) launch_gemv_cfg<3, 8, 1>(packed, scale, n, k, x, y, stream);
      else launch_gemv_cfg<3, 4, 1>(packed, scale, n, k, x, y, stream);
      break;
    default:
      if (big) launch_gemv_cfg<4, 8, 1>(packed, scale, n, k, x, y, stream);
      else launch_gemv_cfg<4, 4, 1>(packed, scale, n, k, x, y, stream);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_ternary_gemm_small(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                                     const uint16_t* x, int m, float* y, hipStream_t stream) {
  if (m == 1) return launch_ternary_gemv(packed, scale, n, k, x, y, stream);
  const int64_t cpl = (words_per_row(k) / 4 + kWave - 1) / kWave;  // chunks per lane of the M-row kernel
  const bool fast = k % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
  // Shared decode on the VALU where it beat the matrix cores in graph-timed
  // sweeps on MI355X: M = 2 and 3 for K <= 4,096 and N < 2,048 (k, v).
  if (fast && (m == 2 || m == 3) && cpl == 1 && n < 2048) {
    if (m == 2) launch_rows_cfg<1, 4, 1, 2>(packed, scale, n, k, x, y, stream);
    else launch_rows_cfg<1, 4, 1, 3>(packed, scale, n, k, x, y, stream);
    return hipGetLastError();
  }
  const int64_t units = (words_per_row(k) / 4 + 3) / 4;  // 256-column units
  if (fast && units <= 64) {
    // Launch shapes from graph-timed sweeps on MI355X at M = 2..8, clocks
    // settled, each shape timed in both orders. More tiles per workgroup
    // (each activation column reused by more rows) beat more waves down to
    // about 192-256 workgroups. n = 12,288 (re-swept with the shared-shift
    // decode): 3 tiles of 4 waves at m = 2 (5.08 us), of 8 waves from m = 3
    // (5.11 / 5.21 / 5.67 us at m = 3 / 4 / 8, against 5.26-5.32 / 5.35-5.37 /
    // 5.73-5.80 for 4 or 16 waves); the q|k|v pack, n = 6,144: 2 tiles (4.45 us at m = 4), one tile
    // of 16 waves at m = 2 (4.25 us); n < 5,120: one tile, 8 waves (q 3.39 /
    // 3.55 / 3.52 / 3.96 us at m = 2 / 3 / 4 / 8; 16 waves 3.48-3.73); K =
    // 8,192: 8 waves (4.69 / 5.50 us at m = 4 / 8); K = 12,288: 8 waves up to
    // m = 4 (5.33 / 6.08 us at m = 2 / 4), 12 beyond (7.36 us at m = 8).
    if (units <= 16) {
      if (n >= 8192 && m == 2) launch_mfma_mp<4, 3, 4, 2>(packed, scale, n, k, x, m, y, stream);
      else if (n >= 8192) launch_mfma_cfg<8, 3, 2>(packed, scale, n, k, x, m, y, stream);
      else if (n >= 5120 && m == 2) launch_mfma_mp<16, 1, 1, 2>(packed, scale, n, k, x, m, y, stream);
      else if (n >= 5120 && m <= 4) launch_mfma_mp<4, 2, 4, 4>(packed, scale, n, k, x, m, y, stream);
      else if (n >= 5120) launch_mfma_mp<4, 2, 4, 8>(packed, scale, n, k, x, m, y, stream);
      else launch_mfma_cfg<8, 1, 2>(packed, scale, n, k, x, m, y, stream);
    } else if (units <= 32) {
      launch_mfma_cfg<8, 1, 4>(packed, scale, n, k, x, m, y, stream);
    } else if (units <= 48 && m == 2) {
      launch_mfma_mp<8, 1, 6, 2>(packed, scale, n, k, x, m, y, stream);
    } else if (units <= 48 && m <= 4) {
      launch_mfma_mp<8, 1, 6, 4>(packed, scale, n, k, x, m, y, stream);
    } else if (units <= 48) {
      launch_mfma_mp<12, 1, 4, 8>(packed, scale, n, k, x, m, y, stream);
    } else {
      launch_mfma_cfg<8, 1, 8>(packed, scale, n, k, x, m, y, stream);  // K <= 16,384
    }
    return hipGetLastError();
  }
  switch (m) {
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
