// ternary3_ffn_swiglu: the gated feed-forward block of one layer with its
// three linears in the 3-bit (five-level) layout (Neutrino-1 8B model page:
// geometry table, gated SwiGLU feed-forward with three linears; "Where the
// bytes live", the 3-bit coded lane and per-row scales).
//
//   launch 1   g = gate x, u = up x, h = fp16(silu(g) * u)  -> h
//   launch 2   y = down h (ternary3_gemv, or ternary3_gemm_small for m rows)
//
// The kernels are those of the 2-bit block (ffn.hip) with 3-bit rows: besides
// its 16-byte sign/nonzero chunk, every lane loads the chunk's two magnitude
// words, and the decode ORs the magnitude bits into each operand
// (pbg_device3.hpp). A row is 6 * chunks words: 4 per chunk in the
// sign/nonzero plane, then 2 per chunk in the magnitude plane.
#include "pbg_device.hpp"
#include "pbg_device3.hpp"
#include "pbg_internal.hpp"

namespace pbg {
namespace {

// M = 1 launch shape: 2 row pairs per wave, 4 waves (8.76-8.84 us at d_ff =
// 12,288 in a graph-timed sweep, against 9.8-10.1 us for 1 or 4 pairs and 2
// or 8 waves).
constexpr int kPairs3 = 2;     // row pairs per wave (M = 1)
constexpr int kFfn3Waves = 4;  // waves per workgroup (M = 1)

// M = 1 (d_model <= 4,096: one chunk per lane). A wave owns R consecutive row
// pairs (gate row r and up row r) and lane l reads sign/nonzero chunk l and
// its magnitude words of each; x is staged through LDS chunk-major. The 2R
// sums are reduced four at a time, one lane swap puts each gate sum beside
// its up sum, and lanes 0 and 16 form and store h of two pairs.
template <int R, int G>
__global__ __launch_bounds__(G* kWave) void swiglu3_gate_up_kernel(
    const uint32_t* __restrict__ gate, const float* __restrict__ gate_scale, const uint32_t* __restrict__ up,
    const float* __restrict__ up_scale, int64_t d_model, int64_t d_ff, int64_t chunks, const uint16_t* x,
    uint16_t* __restrict__ h) {
  static_assert(R == 1 || R == 2 || R == 4, "R pairs fill whole reductions");
  constexpr int kThreads = G * kWave;
  constexpr int kX = kWave * 8;  // 16-byte activation groups of one 4,096-column slice
  __shared__ uint4 buf[kX];      // group (c, q) at q * 64 + c
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t groups = d_model / 8;
  const int64_t row_words = 6 * chunks;
  const int64_t r0 = (static_cast<int64_t>(blockIdx.x) * G + wave) * R;
  const uint4* xg = reinterpret_cast<const uint4*>(x);

  constexpr int kXPer = (kX + kThreads - 1) / kThreads;
  uint4 xv[kXPer];
#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int gi = threadIdx.x + i * kThreads;
    xv[i] = xg[gi < groups ? gi : 0];
  }
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");  // activation loads queue ahead of the weight loads
  __builtin_amdgcn_sched_barrier(0);
  const int64_t cl = lane < chunks ? lane : chunks - 1;  // lanes past the row reread its last chunk (x is 0 there)
  uint4 wg[R], wu[R];
  uint2 mg[R], mu[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t r = r0 + i < d_ff ? r0 + i : d_ff - 1;
    const uint32_t* grow = gate + r * row_words;
    const uint32_t* urow = up + r * row_words;
    wg[i] = load_nt(reinterpret_cast<const uint4*>(grow) + cl);
    mg[i] = load_nt2(reinterpret_cast<const uint2*>(grow + 4 * chunks) + cl);
    wu[i] = load_nt(reinterpret_cast<const uint4*>(urow) + cl);
    mu[i] = load_nt2(reinterpret_cast<const uint2*>(urow + 4 * chunks) + cl);
  }
  constexpr int kRed = (2 * R + 3) / 4;
  const int half = (lane >> 4) & 1;
  float sg[kRed], su[kRed];
#pragma unroll
  for (int q = 0; q < kRed; ++q) {
    const int64_t rs = r0 + (2 * q + half < R ? 2 * q + half : 0);
    sg[q] = gate_scale[rs < d_ff ? rs : d_ff - 1];
    su[q] = up_scale[rs < d_ff ? rs : d_ff - 1];
  }
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int i = 0; i < kXPer; ++i) {
    const int gi = threadIdx.x + i * kThreads;
    if (gi < kX) buf[(gi & 7) * kWave + (gi >> 3)] = masked(xv[i], gi < groups);
  }
  __syncthreads();
  uint32_t xp[32];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 v = buf[q * kWave + lane];
    xp[4 * q + 0] = v.x;
    xp[4 * q + 1] = v.y;
    xp[4 * q + 2] = v.z;
    xp[4 * q + 3] = v.w;
  }

  float acc[4 * kRed];  // per reduction q: gate and up sums of pair 2q, then of pair 2q + 1
#pragma unroll
  for (int i = 0; i < 4 * kRed; ++i) acc[i] = 0.0f;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    acc[4 * (i / 2) + 2 * (i % 2)] = chunk3_dot(wg[i], mg[i], xp, 0.0f);
    acc[4 * (i / 2) + 2 * (i % 2) + 1] = chunk3_dot(wu[i], mu[i], xp, 0.0f);
  }
  float red[kRed];
#pragma unroll
  for (int q = 0; q < kRed; ++q) red[q] = wave_reduce4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  // gate sums of pairs 2q, 2q + 1 in lanes 0 and 16, up sums in lanes 32 and 48
#pragma unroll
  for (int q = 0; q < kRed; ++q) {
    const auto gu = __builtin_amdgcn_permlane32_swap(as_u32(red[q]), as_u32(red[q]), false, false);
    const float g = red[q], u = as_f32(gu[1]);
    const float hv = silu(g * (sg[q] * kCodeUnitInv)) * (u * (su[q] * kCodeUnitInv));
    const int pair = 2 * q + half;
    if ((lane & 47) == 0 && pair < R && r0 + pair < d_ff)
      h[r0 + pair] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(hv));
  }
}

// 2 <= M <= 8 on the matrix cores: the 2-bit block's small-M kernel with
// 3-bit rows. A 16-row tile holds 8 gate rows (lanes i < 8) and the same 8 up
// rows (lanes i >= 8), so the accumulator holds both sums of 8 pairs for every
// activation column; x is loaded a whole line at a time and transposed
// through a per-wave LDS slice; SK waves split the units.
template <int SK, int T, int UPW, int MP>
__global__ __launch_bounds__(SK* kWave) void swiglu3_gate_up_mfma_kernel(
    const uint32_t* __restrict__ gate, const float* __restrict__ gate_scale, const uint32_t* __restrict__ up,
    const float* __restrict__ up_scale, int64_t d_model, int64_t d_ff, int64_t chunks, const uint16_t* __restrict__ x,
    int m, uint16_t* __restrict__ h, float* __restrict__ yz, int64_t yz_n) {
  constexpr int kPairsWg = 8 * T;  // gate/up row pairs of the workgroup
  __shared__ float part[SK][16 * T][8];
  const int lane = threadIdx.x & (kWave - 1);
  const int s = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int li = lane & 15, lg = lane >> 4;
  const int64_t pair_base = static_cast<int64_t>(blockIdx.x) * kPairsWg;
  const int64_t groups = d_model / 8;
  const int64_t row_words = 6 * chunks;
  const uint4* xg = reinterpret_cast<const uint4*>(x);
  const uint32_t* src = li < 8 ? gate : up;

  // outputs (pair, column) o = threadIdx.x + e * SK * 64: pair o / 8, column o % 8
  constexpr int kOut = (kPairsWg * 8 + SK * kWave - 1) / (SK * kWave);
  float sg[kOut], su[kOut];
#pragma unroll
  for (int e = 0; e < kOut; ++e) {
    const int o = threadIdx.x + e * SK * kWave;
    int64_t r = pair_base + (o < kPairsWg * 8 ? o >> 3 : 0);
    r = r < d_ff ? r : d_ff - 1;
    sg[e] = gate_scale[r];
    su[e] = up_scale[r];
  }
  constexpr int kXLoads = MP / 2;
  constexpr int kSlots = 33;  // 16-byte slots per row and unit, one of padding
  __shared__ uint4 xs[SK][2][MP * kSlots];
  const int xrow = li >> 3, xg8 = li & 7;
  auto load_x = [&](int q, uint4 (&xr)[kXLoads]) {
    const int64_t u = s + static_cast<int64_t>(SK) * q;
#pragma unroll
    for (int a = 0; a < kXLoads; ++a) {
      const int row = 2 * a + xrow;
      const int64_t gi = 32 * u + 8 * lg + xg8;
      xr[a] = xg[row < m && gi < groups ? static_cast<int64_t>(row) * groups + gi : 0];
    }
  };
  auto stage_x = [&](int q, const uint4 (&xr)[kXLoads]) {
    const int64_t gi = 32 * (s + static_cast<int64_t>(SK) * q) + 8 * lg + xg8;
#pragma unroll
    for (int a = 0; a < kXLoads; ++a)
      xs[s][q & 1][(2 * a + xrow) * kSlots + 8 * lg + xg8] = masked(xr[a], gi < groups);
  };
  auto load_w = [&](int q, uint4 (&wv)[T], uint2 (&mv)[T]) {
    const int64_t c = 4 * (s + static_cast<int64_t>(SK) * q) + lg;
    const int64_t cc = c < chunks ? c : chunks - 1;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t r = pair_base + 8 * t + (li & 7);
      const uint32_t* row = src + (r < d_ff ? r : d_ff - 1) * row_words;
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
  // partial tiles to LDS: lane (g, j) holds tile rows 4g..4g+3 of column j
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
    const int p = o >> 3, j = o & 7;
    const int64_t r = pair_base + p;
    if (o < kPairsWg * 8 && j < m && r < d_ff) {
      const int tr = 16 * (p >> 3) + (p & 7);  // gate row of the pair in its tile; up row is tr + 8
      float g = part[0][tr][j], uu = part[0][tr + 8][j];
#pragma unroll
      for (int w = 1; w < SK; ++w) {
        g += part[w][tr][j];
        uu += part[w][tr + 8][j];
      }
      const float hv = silu(g * (sg[e] * kCodeUnitInv)) * (uu * (su[e] * kCodeUnitInv));
      h[static_cast<int64_t>(j) * d_ff + r] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(hv));
    }
  }
  // the block's y, cleared for the down linear's slices to add onto (yz_n = 0: none)
  const int64_t nth = static_cast<int64_t>(gridDim.x) * (SK * kWave);
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * (SK * kWave) + threadIdx.x; i < yz_n; i += nth) yz[i] = 0.0f;
}

template <int SK, int T, int UPW, int MP>
void launch_gate_up3_mp(const uint32_t* gate, const float* gate_scale, const uint32_t* up, const float* up_scale,
                        int64_t d_model, int64_t d_ff, const uint16_t* x, int m, uint16_t* h, float* yz, int64_t yz_n,
                        hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((d_ff + 8 * T - 1) / (8 * T)));
  hipLaunchKernelGGL((swiglu3_gate_up_mfma_kernel<SK, T, UPW, MP>), grid, dim3(SK * kWave), 0, stream, gate,
                     gate_scale, up, up_scale, d_model, d_ff, words_per_row3(d_model) / 6, x, m, h, yz, yz_n);
}

// MP = m rounded up to 2, 4 or 8.
template <int SK, int T, int UPW>
void launch_gate_up3_mfma(const uint32_t* gate, const float* gate_scale, const uint32_t* up, const float* up_scale,
                          int64_t d_model, int64_t d_ff, const uint16_t* x, int m, uint16_t* h, float* yz,
                          int64_t yz_n, hipStream_t stream) {
  if (m <= 2)
    launch_gate_up3_mp<SK, T, UPW, 2>(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, yz, yz_n, stream);
  else if (m <= 4)
    launch_gate_up3_mp<SK, T, UPW, 4>(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, yz, yz_n, stream);
  else launch_gate_up3_mp<SK, T, UPW, 8>(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, yz, yz_n, stream);
}

// 2 <= m <= 8: the matrix-core gate|up launch by shape; yz_n > 0 also clears
// yz[0 .. yz_n).
hipError_t gate_up3_small(const uint32_t* gate, const float* gate_scale, const uint32_t* up, const float* up_scale,
                          int64_t d_model, int64_t d_ff, const uint16_t* x, int m, uint16_t* h, float* yz,
                          int64_t yz_n, hipStream_t stream) {
  // d_model <= 4,096: at most 16 units of 256 columns. Launch shapes from a
  // graph-timed sweep on MI355X at d_ff = 12,288 (pools of 36 layers, both
  // orders): three tiles of 4 waves, 13.2 / 13.4 / 14.4 us at m = 2 / 4 / 8,
  // within 0.15 us of the best of nine shapes at every m (six tiles of 8
  // waves, the 2-bit block's shape from m = 3: 13.8 / 14.0 / 14.5 us).
  if (d_ff >= 8192) {
    launch_gate_up3_mfma<4, 3, 4>(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, yz, yz_n, stream);
  } else {
    launch_gate_up3_mfma<4, 2, 4>(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, yz, yz_n, stream);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_swiglu3_gate_up(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                  const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, uint16_t* h,
                                  hipStream_t stream) {
  constexpr int64_t kRowsPerBlock = static_cast<int64_t>(kPairs3) * kFfn3Waves;
  const dim3 grid(static_cast<unsigned>((d_ff + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((swiglu3_gate_up_kernel<kPairs3, kFfn3Waves>), grid, dim3(kFfn3Waves * kWave), 0, stream, gate,
                     gate_scale, up, up_scale, d_model, d_ff, words_per_row3(d_model) / 6, x, h);
  return hipGetLastError();
}

hipError_t launch_ffn3_swiglu(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                              const float* up_scale, const uint32_t* down, const float* down_scale, int64_t d_model,
                              int64_t d_ff, const uint16_t* x, uint16_t* h, float* y, hipStream_t stream) {
  const hipError_t e = launch_swiglu3_gate_up(gate, gate_scale, up, up_scale, d_model, d_ff, x, h, stream);
  if (e != hipSuccess) return e;
  return launch_ternary3_gemv(down, down_scale, d_model, d_ff, h, y, stream);
}

hipError_t launch_swiglu3_gate_up_small(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                        const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x,
                                        int m, uint16_t* h, hipStream_t stream) {
  if (m == 1) return launch_swiglu3_gate_up(gate, gate_scale, up, up_scale, d_model, d_ff, x, h, stream);
  return gate_up3_small(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, nullptr, 0, stream);
}

hipError_t launch_ffn3_swiglu_small(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                    const float* up_scale, const uint32_t* down, const float* down_scale,
                                    int64_t d_model, int64_t d_ff, const uint16_t* x, int m, uint16_t* h, float* y,
                                    hipStream_t stream) {
  if (m == 1)
    return launch_ffn3_swiglu(gate, gate_scale, up, up_scale, down, down_scale, d_model, d_ff, x, h, y, stream);
  // as the 2-bit block: down split over K in two slices that add onto y,
  // which the gate|up launch clears
  if (ternary3_split2_applies(d_model, d_ff, m, h)) {
    const hipError_t e = gate_up3_small(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, y,
                                        static_cast<int64_t>(m) * d_model, stream);
    if (e != hipSuccess) return e;
    return launch_ternary3_gemm_split2(down, down_scale, d_model, d_ff, h, m, y, stream);
  }
  const hipError_t e = gate_up3_small(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, nullptr, 0, stream);
  if (e != hipSuccess) return e;
  return launch_ternary3_gemm_small(down, down_scale, d_model, d_ff, h, m, y, stream);
}

}  // namespace pbg
