// ternary_ffn_swiglu: the gated feed-forward block of one layer at M = 1
// (Neutrino-1 8B model page: geometry table, gated SwiGLU feed-forward with
// three linears; per-row scales, "Where the bytes live").
//
//   launch 1   g = gate x, u = up x, h = fp16(silu(g) * u)  -> h
//   launch 2   y = down h (the M = 1 GEMV of ternary.hip)   -> y
//
// Launch 1 reads gate and up (same K, same x) in one pass and forms h in its
// epilogue, so the gate and up outputs never reach memory. A single
// persistent launch with a grid-wide barrier between the two phases was
// measured slower on gfx950: the barrier, the exchange of h through memory
// and the down decode after the barrier cost more than the second launch.
//
// Work split of launch 1: a wave owns R consecutive row pairs (gate row r and
// up row r) and reads 16-byte chunk `lane` (64 codes) of each; x is staged
// through LDS like the M = 1 GEMV. The 2R row sums are reduced four at a time
// across the wave, one lane swap puts each gate sum beside its up sum, and
// two lanes per reduction form and store the fp16 results.
#include "pbg_device.hpp"
#include "pbg_internal.hpp"

namespace pbg {
namespace {

constexpr int kPairs = 2;      // row pairs per wave
constexpr int kFfnWaves = 4;   // waves per workgroup

// z * sigmoid(z) with the hardware reciprocal (1 ulp): h is rounded to fp16
// right after, so an IEEE division would only cost instructions.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

template <int R, int G>
__global__ __launch_bounds__(G* kWave) void swiglu_gate_up_kernel(
    const uint4* __restrict__ gate, const float* __restrict__ gate_scale, const uint4* __restrict__ up,
    const float* __restrict__ up_scale, int64_t d_model, int64_t d_ff, int64_t chunks, const uint16_t* x,
    uint16_t* __restrict__ h) {
  static_assert(R == 1 || R == 2 || R == 4, "R pairs fill whole reductions");
  constexpr int kThreads = G * kWave;
  constexpr int kX = kWave * 8;  // 16-byte activation groups of one 4,096-column slice
  __shared__ uint4 buf[kX];      // group (c, q) at q * 64 + c
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t groups = d_model / 8;
  const int64_t r0 = (static_cast<int64_t>(blockIdx.x) * G + wave) * R;  // first row pair
  const uint4* xg = reinterpret_cast<const uint4*>(x);

  // activations first, then every weight load of the wave
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
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t r = r0 + i < d_ff ? r0 + i : d_ff - 1;
    wg[i] = load_nt(gate + r * chunks + cl);
    wu[i] = load_nt(up + r * chunks + cl);
  }
  // lanes 0 and 16 form pairs 2q and 2q + 1 of reduction q (below); their scales
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
    acc[4 * (i / 2) + 2 * (i % 2)] = chunk_dot(wg[i], xp, 0.0f);
    acc[4 * (i / 2) + 2 * (i % 2) + 1] = chunk_dot(wu[i], xp, 0.0f);
  }
  float red[kRed];
#pragma unroll
  for (int q = 0; q < kRed; ++q) red[q] = wave_reduce4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);

  // wave_reduce4 leaves operands 0..3 in lanes 0, 32, 16, 48: the gate sums
  // of pairs 2q and 2q + 1 in lanes 0 and 16, their up sums in lanes 32 and
  // 48. One lane swap brings those to lanes 0 and 16 of a second register,
  // and lanes 0 and 16 form and store h of the two pairs.
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

template <int SK, int T, int UPW, int MP>
__global__ __launch_bounds__(SK* kWave) void swiglu_gate_up_mfma_kernel(
    const uint4* __restrict__ gate, const float* __restrict__ gate_scale, const uint4* __restrict__ up,
    const float* __restrict__ up_scale, int64_t d_model, int64_t d_ff, int64_t chunks, const uint16_t* __restrict__ x,
    int m, uint16_t* __restrict__ h) {
  typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
  typedef float float4_t __attribute__((ext_vector_type(4)));
  constexpr int kPairsWg = 8 * T;  // gate/up row pairs of the workgroup
  __shared__ float part[SK][16 * T][8];
  const int lane = threadIdx.x & (kWave - 1);
  const int s = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int li = lane & 15, lg = lane >> 4;
  const int64_t pair_base = static_cast<int64_t>(blockIdx.x) * kPairsWg;
  const int64_t groups = d_model / 8;
  const uint4* xg = reinterpret_cast<const uint4*>(x);
  const uint4* src = li < 8 ? gate : up;

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
  // x: line-wise loads staged through this wave's LDS slice, as in the
  // small-M GEMM
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
  auto load_w = [&](int q, uint4 (&wv)[T]) {
    const int64_t c = 4 * (s + static_cast<int64_t>(SK) * q) + lg;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int64_t r = pair_base + 8 * t + (li & 7);
      wv[t] = load_nt(src + (r < d_ff ? r : d_ff - 1) * chunks + (c < chunks ? c : chunks - 1));
    }
  };

  float4_t d[T];
#pragma unroll
  for (int t = 0; t < T; ++t) d[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  uint4 xr[kXLoads], wv[2][T];
  load_x(0, xr);
  load_w(0, wv[0]);
  stage_x(0, xr);
  if (UPW > 1) {
    load_x(1, xr);
    load_w(1, wv[1]);
  }
  const int brow = (li % MP) * kSlots + 8 * lg;
#pragma unroll
  for (int q = 0; q < UPW; ++q) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const half8_t b = __builtin_bit_cast(half8_t, xs[s][q & 1][brow + v]);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const uint32_t wd = (&wv[q & 1][t].x)[v >> 1];
        const int hh = v & 1;
        const uint4 ap = make_uint4(code_pair(wd, 4 * hh + 0), code_pair(wd, 4 * hh + 1), code_pair(wd, 4 * hh + 2),
                                    code_pair(wd, 4 * hh + 3));
        d[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ap), b, d[t], 0, 0, 0);
      }
    }
    if (q + 1 < UPW) {
      stage_x(q + 1, xr);
      if (q + 2 < UPW) {
        load_x(q + 2, xr);
        load_w(q + 2, wv[q & 1]);
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
}

template <int SK, int T, int UPW, int MP>
void launch_gate_up_mp(const uint32_t* gate, const float* gate_scale, const uint32_t* up, const float* up_scale,
                       int64_t d_model, int64_t d_ff, const uint16_t* x, int m, uint16_t* h, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((d_ff + 8 * T - 1) / (8 * T)));
  hipLaunchKernelGGL((swiglu_gate_up_mfma_kernel<SK, T, UPW, MP>), grid, dim3(SK * kWave), 0, stream,
                     reinterpret_cast<const uint4*>(gate), gate_scale, reinterpret_cast<const uint4*>(up), up_scale,
                     d_model, d_ff, words_per_row(d_model) / 4, x, m, h);
}

// MP = m rounded up to 2, 4 or 8: the activation rows one x slice holds.
template <int SK, int T, int UPW>
void launch_gate_up_mfma(const uint32_t* gate, const float* gate_scale, const uint32_t* up, const float* up_scale,
                         int64_t d_model, int64_t d_ff, const uint16_t* x, int m, uint16_t* h, hipStream_t stream) {
  if (m <= 2) launch_gate_up_mp<SK, T, UPW, 2>(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, stream);
  else if (m <= 4) launch_gate_up_mp<SK, T, UPW, 4>(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, stream);
  else launch_gate_up_mp<SK, T, UPW, 8>(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, stream);
}
}  // namespace

hipError_t launch_swiglu_gate_up(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                 const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, uint16_t* h,
                                 hipStream_t stream) {
  constexpr int64_t kRowsPerBlock = static_cast<int64_t>(kPairs) * kFfnWaves;
  const dim3 grid(static_cast<unsigned>((d_ff + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((swiglu_gate_up_kernel<kPairs, kFfnWaves>), grid, dim3(kFfnWaves * kWave), 0, stream,
                     reinterpret_cast<const uint4*>(gate), gate_scale, reinterpret_cast<const uint4*>(up), up_scale,
                     d_model, d_ff, words_per_row(d_model) / 4, x, h);
  return hipGetLastError();
}

hipError_t launch_ffn_swiglu(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                             const float* up_scale, const uint32_t* down, const float* down_scale, int64_t d_model,
                             int64_t d_ff, const uint16_t* x, uint16_t* h, float* y, hipStream_t stream) {
  const hipError_t e = launch_swiglu_gate_up(gate, gate_scale, up, up_scale, d_model, d_ff, x, h, stream);
  if (e != hipSuccess) return e;
  return launch_ternary_gemv(down, down_scale, d_model, d_ff, h, y, stream);
}

hipError_t launch_swiglu_gate_up_small(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                       const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x,
                                       int m, uint16_t* h, hipStream_t stream) {
  if (m == 1) return launch_swiglu_gate_up(gate, gate_scale, up, up_scale, d_model, d_ff, x, h, stream);
  // d_model <= 4,096: at most 16 units of 256 columns. Launch shapes from
  // graph-timed sweeps on MI355X at d_ff = 12,288: three tiles (24 pairs, 512
  // workgroups) of 4 waves up to m = 4 (7.7-8.2 us), six tiles of 8 waves
  // beyond (8.9 us at m = 8); four tiles took 9.3-10.6 us.
  if (d_ff >= 8192 && m <= 4) {
    launch_gate_up_mfma<4, 3, 4>(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, stream);
  } else if (d_ff >= 8192) {
    launch_gate_up_mp<8, 6, 2, 8>(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, stream);
  } else {
    launch_gate_up_mfma<4, 2, 4>(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, stream);
  }
  return hipGetLastError();
}

hipError_t launch_ffn_swiglu_small(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                   const float* up_scale, const uint32_t* down, const float* down_scale,
                                   int64_t d_model, int64_t d_ff, const uint16_t* x, int m, uint16_t* h, float* y,
                                   hipStream_t stream) {
  const hipError_t e = launch_swiglu_gate_up_small(gate, gate_scale, up, up_scale, d_model, d_ff, x, m, h, stream);
  if (e != hipSuccess) return e;
  return launch_ternary_gemm_small(down, down_scale, d_model, d_ff, h, m, y, stream);
}

}  // namespace pbg
