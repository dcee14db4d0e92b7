// Device helpers shared by the gfx950 kernels of libpackedbitgemv.
//
// Decoding follows the packed layout declared in include/packed_bit_gemv.h:
// a word shifted left by 2t and masked with 0xC000C000 holds two fp16 values
// 2*c[2t] and 2*c[2t+1] (nonzero flag in the top exponent bit, sign in the
// fp16 sign bit). One v_dot2 then adds or subtracts two fp16 activations (or
// skips them for a zero code) into an fp32 sum; the factor 2 is folded into
// the per-row scale. Products 2 * c * x are exact in fp32. On gfx950 the
// shift and the mask each issue at about half the cost of a rotate, which is
// why the fields sit at the top of each 16-bit half.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pbg {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr uint32_t kPairMask = 0xC000C000u;
constexpr float kCodeUnitInv = 0.5f;  // undoes the factor 2 of a decoded code
constexpr int kWave = 64;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// Operand t (0..7) of a word: codes 2t and 2t+1 as fp16 2*c.
__device__ __forceinline__ uint32_t code_pair(uint32_t w, int t) { return (w << (2 * t)) & kPairMask; }

// Sum over the 16 codes of one word against 8 fp16 activation pairs
// (xp[t] holds x[2t] in the low half and x[2t+1] in the high half).
__device__ __forceinline__ float word_dot(uint32_t w, const uint32_t* xp, float acc) {
#pragma unroll
  for (int t = 0; t < 8; ++t) acc = dot2(code_pair(w, t), xp[t], acc);
  return acc;
}

// Two words shifted left by S in one 64-bit shift (v_lshlrev_b64 issues at the
// cost of a 32-bit shift). For S <= 14 the bits carried from the low word into
// the high word land below bit S, where kPairMask clears them, so both halves
// decode exactly as separate 32-bit shifts would.
template <int S>
__device__ __forceinline__ uint64_t shl64(uint64_t v) {
  static_assert(S > 0 && S <= 14, "carried bits must stay below the code fields");
  uint64_t r;
  asm("v_lshlrev_b64 %0, %1, %2" : "=v"(r) : "n"(S), "v"(v));
  return r;
}

// Operands t of the words (w0, w1) packed as w1:w0.
template <int T>
__device__ __forceinline__ void pair_ops(uint64_t w, uint32_t& op0, uint32_t& op1) {
  if constexpr (T == 0) {
    op0 = static_cast<uint32_t>(w) & kPairMask;
    op1 = static_cast<uint32_t>(w >> 32) & kPairMask;
  } else {
    const uint64_t s = shl64<2 * T>(w);
    op0 = static_cast<uint32_t>(s) & kPairMask;
    op1 = static_cast<uint32_t>(s >> 32) & kPairMask;
  }
}

// Step T of a chunk: operand T of each of the four words, then step T + 1.
// Each step's operands die at once, so only a few decode registers are live
// at any time. One accumulator chain: with several waves per SIMD the
// dependent dot2s cost no issue slots, while split accumulators would cost a
// zeroing move and a combining add each per chunk.
template <int T>
__device__ __forceinline__ void chunk_steps(uint64_t lo, uint64_t hi, const uint32_t* xp, float& a) {
  uint32_t o0, o1, o2, o3;
  pair_ops<T>(lo, o0, o1);
  pair_ops<T>(hi, o2, o3);
  a = dot2(o0, xp[T], a);
  a = dot2(o1, xp[8 + T], a);
  a = dot2(o2, xp[16 + T], a);
  a = dot2(o3, xp[24 + T], a);
  if constexpr (T < 7) chunk_steps<T + 1>(lo, hi, xp, a);
}

// acc + the sum over one 16-byte chunk (4 words, 64 codes) against 32
// activation pairs.
__device__ __forceinline__ float chunk_dot(const uint4& w, const uint32_t* xp, float acc) {
  chunk_steps<0>(static_cast<uint64_t>(w.y) << 32 | w.x, static_cast<uint64_t>(w.w) << 32 | w.z, xp, acc);
  return acc;
}

// M activation rows at once: operand t of the four words is decoded once and
// feeds one dot2 per activation row (xp[m] holds row m's 32 pairs).
template <int M, int T>
__device__ __forceinline__ void chunk_steps_m(uint64_t lo, uint64_t hi, const uint32_t (*xp)[32], float* a) {
  uint32_t o0, o1, o2, o3;
  pair_ops<T>(lo, o0, o1);
  pair_ops<T>(hi, o2, o3);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    a[m] = dot2(o0, xp[m][T], a[m]);
    a[m] = dot2(o1, xp[m][8 + T], a[m]);
    a[m] = dot2(o2, xp[m][16 + T], a[m]);
    a[m] = dot2(o3, xp[m][24 + T], a[m]);
  }
  if constexpr (T < 7) chunk_steps_m<M, T + 1>(lo, hi, xp, a);
}

// Matrix-core A operands of half H (0 or 1) of a 16-byte chunk: a[w] holds
// codes 8H .. 8H + 7 of word w (operands 4H .. 4H + 3) as eight fp16 2*c.
// Each 64-bit shift serves two words, as in chunk_steps.
template <int H>
__device__ __forceinline__ void chunk_half_ops(const uint4& c, uint4 (&a)[4]) {
  const uint64_t lo = static_cast<uint64_t>(c.y) << 32 | c.x;
  const uint64_t hi = static_cast<uint64_t>(c.w) << 32 | c.z;
  uint32_t o[4][4];
  pair_ops<4 * H + 0>(lo, o[0][0], o[1][0]);
  pair_ops<4 * H + 0>(hi, o[2][0], o[3][0]);
  pair_ops<4 * H + 1>(lo, o[0][1], o[1][1]);
  pair_ops<4 * H + 1>(hi, o[2][1], o[3][1]);
  pair_ops<4 * H + 2>(lo, o[0][2], o[1][2]);
  pair_ops<4 * H + 2>(hi, o[2][2], o[3][2]);
  pair_ops<4 * H + 3>(lo, o[0][3], o[1][3]);
  pair_ops<4 * H + 3>(hi, o[2][3], o[3][3]);
#pragma unroll
  for (int w = 0; w < 4; ++w) a[w] = make_uint4(o[w][0], o[w][1], o[w][2], o[w][3]);
}

// z * sigmoid(z) with the hardware reciprocal (1 ulp), for the SwiGLU
// epilogues: h is rounded to fp16 right after, so an IEEE division would only
// cost instructions.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

typedef _Float16 mfma_half8_t __attribute__((ext_vector_type(8)));
typedef float mfma_float4_t __attribute__((ext_vector_type(4)));

// Half H of one 256-column unit on the matrix cores, for T 16-row tiles:
// tile t's lane chunk wv[t], and xb the lane's 8 B slots of the unit, where
// slot v holds the activation columns of codes 8 (v % 2) .. 8 (v % 2) + 7 of
// word v / 2. Word w's half H is multiplied by slot 2w + H; the 4 slots are
// read once for all T tiles.
template <int H, int T>
__device__ __forceinline__ void mfma_unit_half(const uint4 (&wv)[T], const uint4* xb, mfma_float4_t (&d)[T]) {
  mfma_half8_t b[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) b[w] = __builtin_bit_cast(mfma_half8_t, xb[2 * w + H]);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    uint4 a[4];
    chunk_half_ops<H>(wv[t], a);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      d[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mfma_half8_t, a[w]), b[w], d[t], 0, 0, 0);
  }
}

// acc[m] += the chunk's sum against activation row m.
template <int M>
__device__ __forceinline__ void chunk_dot_m(const uint4& w, const uint32_t (*xp)[32], float* acc) {
  chunk_steps_m<M, 0>(static_cast<uint64_t>(w.y) << 32 | w.x, static_cast<uint64_t>(w.w) << 32 | w.z, xp, acc);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// v if keep, else zero, by AND masks (no branch, no register copies).
__device__ __forceinline__ uint4 masked(const uint4& v, bool keep) {
  const uint32_t k = keep ? 0xFFFFFFFFu : 0u;
  return make_uint4(v.x & k, v.y & k, v.z & k, v.w & k);
}

// 16-byte load marked non-temporal (streamed once, not kept in the caches).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t as_u32(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float as_f32(uint32_t v) { return __builtin_bit_cast(float, v); }

// DPP row rotate: lane j of every 16-lane row reads lane (j - N) mod 16 of
// that row.
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return as_f32(__builtin_amdgcn_update_dpp(0u, as_u32(v), 0x120 + N, 0xF, 0xF, false));
}

// Sum of a value over the 16 lanes of each row; every lane gets its row's sum.
__device__ __forceinline__ float row_sum16(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v;
}

// Transposed reduction of four per-lane partial sums over the 64 lanes of a
// wave. Afterwards lane 0 holds sum(a), lane 32 sum(b), lane 16 sum(c) and
// lane 48 sum(d). Uses the gfx950 lane swaps: permlane32_swap exchanges lanes
// 32..63 of its first operand with lanes 0..31 of its second, permlane16_swap
// exchanges the odd 16-lane rows of the first with the even rows of the
// second. Needs all 64 lanes active.
__device__ __forceinline__ float wave_reduce4(float a, float b, float c, float d) {
  auto ab = __builtin_amdgcn_permlane32_swap(as_u32(a), as_u32(b), false, false);
  auto cd = __builtin_amdgcn_permlane32_swap(as_u32(c), as_u32(d), false, false);
  float p = as_f32(ab[0]) + as_f32(ab[1]);  // lanes 0..31: a folded, 32..63: b folded
  float q = as_f32(cd[0]) + as_f32(cd[1]);  // lanes 0..31: c folded, 32..63: d folded
  auto pq = __builtin_amdgcn_permlane16_swap(as_u32(p), as_u32(q), false, false);
  float s = as_f32(pq[0]) + as_f32(pq[1]);  // rows: a, c, b, d (16 lanes each)
  return row_sum16(s);
}

// Lane of wave_reduce4's result for operand i (0 = a, 1 = b, 2 = c, 3 = d),
// and the inverse map (-1 for lanes that hold no result).
__device__ __forceinline__ int reduce4_slot(int lane) {
  return lane == 0 ? 0 : lane == 32 ? 1 : lane == 16 ? 2 : lane == 48 ? 3 : -1;
}

// Greedy-argmax key of a logit: the order-preserving image of the fp32 bits
// in the high half and (2^32 - 1 - row) in the low half, so that the largest
// key is the largest logit and, among equal logits, the lowest row. -0 is
// keyed as +0 (the two compare equal, so the lower row must win between
// them). Logits are finite.
__device__ __forceinline__ unsigned long long argmax_key(float v, int64_t row) {
  uint32_t b = __builtin_bit_cast(uint32_t, v);
  b = b == 0x80000000u ? 0u : b;
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<unsigned long long>(ord) << 32) | static_cast<uint32_t>(0xFFFFFFFFu - static_cast<uint32_t>(row));
}

__device__ __forceinline__ float argmax_key_logit(unsigned long long key) {
  const uint32_t ord = static_cast<uint32_t>(key >> 32);
  return __builtin_bit_cast(float, (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

__device__ __forceinline__ int32_t argmax_key_row(unsigned long long key) {
  return static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key));
}

// K split across workgroups. The S slices of a row block meet in one 64-bit
// integer per output (in a caller workspace that is zero between calls):
// each slice adds its fp32 partial, converted exactly to fixed point with 23
// fractional bits, shifted left by 4, plus 1 in the low 4 bits, which count
// arrivals. The add that brings the count to S returns the sum of all the
// others, so that workgroup adds its own, writes the output and sets the
// accumulator back to zero; no workgroup waits for another. Integer addition
// is exact and associative, so the result does not depend on the order of
// arrival: it is the exact sum of the S fp32 partials, rounded once to fp32.
// Exactness of the conversion: products 2 * c * x of fp16 activations are
// multiples of 2^-23, so every fp32 partial of them is too, and |partial| <
// 2^31 for K <= 16,384 (|x| <= 65,504), so partial * 2^23 is an integer below
// 2^54 and S <= 15 of them, times 16, stay below 2^63.
struct SplitK {
  unsigned long long* acc;  // [row blocks][outputs per workgroup]
  int S;                    // slices, 1 <= S <= 15
};

constexpr float kFix = 8388608.0f;  // 2^23

// Adds `partial` (slice contribution to one output) to its accumulator; true
// for the last of the S slices, which then gets the full sum in `total`.
__device__ __forceinline__ bool splitk_add(unsigned long long* acc, float partial, int S, float& total) {
  const long long fx = static_cast<long long>(partial * kFix);
  const unsigned long long add = (static_cast<unsigned long long>(fx) << 4) + 1ull;
  const unsigned long long before = __hip_atomic_fetch_add(acc, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (static_cast<int>(before & 15ull) != S - 1) return false;
  __hip_atomic_store(acc, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  total = static_cast<float>(static_cast<long long>(before + add) >> 4) * (1.0f / kFix);
  return true;
}

// Loads x[base .. base+2*NPAIR-1] as NPAIR fp16 pairs; columns >= k read 0.
template <int NPAIR>
__device__ __forceinline__ void load_x_pairs(const uint16_t* __restrict__ x, int64_t k, int64_t base,
                                             uint32_t* xp) {
  static_assert(NPAIR % 4 == 0, "whole 16-byte groups");
  const uint16_t* p = x + base;
  if (base + 2 * NPAIR <= k && (reinterpret_cast<uintptr_t>(p) & 15u) == 0) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < NPAIR / 4; ++i) {
      uint4 v = q[i];
      xp[4 * i + 0] = v.x;
      xp[4 * i + 1] = v.y;
      xp[4 * i + 2] = v.z;
      xp[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < NPAIR; ++e) {
      const int64_t c0 = base + 2 * e;
      uint32_t lo = c0 < k ? p[2 * e] : 0u;
      uint32_t hi = c0 + 1 < k ? p[2 * e + 1] : 0u;
      xp[e] = lo | (hi << 16);
    }
  }
}

}  // namespace pbg
