// Device helpers of the 3-bit (five-level) layout, shared by ternary3.hip
// and ffn3.hip. The layout is declared in include/packed_bit_gemv.h: a row is
// its sign/nonzero plane in the 2-bit layout followed by a magnitude plane
// (bit 16h + 8i + t of a 32-code word for code 16i + 2t + h).
//
// Decode of a pair of codes (2t, 2t + 1) of a sign/nonzero word w: the 2-bit
// operand (w << 2t) & 0xC000C000 gives fp16 +-2 or 0, and the pair's two
// magnitude bits OR-ed in at bits 10 and 26 (the fp16 exponent's lowest bit)
// turn +-2 into +-4, so the operand is 2c and one v_dot2 adds, subtracts or
// skips c * x exactly. For a 16-byte chunk w0..w3 of the sign/nonzero plane
// and its two magnitude words M = m1:m0, pair t of w0 and w2 sits at bits 10
// and 26 of the two halves of M << (10 - t), and of w1 and w3 in those of M
// shifted left by 2 - t (right by t - 2).
#pragma once

#include "pbg_device.hpp"

namespace pbg {

constexpr uint32_t kMagMask = 0x04000400u;

// 64-bit right shift (v_lshrrev_b64), the counterpart of shl64.
template <int S>
__device__ __forceinline__ uint64_t shr64(uint64_t v) {
  static_assert(S > 0 && S < 32, "shift within one word");
  uint64_t r;
  asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "n"(S), "v"(v));
  return r;
}

// M = m1:m0 shifted so that pair T of sign/nonzero words 0 (low half) and 2
// (high half) sits at bits 10 and 26.
template <int T>
__device__ __forceinline__ uint64_t mag_a(uint64_t m) {
  return shl64<10 - T>(m);
}

// The same for words 1 (low half) and 3 (high half).
template <int T>
__device__ __forceinline__ uint64_t mag_b(uint64_t m) {
  if constexpr (T < 2) return shl64<2 - T>(m);
  else if constexpr (T == 2) return m;
  else return shr64<T - 2>(m);
}

__device__ __forceinline__ uint32_t with_mag(uint32_t op2, uint32_t mag_src) { return (mag_src & kMagMask) | op2; }

// Magnitude bits of pair t of sign/nonzero word i (0 or 1) of a magnitude
// word, placed at bits 10 and 26 (bits 8i + t and 16 + 8i + t move there).
__device__ __forceinline__ uint32_t mag_pair(uint32_t mw, int i, int t) {
  const int s = 10 - 8 * i - t;
  return (s >= 0 ? mw << s : mw >> -s) & kMagMask;
}

// Step T of a chunk: the four operands of pair T, each fed to its dot2.
template <int T>
__device__ __forceinline__ void chunk3_steps(uint64_t lo, uint64_t hi, uint64_t m, const uint32_t* xp, float& a) {
  uint32_t o0, o1, o2, o3;
  pair_ops<T>(lo, o0, o1);
  pair_ops<T>(hi, o2, o3);
  const uint64_t ma = mag_a<T>(m), mb = mag_b<T>(m);
  a = dot2(with_mag(o0, static_cast<uint32_t>(ma)), xp[T], a);
  a = dot2(with_mag(o1, static_cast<uint32_t>(mb)), xp[8 + T], a);
  a = dot2(with_mag(o2, static_cast<uint32_t>(ma >> 32)), xp[16 + T], a);
  a = dot2(with_mag(o3, static_cast<uint32_t>(mb >> 32)), xp[24 + T], a);
  if constexpr (T < 7) chunk3_steps<T + 1>(lo, hi, m, xp, a);
}

// acc + the sum over one chunk (64 codes: sign/nonzero words w, magnitude
// words mg) against 32 activation pairs.
__device__ __forceinline__ float chunk3_dot(const uint4& w, const uint2& mg, const uint32_t* xp, float acc) {
  chunk3_steps<0>(static_cast<uint64_t>(w.y) << 32 | w.x, static_cast<uint64_t>(w.w) << 32 | w.z,
                  static_cast<uint64_t>(mg.y) << 32 | mg.x, xp, acc);
  return acc;
}

__device__ __forceinline__ uint2 load_nt2(const uint2* p) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v[0], v[1]);
}

// The four operands of pair T of a chunk (sign/nonzero words lo = w1:w0 and
// hi = w3:w2, magnitude words m = m1:m0) with their magnitude bits.
template <int T>
__device__ __forceinline__ void pair3_ops(uint64_t lo, uint64_t hi, uint64_t m, uint32_t& o0, uint32_t& o1,
                                          uint32_t& o2, uint32_t& o3) {
  pair_ops<T>(lo, o0, o1);
  pair_ops<T>(hi, o2, o3);
  const uint64_t ma = mag_a<T>(m), mb = mag_b<T>(m);
  o0 = with_mag(o0, static_cast<uint32_t>(ma));
  o1 = with_mag(o1, static_cast<uint32_t>(mb));
  o2 = with_mag(o2, static_cast<uint32_t>(ma >> 32));
  o3 = with_mag(o3, static_cast<uint32_t>(mb >> 32));
}

// Matrix-core A operands of half H of a chunk: a[w] holds codes 8H .. 8H + 7
// of word w as eight fp16 2*c (chunk_half_ops of the 2-bit layout with the
// magnitude bits OR-ed in; every 64-bit shift serves two words).
template <int H>
__device__ __forceinline__ void chunk3_half_ops(const uint4& c, const uint2& mg, uint4 (&a)[4]) {
  const uint64_t lo = static_cast<uint64_t>(c.y) << 32 | c.x;
  const uint64_t hi = static_cast<uint64_t>(c.w) << 32 | c.z;
  const uint64_t m = static_cast<uint64_t>(mg.y) << 32 | mg.x;
  uint32_t o[4][4];
  pair3_ops<4 * H + 0>(lo, hi, m, o[0][0], o[1][0], o[2][0], o[3][0]);
  pair3_ops<4 * H + 1>(lo, hi, m, o[0][1], o[1][1], o[2][1], o[3][1]);
  pair3_ops<4 * H + 2>(lo, hi, m, o[0][2], o[1][2], o[2][2], o[3][2]);
  pair3_ops<4 * H + 3>(lo, hi, m, o[0][3], o[1][3], o[2][3], o[3][3]);
#pragma unroll
  for (int w = 0; w < 4; ++w) a[w] = make_uint4(o[w][0], o[w][1], o[w][2], o[w][3]);
}

// Half H of one 256-column unit for T tiles (mfma_unit_half of the 2-bit
// layout): word w's half H against B slot 2w + H, the 4 slots read once.
template <int H, int T>
__device__ __forceinline__ void mfma3_unit_half(const uint4 (&wv)[T], const uint2 (&mv)[T], const uint4* xb,
                                                mfma_float4_t (&d)[T]) {
  mfma_half8_t b[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) b[w] = __builtin_bit_cast(mfma_half8_t, xb[2 * w + H]);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    uint4 a[4];
    chunk3_half_ops<H>(wv[t], mv[t], a);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      d[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mfma_half8_t, a[w]), b[w], d[t], 0, 0, 0);
  }
}

}  // namespace pbg
