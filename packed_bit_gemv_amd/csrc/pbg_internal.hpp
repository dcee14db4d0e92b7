// Host-side launchers behind the C ABI. Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pbg {

hipError_t launch_pack(const int8_t* codes, int64_t n, int64_t k, uint32_t* packed, int32_t* row_sum,
                       int64_t* stats, hipStream_t stream);

hipError_t launch_ternary_gemv(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                               const uint16_t* x, float* y, hipStream_t stream);

hipError_t launch_ternary_gemm_small(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                                     const uint16_t* x, int m, float* y, hipStream_t stream);

// ternary_gemm_small with K split across workgroups (1 <= m <= 8); the
// slices meet in `ws` (splitk_workspace_bytes(n, k) bytes, zero before the
// first call, left ready by every call). Shapes that are not split run the
// plain dispatch.
constexpr int64_t kSplitMaxK = 16384;
int64_t splitk_workspace_bytes(int64_t n, int64_t k);
hipError_t launch_ternary_gemm_splitk(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                                      const uint16_t* x, int m, float* y, void* ws, int64_t ws_bytes,
                                      hipStream_t stream);

// Small-M GEMM split over K into at most two slices that add s * partial to y
// with fp32 atomics; y must hold +0 in every element on entry (the FFN block
// clears it in its gate|up launch). Applies when ternary_split2_applies.
bool ternary_split2_applies(int64_t n, int64_t k, int m, const uint16_t* x);
hipError_t launch_ternary_gemm_split2(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                                      const uint16_t* x, int m, float* y, hipStream_t stream);

hipError_t launch_int8_head(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                            int m, float* y, hipStream_t stream);

hipError_t launch_int8_head_argmax(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                                   int m, unsigned long long* keys, int32_t* token, float* logit, hipStream_t stream);

// int8_head_argmax with its keys in the library's own device array (allocates nothing).
hipError_t launch_int8_head_argmax_noalloc(const int8_t* w, const float* scale, int64_t n, int64_t k,
                                           const uint16_t* x, int m, int32_t* token, float* logit,
                                           hipStream_t stream);

hipError_t launch_embedding_gather(const int8_t* table, const float* scale, int64_t n, int64_t k,
                                   const int32_t* tokens, int64_t m, float* out, hipStream_t stream);

hipError_t launch_swiglu_gate_up(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                 const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, uint16_t* h,
                                 hipStream_t stream);

hipError_t launch_ffn_swiglu(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                             const float* up_scale, const uint32_t* down, const float* down_scale, int64_t d_model,
                             int64_t d_ff, const uint16_t* x, uint16_t* h, float* y, hipStream_t stream);

// The same two for 1 <= m <= 8 activation rows: x [m][d_model], h [m][d_ff], y [m][d_model].
hipError_t launch_swiglu_gate_up_small(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                       const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x,
                                       int m, uint16_t* h, hipStream_t stream);

hipError_t launch_ffn_swiglu_small(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                   const float* up_scale, const uint32_t* down, const float* down_scale,
                                   int64_t d_model, int64_t d_ff, const uint16_t* x, int m, uint16_t* h, float* y,
                                   hipStream_t stream);

// One read of `bytes` (a multiple of 16) from 16-byte aligned src, folded into sink.
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

// Workgroups one embedding gather launches (the grid must stay below 2^31 / 256).
int64_t embedding_blocks(int64_t m, int64_t k);

inline int64_t words_per_row(int64_t k) { return k <= 0 ? 0 : 4 * ((k + 63) / 64); }

// The 3-bit variant: 12 words per 128 codes (sign/nonzero plane, then magnitude plane).
inline int64_t words_per_row3(int64_t k) { return k <= 0 ? 0 : 12 * ((k + 127) / 128); }

hipError_t launch_pack3(const int8_t* codes, int64_t n, int64_t k, uint32_t* packed, int32_t* row_sum,
                        int64_t* stats, hipStream_t stream);
hipError_t launch_ternary3_gemv(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                                float* y, hipStream_t stream);
hipError_t launch_ternary3_gemm_small(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                                      const uint16_t* x, int m, float* y, hipStream_t stream);
// The 3-bit form of ternary_split2_applies / launch_ternary_gemm_split2 (y +0 on entry).
bool ternary3_split2_applies(int64_t n, int64_t k, int m, const uint16_t* x);
hipError_t launch_ternary3_gemm_split2(const uint32_t* packed, const float* scale, int64_t n, int64_t k,
                                       const uint16_t* x, int m, float* y, hipStream_t stream);

// The SwiGLU block with 3-bit linears (d_model <= PBG_FFN_MAX_MODEL, 16-byte aligned x and h).
hipError_t launch_swiglu3_gate_up(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                  const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, uint16_t* h,
                                  hipStream_t stream);
hipError_t launch_ffn3_swiglu(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                              const float* up_scale, const uint32_t* down, const float* down_scale, int64_t d_model,
                              int64_t d_ff, const uint16_t* x, uint16_t* h, float* y, hipStream_t stream);
hipError_t launch_swiglu3_gate_up_small(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                        const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x,
                                        int m, uint16_t* h, hipStream_t stream);
hipError_t launch_ffn3_swiglu_small(const uint32_t* gate, const float* gate_scale, const uint32_t* up,
                                    const float* up_scale, const uint32_t* down, const float* down_scale,
                                    int64_t d_model, int64_t d_ff, const uint16_t* x, int m, uint16_t* h, float* y,
                                    hipStream_t stream);

}  // namespace pbg
