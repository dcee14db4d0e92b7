// C ABI of libpackedbitgemv: argument validation (before any HIP call),
// error mapping and dispatch to the gfx950 launchers.
#include "packed_bit_gemv.h"
#include "pbg_internal.hpp"

namespace {

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

bool bad_nk(int64_t n, int64_t k) { return n < 1 || n > PBG_MAX_N || k < 1 || k > PBG_MAX_K; }

bool bad_m(int64_t m) { return m < 1 || m > PBG_MAX_M; }

bool bad_ffn(int64_t d_model, int64_t d_ff) {
  return d_model < 8 || d_model > PBG_FFN_MAX_MODEL || d_model % 8 != 0 || bad_nk(d_ff, d_model);
}

// True when earlier work on this thread left a HIP error pending. Such an
// error is the caller's: it is left in place (not cleared) and the call
// enqueues nothing. hipErrorNotReady from a completion query is a status,
// not a failure, and is cleared so that the launch check below sees only
// this call's errors.
bool pending_error() {
  const hipError_t e = hipPeekAtLastError();
  if (e == hipSuccess) return false;
  if (e == hipErrorNotReady) {
    (void)hipGetLastError();
    return false;
  }
  return true;
}

int finish(hipError_t launch_status) {
  if (launch_status != hipSuccess) return PBG_ERR_HIP;
  return hipGetLastError() == hipSuccess ? PBG_OK : PBG_ERR_HIP;
}

}  // namespace

extern "C" {

int pbg_abi_version(void) { return PBG_ABI_VERSION; }

const char* pbg_strerror(int code) {
  switch (code) {
    case PBG_OK: return "ok";
    case PBG_ERR_NULL: return "a required pointer is NULL";
    case PBG_ERR_SHAPE: return "n, k or m out of range";
    case PBG_ERR_ALIGN: return "a pointer lacks its required alignment";
    case PBG_ERR_CODE: return "pack input held a value outside {-1, 0, +1}";
    case PBG_ERR_HIP: return "a HIP launch or copy failed";
    case PBG_ERR_WORKSPACE: return "workspace smaller than the call needs";
    default: return "unknown error code";
  }
}

int64_t pbg_words_per_row(int64_t k) { return pbg::words_per_row(k); }

int pack_ternary(const int8_t* codes, int64_t n, int64_t k, uint32_t* packed, int32_t* row_sum, int64_t* stats,
                 int64_t* stats_host, hipStream_t stream) {
  if (!codes || !packed || !row_sum || !stats) return PBG_ERR_NULL;
  if (bad_nk(n, k)) return PBG_ERR_SHAPE;
  if (misaligned(packed, 16) || misaligned(row_sum, 4) || misaligned(stats, 8)) return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  int rc = finish(pbg::launch_pack(codes, n, k, packed, row_sum, stats, stream));
  if (rc != PBG_OK || !stats_host) return rc;
  if (hipMemcpyAsync(stats_host, stats, 4 * sizeof(int64_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return PBG_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return PBG_ERR_HIP;
  return stats_host[3] > 0 ? PBG_ERR_CODE : PBG_OK;
}

int64_t pbg_words_per_row3(int64_t k) { return pbg::words_per_row3(k); }

int pack_ternary3(const int8_t* codes, int64_t n, int64_t k, uint32_t* packed, int32_t* row_sum, int64_t* stats,
                  int64_t* stats_host, hipStream_t stream) {
  if (!codes || !packed || !row_sum || !stats) return PBG_ERR_NULL;
  if (bad_nk(n, k)) return PBG_ERR_SHAPE;
  if (misaligned(packed, 16) || misaligned(row_sum, 4) || misaligned(stats, 8)) return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  int rc = finish(pbg::launch_pack3(codes, n, k, packed, row_sum, stats, stream));
  if (rc != PBG_OK || !stats_host) return rc;
  if (hipMemcpyAsync(stats_host, stats, 6 * sizeof(int64_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return PBG_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return PBG_ERR_HIP;
  return stats_host[5] > 0 ? PBG_ERR_CODE : PBG_OK;
}

int ternary3_gemv(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                  hipStream_t stream) {
  if (!packed || !scale || !x || !y) return PBG_ERR_NULL;
  if (bad_nk(n, k)) return PBG_ERR_SHAPE;
  if (misaligned(packed, 16) || misaligned(scale, 4) || misaligned(x, 2) || misaligned(y, 4)) return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_ternary3_gemv(packed, scale, n, k, x, y, stream));
}

int ternary3_gemm_small(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                        int64_t m, float* y, hipStream_t stream) {
  if (!packed || !scale || !x || !y) return PBG_ERR_NULL;
  if (bad_nk(n, k) || bad_m(m)) return PBG_ERR_SHAPE;
  if (misaligned(packed, 16) || misaligned(scale, 4) || misaligned(x, 2) || misaligned(y, 4)) return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_ternary3_gemm_small(packed, scale, n, k, x, static_cast<int>(m), y, stream));
}

int ternary_gemv(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x, float* y,
                 hipStream_t stream) {
  if (!packed || !scale || !x || !y) return PBG_ERR_NULL;
  if (bad_nk(n, k)) return PBG_ERR_SHAPE;
  if (misaligned(packed, 16) || misaligned(scale, 4) || misaligned(x, 2) || misaligned(y, 4)) return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_ternary_gemv(packed, scale, n, k, x, y, stream));
}

int ternary_gemm_small(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                       int64_t m, float* y, hipStream_t stream) {
  if (!packed || !scale || !x || !y) return PBG_ERR_NULL;
  if (bad_nk(n, k) || bad_m(m)) return PBG_ERR_SHAPE;
  if (misaligned(packed, 16) || misaligned(scale, 4) || misaligned(x, 2) || misaligned(y, 4)) return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_ternary_gemm_small(packed, scale, n, k, x, static_cast<int>(m), y, stream));
}

int64_t pbg_splitk_workspace_bytes(int64_t n, int64_t k) {
  if (bad_nk(n, k)) return 0;
  return pbg::splitk_workspace_bytes(n, k);
}

int ternary_gemm_splitk(const uint32_t* packed, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                        int64_t m, float* y, void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  if (!packed || !scale || !x || !y || !workspace) return PBG_ERR_NULL;
  if (bad_nk(n, k) || bad_m(m)) return PBG_ERR_SHAPE;
  if (misaligned(packed, 16) || misaligned(scale, 4) || misaligned(x, 2) || misaligned(y, 4) ||
      misaligned(workspace, 256))
    return PBG_ERR_ALIGN;
  if (workspace_bytes < pbg::splitk_workspace_bytes(n, k)) return PBG_ERR_WORKSPACE;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_ternary_gemm_splitk(packed, scale, n, k, x, static_cast<int>(m), y, workspace,
                                                workspace_bytes, stream));
}

int int8_head_gemv(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, int64_t m,
                   float* y, hipStream_t stream) {
  if (!w || !scale || !x || !y) return PBG_ERR_NULL;
  if (bad_nk(n, k) || bad_m(m)) return PBG_ERR_SHAPE;
  if (misaligned(w, 16) || misaligned(scale, 4) || misaligned(x, 2) || misaligned(y, 4)) return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_int8_head(w, scale, n, k, x, static_cast<int>(m), y, stream));
}

int int8_head_argmax(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x, int64_t m,
                     uint64_t* keys, int32_t* token, float* logit, hipStream_t stream) {
  if (!w || !scale || !x || !keys || !token) return PBG_ERR_NULL;
  if (bad_nk(n, k) || bad_m(m)) return PBG_ERR_SHAPE;
  if (misaligned(w, 16) || misaligned(scale, 4) || misaligned(x, 2) || misaligned(keys, 8) || misaligned(token, 4) ||
      misaligned(logit, 4))
    return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_int8_head_argmax(w, scale, n, k, x, static_cast<int>(m),
                                             reinterpret_cast<unsigned long long*>(keys), token, logit, stream));
}

int int8_head_argmax_noalloc(const int8_t* w, const float* scale, int64_t n, int64_t k, const uint16_t* x,
                             int64_t m, int32_t* token, float* logit, hipStream_t stream) {
  if (!w || !scale || !x || !token) return PBG_ERR_NULL;
  if (bad_nk(n, k) || bad_m(m)) return PBG_ERR_SHAPE;
  if (misaligned(w, 16) || misaligned(scale, 4) || misaligned(x, 2) || misaligned(token, 4) || misaligned(logit, 4))
    return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_int8_head_argmax_noalloc(w, scale, n, k, x, static_cast<int>(m), token, logit, stream));
}

int int8_embedding_gather(const int8_t* table, const float* scale, int64_t n, int64_t k, const int32_t* tokens,
                          int64_t m, float* out, hipStream_t stream) {
  if (!table || !scale || !tokens || !out) return PBG_ERR_NULL;
  if (bad_nk(n, k) || m < 1 || m > PBG_MAX_N || pbg::embedding_blocks(m, k) > (1LL << 23)) return PBG_ERR_SHAPE;
  if (misaligned(scale, 4) || misaligned(tokens, 4) || misaligned(out, 4)) return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_embedding_gather(table, scale, n, k, tokens, m, out, stream));
}

int pbg_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink) return PBG_ERR_NULL;
  if (bytes < 16 || bytes > PBG_STREAM_READ_MAX_BYTES || bytes % 16 != 0) return PBG_ERR_SHAPE;
  if (misaligned(src, 16) || misaligned(sink, 4)) return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_stream_read(src, bytes, sink, stream));
}

int ternary_swiglu_gate_up(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                           const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, uint16_t* h,
                           hipStream_t stream) {
  if (!gate_packed || !gate_scale || !up_packed || !up_scale || !x || !h) return PBG_ERR_NULL;
  if (bad_ffn(d_model, d_ff)) return PBG_ERR_SHAPE;
  if (misaligned(gate_packed, 16) || misaligned(up_packed, 16) || misaligned(gate_scale, 4) ||
      misaligned(up_scale, 4) || misaligned(x, 16) || misaligned(h, 16))
    return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_swiglu_gate_up(gate_packed, gate_scale, up_packed, up_scale, d_model, d_ff, x, h, stream));
}

int ternary_ffn_swiglu(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                       const float* up_scale, const uint32_t* down_packed, const float* down_scale, int64_t d_model,
                       int64_t d_ff, const uint16_t* x, uint16_t* h, float* y, hipStream_t stream) {
  if (!gate_packed || !gate_scale || !up_packed || !up_scale || !down_packed || !down_scale || !x || !h || !y)
    return PBG_ERR_NULL;
  if (bad_ffn(d_model, d_ff)) return PBG_ERR_SHAPE;
  if (misaligned(gate_packed, 16) || misaligned(up_packed, 16) || misaligned(down_packed, 16) ||
      misaligned(gate_scale, 4) || misaligned(up_scale, 4) || misaligned(down_scale, 4) || misaligned(x, 16) ||
      misaligned(h, 16) || misaligned(y, 4))
    return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_ffn_swiglu(gate_packed, gate_scale, up_packed, up_scale, down_packed, down_scale, d_model,
                                       d_ff, x, h, y, stream));
}

int ternary_swiglu_gate_up_small(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                                 const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, int64_t m,
                                 uint16_t* h, hipStream_t stream) {
  if (!gate_packed || !gate_scale || !up_packed || !up_scale || !x || !h) return PBG_ERR_NULL;
  if (bad_ffn(d_model, d_ff) || bad_m(m)) return PBG_ERR_SHAPE;
  if (misaligned(gate_packed, 16) || misaligned(up_packed, 16) || misaligned(gate_scale, 4) ||
      misaligned(up_scale, 4) || misaligned(x, 16) || misaligned(h, 16))
    return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_swiglu_gate_up_small(gate_packed, gate_scale, up_packed, up_scale, d_model, d_ff, x,
                                                 static_cast<int>(m), h, stream));
}

int ternary_ffn_swiglu_small(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                             const float* up_scale, const uint32_t* down_packed, const float* down_scale,
                             int64_t d_model, int64_t d_ff, const uint16_t* x, int64_t m, uint16_t* h, float* y,
                             hipStream_t stream) {
  if (!gate_packed || !gate_scale || !up_packed || !up_scale || !down_packed || !down_scale || !x || !h || !y)
    return PBG_ERR_NULL;
  if (bad_ffn(d_model, d_ff) || bad_m(m)) return PBG_ERR_SHAPE;
  if (misaligned(gate_packed, 16) || misaligned(up_packed, 16) || misaligned(down_packed, 16) ||
      misaligned(gate_scale, 4) || misaligned(up_scale, 4) || misaligned(down_scale, 4) || misaligned(x, 16) ||
      misaligned(h, 16) || misaligned(y, 4))
    return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_ffn_swiglu_small(gate_packed, gate_scale, up_packed, up_scale, down_packed, down_scale,
                                             d_model, d_ff, x, static_cast<int>(m), h, y, stream));
}

int ternary3_swiglu_gate_up(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                            const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, uint16_t* h,
                            hipStream_t stream) {
  if (!gate_packed || !gate_scale || !up_packed || !up_scale || !x || !h) return PBG_ERR_NULL;
  if (bad_ffn(d_model, d_ff)) return PBG_ERR_SHAPE;
  if (misaligned(gate_packed, 16) || misaligned(up_packed, 16) || misaligned(gate_scale, 4) ||
      misaligned(up_scale, 4) || misaligned(x, 16) || misaligned(h, 16))
    return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_swiglu3_gate_up(gate_packed, gate_scale, up_packed, up_scale, d_model, d_ff, x, h, stream));
}

int ternary3_ffn_swiglu(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                        const float* up_scale, const uint32_t* down_packed, const float* down_scale, int64_t d_model,
                        int64_t d_ff, const uint16_t* x, uint16_t* h, float* y, hipStream_t stream) {
  if (!gate_packed || !gate_scale || !up_packed || !up_scale || !down_packed || !down_scale || !x || !h || !y)
    return PBG_ERR_NULL;
  if (bad_ffn(d_model, d_ff)) return PBG_ERR_SHAPE;
  if (misaligned(gate_packed, 16) || misaligned(up_packed, 16) || misaligned(down_packed, 16) ||
      misaligned(gate_scale, 4) || misaligned(up_scale, 4) || misaligned(down_scale, 4) || misaligned(x, 16) ||
      misaligned(h, 16) || misaligned(y, 4))
    return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_ffn3_swiglu(gate_packed, gate_scale, up_packed, up_scale, down_packed, down_scale, d_model,
                                        d_ff, x, h, y, stream));
}

int ternary3_swiglu_gate_up_small(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                                  const float* up_scale, int64_t d_model, int64_t d_ff, const uint16_t* x, int64_t m,
                                  uint16_t* h, hipStream_t stream) {
  if (!gate_packed || !gate_scale || !up_packed || !up_scale || !x || !h) return PBG_ERR_NULL;
  if (bad_ffn(d_model, d_ff) || bad_m(m)) return PBG_ERR_SHAPE;
  if (misaligned(gate_packed, 16) || misaligned(up_packed, 16) || misaligned(gate_scale, 4) ||
      misaligned(up_scale, 4) || misaligned(x, 16) || misaligned(h, 16))
    return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_swiglu3_gate_up_small(gate_packed, gate_scale, up_packed, up_scale, d_model, d_ff, x,
                                                  static_cast<int>(m), h, stream));
}

int ternary3_ffn_swiglu_small(const uint32_t* gate_packed, const float* gate_scale, const uint32_t* up_packed,
                              const float* up_scale, const uint32_t* down_packed, const float* down_scale,
                              int64_t d_model, int64_t d_ff, const uint16_t* x, int64_t m, uint16_t* h, float* y,
                              hipStream_t stream) {
  if (!gate_packed || !gate_scale || !up_packed || !up_scale || !down_packed || !down_scale || !x || !h || !y)
    return PBG_ERR_NULL;
  if (bad_ffn(d_model, d_ff) || bad_m(m)) return PBG_ERR_SHAPE;
  if (misaligned(gate_packed, 16) || misaligned(up_packed, 16) || misaligned(down_packed, 16) ||
      misaligned(gate_scale, 4) || misaligned(up_scale, 4) || misaligned(down_scale, 4) || misaligned(x, 16) ||
      misaligned(h, 16) || misaligned(y, 4))
    return PBG_ERR_ALIGN;
  if (pending_error()) return PBG_ERR_HIP;
  return finish(pbg::launch_ffn3_swiglu_small(gate_packed, gate_scale, up_packed, up_scale, down_packed, down_scale,
                                              d_model, d_ff, x, static_cast<int>(m), h, y, stream));
}

}  // extern "C"
