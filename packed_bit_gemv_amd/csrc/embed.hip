// int8_embedding_gather: out[i][j] = s_t * w_t[j] for token t = tokens[i] of the
// untied int8 input embedding with a per-row scale, read one row per token
// (Neutrino-1 8B model page, "Where the bytes live").
//
// The product of an fp32 scale and an int8 value is exact in fp64; it is
// rounded once to fp32. Token ids outside [0, n) produce a row of NaN.
#include "pbg_device.hpp"
#include "pbg_internal.hpp"

namespace pbg {
namespace {

constexpr int kEmbedThreads = 256;
constexpr int kEmbedCols = 4 * kEmbedThreads;  // columns per workgroup

__global__ __launch_bounds__(kEmbedThreads) void embedding_gather_kernel(const int8_t* __restrict__ table,
                                                                         const float* __restrict__ scale, int64_t n,
                                                                         int64_t k, const int32_t* __restrict__ tokens,
                                                                         int64_t col_blocks, float* __restrict__ out) {
  const int64_t i = blockIdx.x / col_blocks;
  const int64_t c0 = (blockIdx.x % col_blocks) * kEmbedCols + 4 * threadIdx.x;
  const int32_t t = tokens[i];
  float* o = out + i * k;
  const bool ok = t >= 0 && t < n;
  const double s = ok ? static_cast<double>(scale[t]) : 0.0;
  const int8_t* row = table + (ok ? static_cast<int64_t>(t) : 0) * k;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t c = c0 + j;
    if (c < k) o[c] = ok ? static_cast<float>(s * static_cast<double>(row[c])) : __builtin_nanf("");
  }
}

}  // namespace

hipError_t launch_embedding_gather(const int8_t* table, const float* scale, int64_t n, int64_t k,
                                   const int32_t* tokens, int64_t m, float* out, hipStream_t stream) {
  const int64_t col_blocks = (k + kEmbedCols - 1) / kEmbedCols;
  hipLaunchKernelGGL(embedding_gather_kernel, dim3(static_cast<unsigned>(m * col_blocks)), dim3(kEmbedThreads), 0,
                     stream, table, scale, n, k, tokens, col_blocks, out);
  return hipGetLastError();
}

int64_t embedding_blocks(int64_t m, int64_t k) { return m * ((k + kEmbedCols - 1) / kEmbedCols); }

}  // namespace pbg
