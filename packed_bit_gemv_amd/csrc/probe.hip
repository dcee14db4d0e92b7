// pbg_stream_read: a measurement helper beside the decode path. It reads a
// byte range once, with the same 16-byte non-temporal loads the GEMVs use
// (each wave-wide load covers 1 KiB of consecutive bytes, up to four loads in
// flight per lane), and does nothing else with the data but fold it by XOR. Its
// duration is what one launch that streams the same bytes can at best reach,
// the practical ceiling for the GEMVs: the Neutrino-1 8B model page
// (introduction) puts single-stream decode speed down to the bytes moved per
// token.
//
// The fold makes every load observable, so none can be optimised away, and
// lets a test check that each byte was read: XOR-ed over the sink, it equals
// the XOR of all 32-bit words of the range.
#include "packed_bit_gemv.h"
#include "pbg_device.hpp"
#include "pbg_internal.hpp"

namespace pbg {
namespace {

constexpr int kSinkStride = 32;     // one sink slot per 128-byte line
constexpr int kSinkSlots = PBG_STREAM_READ_SINK_WORDS / kSinkStride;

// T threads per workgroup, each with U 16-byte chunks T apart.
template <int T, int U>
__global__ __launch_bounds__(T) void stream_read_kernel(const uint4* __restrict__ src, int64_t chunks,
                                                        uint32_t* __restrict__ sink) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * (T * U) + threadIdx.x;
  uint4 v[U];
  // every load is issued before the first use; chunks past the end re-read
  // the last one and are masked to zero
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + u * T;
    v[u] = load_nt(src + (i < chunks ? i : chunks - 1));
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint4 w = masked(v[u], base + u * T < chunks);
    acc ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  for (int off = kWave / 2; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t part[T / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < T / kWave; ++w) a ^= part[w];
    // slots on separate 128-byte lines, so that workgroups finishing together
    // do not queue on one address
    atomicXor(sink + (blockIdx.x % kSinkSlots) * kSinkStride, a);
  }
}

template <int T, int U>
hipError_t launch_read(const void* src, int64_t chunks, uint32_t* sink, hipStream_t stream) {
  const int64_t blocks = (chunks + T * U - 1) / (T * U);
  hipLaunchKernelGGL((stream_read_kernel<T, U>), dim3(static_cast<unsigned>(blocks)), dim3(T), 0, stream,
                     static_cast<const uint4*>(src), chunks, sink);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  // the fastest of the shapes swept on MI355X (graph of launches over a
  // rotating pool, settled clocks), as threads x loads per lane: 256 x 1
  // below 8 MiB (1 MB 2.33 us, 256 x 4: 2.45-2.69; 4.2 MB 2.74 us, 256 x 4:
  // 2.99), 256 x 4 up to 16 MiB (12.6 MB 3.86-3.90 us, 256 x 1: 4.03), 512 x 4
  // beyond (25.2 MB 5.60 us, 256 x 4: 5.74; 622 MB 91.0-91.3 us, 256 x 4:
  // 92.8-93.6); plain loads were 3-11 % slower than non-temporal ones
  const int64_t chunks = bytes / 16;
  if (bytes < (8LL << 20)) return launch_read<256, 1>(src, chunks, sink, stream);
  if (bytes < (16LL << 20)) return launch_read<256, 4>(src, chunks, sink, stream);
  return launch_read<512, 4>(src, chunks, sink, stream);
}

}  // namespace pbg
