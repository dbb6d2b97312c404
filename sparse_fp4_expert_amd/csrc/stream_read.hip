// Measurement utility: a plain streaming read of a device buffer, the
// ceiling any HBM-bound kernel of this library can reach on the device (the
// published peak is the pin rate, not what a read stream achieves).  Not
// part of the MoE path.
#include "common.hpp"

namespace moesq {

constexpr int READ_THREADS = 256;
constexpr int READ_UNROLL = 8;   // 16-byte loads in flight per lane

// Every lane issues READ_UNROLL 16-byte loads before using any of them;
// grid-stride over the buffer; the XOR of all words goes to `sink` only when
// it equals an impossible marker, so the loads stay live.
__global__ __launch_bounds__(READ_THREADS) void stream_read_kernel(const uint4 *__restrict__ p,
                                                                   long long n16, uint32_t *sink) {
  uint32_t acc = 0;
  const long long stride = (long long)gridDim.x * READ_THREADS;
  long long i = blockIdx.x * (long long)READ_THREADS + threadIdx.x;
  for (; i + (READ_UNROLL - 1) * stride < n16; i += READ_UNROLL * stride) {
    uint4 v[READ_UNROLL];
#pragma unroll
    for (int u = 0; u < READ_UNROLL; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < READ_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace moesq

using namespace moesq;

extern "C" moesq_status_t moesq_stream_read(const void *buf, size_t bytes, uint32_t *sink,
                                            hipStream_t stream) {
  clear_error();
  if (!buf || !sink) return fail(MOESQ_ERR_NULL, "moesq_stream_read: NULL pointer");
  if (bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15))
    return fail(MOESQ_ERR_ARG, "moesq_stream_read: bytes and buf must be multiples of 16");
  const long long n16 = (long long)(bytes / 16);
  if (n16 == 0) return MOESQ_OK;
  long long blocks = (long long)device_cu_count() * 32;
  const long long need = (n16 + READ_THREADS - 1) / READ_THREADS;
  if (blocks > need) blocks = need;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(READ_THREADS), 0, stream,
                     (const uint4 *)buf, n16, sink);
  return launch_status("moesq_stream_read");
}
