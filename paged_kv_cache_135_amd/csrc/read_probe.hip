// Streaming-read ceiling of the device: one pass over a device buffer with
// the widest vector loads and the non-temporal hint, nothing else.  It is the
// attainable-bandwidth yardstick the decode kernels' byte rates are reported
// against, next to the 8 TB/s datasheet peak.  Every 16-byte word is read
// exactly once; each workgroup folds what it read with XOR into one sink word,
// so the loads cannot be dropped and a caller can check the pass.
//
// Each workgroup streams one contiguous chunk of the buffer, so the requests
// in flight at any moment are spread over the whole buffer (every HBM channel
// and bank busy).  Measured on MI355X (2 GiB): 7.05 TB/s this way, against
// 5.9 TB/s when consecutive workgroups interleave 16-byte words (all requests
// then fall in one narrow window of addresses) and 5.5 TB/s with cached loads.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // loads in flight per thread before they are folded

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4* buf, int64_t n16,
                                                              uint32_t* sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;  // this workgroup's chunk
  const int64_t lo = (int64_t)blockIdx.x * per, hi = lo + per < n16 ? lo + per : n16;
  constexpr int64_t stride = kThreads;
  u32x4 acc = {0, 0, 0, 0};
  for (int64_t i = lo + threadIdx.x; i < hi; i += stride * kUnroll) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      x[u] = i + u * stride < hi ? __builtin_nontemporal_load(buf + i + u * stride) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
  }
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v ^= __shfl_xor(v, o);
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) w ^= part[i];
    sink[blockIdx.x] = w;
  }
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks,
                             hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkv
