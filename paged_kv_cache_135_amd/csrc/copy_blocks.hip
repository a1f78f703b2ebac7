// Copy-on-write block copies for gfx950.
//
// Source: "PagedAttention Memory Management", section "Complex Topologies and
// Memory Sharing", and "What problem does PagedAttention solve...", section
// "Sharing, the second dividend": a physical block listed by several block
// tables is copied to a fresh block before one branch writes into it.  For each
// (src, dst) pair the whole block (every KV head, every slot) of the K pool and
// of the V pool is copied.
//
// One workgroup moves one block of one pool: 256 threads, 16 bytes each, four
// loads in flight per thread before the stores.  Pure HBM traffic.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CopyArgs a) {
  const int64_t pair = blockIdx.x >> 1;
  const int is_v = blockIdx.x & 1;
  const int32_t src = a.pairs[2 * pair], dst = a.pairs[2 * pair + 1];
  if (src < 0 || dst < 0 || src == dst) return;
  char* pool = static_cast<char*>(is_v ? a.vc : a.kc);
  const u32x4* from = reinterpret_cast<const u32x4*>(pool + (int64_t)src * a.block_bytes);
  u32x4* to = reinterpret_cast<u32x4*>(pool + (int64_t)dst * a.block_bytes);
  const int64_t n16 = a.block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n16; i += kThreads * kUnroll) {
    u32x4 x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i + u * kThreads < n16) x[u] = from[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (i + u * kThreads < n16) to[i + u * kThreads] = x[u];
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream) {
  if (a.num_pairs == 0 || a.block_bytes == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)(2 * a.num_pairs)), dim3(kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace pkv
