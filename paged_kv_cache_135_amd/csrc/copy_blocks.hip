// Whole-block moves for gfx950: copy-on-write copies inside the pools, and the
// gather / scatter of a sequence's blocks to and from a staging buffer when it
// is swapped out and back in.
//
// Sources: "PagedAttention Memory Management", section "Complex Topologies and
// Memory Sharing", and "What problem does PagedAttention solve...", section
// "Sharing, the second dividend": a physical block listed by several block
// tables is copied to a fresh block before one branch writes into it.  Same
// page, section "Operational consequences": under memory pressure a sequence
// is preempted, its blocks freed and its state swapped out (or recomputed);
// swapping in writes it back into whatever blocks are free then.  Each move
// copies a whole block (every KV head, every slot) of the K buffer and of the
// V buffer.
//
// One workgroup moves one block of one buffer: 256 threads, 16 bytes each,
// four loads in flight per thread before the stores.  Pure HBM traffic: every
// buffer is device memory (a host copy of a staging buffer is a separate
// copy-engine transfer).
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CopyArgs a) {
  const int64_t p = blockIdx.x >> 1;
  const int is_v = blockIdx.x & 1;
  const int64_t src = a.src_ids ? a.src_ids[p * a.id_stride] : p;
  const int64_t dst = a.dst_ids ? a.dst_ids[p * a.id_stride] : p;
  if (src < 0 || dst < 0 || (a.skip_same && src == dst)) return;
  const char* from_base = static_cast<const char*>(is_v ? a.src_v : a.src_k);
  char* to_base = static_cast<char*>(is_v ? a.dst_v : a.dst_k);
  const u32x4* from = reinterpret_cast<const u32x4*>(from_base + src * a.block_bytes);
  u32x4* to = reinterpret_cast<u32x4*>(to_base + dst * a.block_bytes);
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
