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

// ---------------------------------------------------------------------------
// Gather ceiling of the decode's tile stream: the K and V 16-row tiles of a
// bf16 head-dim-128 pool, named by a list of first rows, each wavefront taking
// an equal contiguous run of the list (the balanced split without its
// arithmetic), in one of two ways:
//   mode 0  the decode's operand loads, straight into registers: K as the
//           MFMA A operand (lane l: row l % 16, 16-byte chunks l / 16 + 4c,
//           so one instruction covers half of each of 16 rows), V as 4 rows
//           of 16 bytes per lane; the non-temporal hint as in the decode;
//   mode 1  staged through LDS: each tile copied global -> LDS (16 bytes per
//           lane, 1 KB contiguous per instruction, a ring of two tiles per
//           wavefront), then the same operands read from LDS.
// Everything loaded is folded with XOR into one sink word per workgroup.
namespace {

constexpr int kGatherRow = 256;        // bytes per pool row (128 bf16)
constexpr int kGatherTile = 16 * kGatherRow;

__device__ __forceinline__ uint32_t fold(u32x4 x) { return x[0] ^ x[1] ^ x[2] ^ x[3]; }

template <int MODE>
__global__ __launch_bounds__(kThreads) void gather_probe_kernel(const char* __restrict__ kc,
                                                                const char* __restrict__ vc,
                                                                const int32_t* __restrict__ rows,
                                                                int64_t num_tiles, int64_t num_rows,
                                                                int32_t workers, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) char ring[MODE == 1 ? 4 * 2 * 2 * kGatherTile : 16];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * 4 + wv;
  uint32_t acc = 0;
  if (w < workers) {
    const int64_t per = (num_tiles + workers - 1) / workers;
    const int64_t t0 = (int64_t)w * per, t1 = t0 + per < num_tiles ? t0 + per : num_tiles;
    // a row past the pool (a bad list) reads row 0 instead: never out of bounds
    auto base = [&](int64_t t) -> int64_t {
      const int64_t r = rows[t];
      return (r >= 0 && r + 16 <= num_rows ? r : 0) * kGatherRow;
    };
    if (MODE == 0) {
      for (int64_t t = t0; t < t1; t += 2) {
        u32x4 x[2][8];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int64_t b = base(t + j < t1 ? t + j : t1 - 1);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            x[j][c] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(kc + b + (lane & 15) * kGatherRow + 16 * ((lane >> 4) + 4 * c)));
            x[j][4 + c] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(vc + b + (4 * (lane >> 4) + c) * kGatherRow + 16 * (lane & 15)));
          }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (t + j < t1)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc ^= fold(x[j][c]);
      }
    } else {
      char* my = ring + wv * 2 * 2 * kGatherTile;  // two slots of K + V
      auto issue = [&](int64_t t, int slot) {
        const int64_t b = base(t < t1 ? t : t1 - 1);
        char* dst = my + slot * 2 * kGatherTile;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(kc + b + 1024 * i + 16 * lane),
                                           (__attribute__((address_space(3))) void*)(dst + 1024 * i),
                                           16, 0, 0);
          __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(vc + b + 1024 * i + 16 * lane),
                                           (__attribute__((address_space(3))) void*)(dst + kGatherTile + 1024 * i),
                                           16, 0, 0);
        }
      };
      const int64_t n = t1 - t0;
      if (n > 0) {
        issue(t0, 0);
        issue(t0 + 1, 1);
        for (int64_t k = 0; k < n; ++k) {
          const int slot = (int)(k & 1);
          // tile k has landed once only the 8 copies of tile k + 1 are outstanding
          asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
          // The LDS reads are written as inline asm: the compiler would
          // otherwise wait for every outstanding global-to-LDS copy (the next
          // tile's too) before the first of them, which is what the ring is
          // there to avoid.  The explicit waits above and below order them.
          const uint32_t s = (uint32_t)(uintptr_t)(my + slot * 2 * kGatherTile);
          const uint32_t ka = s + (lane & 15) * kGatherRow + 16 * (lane >> 4);
          const uint32_t va = s + kGatherTile + 4 * (lane >> 4) * kGatherRow + 16 * (lane & 15);
          u32x4 x[8];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(x[c]) : "v"(ka), "i"(64 * c));
            asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(x[4 + c]) : "v"(va), "i"(kGatherRow * c));
          }
          // every LDS read of this slot has returned before it is refilled
          asm volatile("s_waitcnt lgkmcnt(0)"
                       : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                         "+v"(x[6]), "+v"(x[7])
                       :
                       : "memory");
#pragma unroll
          for (int c = 0; c < 8; ++c) acc ^= fold(x[c]);
          issue(t0 + k + 2, slot);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no copy lands after the wave ends
    }
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t part[kThreads / 64];
  if (lane == 0) part[wv] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_gather_probe(const void* kc, const void* vc, const int32_t* rows, int64_t num_tiles,
                               int64_t num_rows, int32_t workers, int32_t mode, uint32_t* sink,
                               hipStream_t stream) {
  const dim3 grid((unsigned)((workers + 3) / 4)), block(kThreads);
  if (mode == 0)
    hipLaunchKernelGGL(gather_probe_kernel<0>, grid, block, 0, stream, static_cast<const char*>(kc),
                       static_cast<const char*>(vc), rows, num_tiles, num_rows, workers, sink);
  else
    hipLaunchKernelGGL(gather_probe_kernel<1>, grid, block, 0, stream, static_cast<const char*>(kc),
                       static_cast<const char*>(vc), rows, num_tiles, num_rows, workers, sink);
  return hipGetLastError();
}

}  // namespace pkv
