// Slot-mapped KV-cache write for gfx950.
//
// Source: "PagedAttention, clearly explained" (a block holds the K/V of a fixed
// number of consecutive tokens; a token's logical position maps to a physical
// block recorded in the block table) and "What problem does PagedAttention
// solve...", section "The paging idea".  The caller hands each token's slot
// (physical block * block_size + offset); the kernel stores the token's rows for
// every KV head at that slot of the [NB, Hkv, bs, D] pools and nothing else.
//
// Work split: one thread moves one 16-byte chunk of a token's K or V row.  A
// token's K row for all heads is contiguous in the source, so adjacent threads
// read adjacent 16 bytes; each (head, chunk) lands in a D-element row of the
// pool.  The work is pure HBM traffic, so there is no LDS staging.
#include "e4m3.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

__device__ __forceinline__ float f32_from_bf16_bits(uint32_t b) { return __uint_as_float(b << 16); }

template <int IN, int OUT>
__global__ __launch_bounds__(kThreads) void kv_write_kernel(WriteArgs a, int tokens_per_group) {
  constexpr int kInBytes = IN == PKV_F32 ? 4 : 2;
  constexpr int kPerChunk = 16 / kInBytes;  // elements per 16-byte chunk
  const int H = a.num_heads, D = a.head_dim, bs = a.block_size;
  const int per_row = D / kPerChunk;
  const int per_kv = H * per_row;
  const int per_token = 2 * per_kv;
  const int64_t tok0 = (int64_t)blockIdx.x * tokens_per_group;
  const int64_t left = a.num_tokens - tok0;
  const int n_local = (int)(left < tokens_per_group ? left : tokens_per_group) * per_token;

  for (int i = threadIdx.x; i < n_local; i += kThreads) {
    const int tl = i / per_token;
    const int r = i - tl * per_token;
    const int is_v = r >= per_kv;
    const int r2 = r - is_v * per_kv;
    const int h = r2 / per_row;
    const int c = r2 - h * per_row;
    const int64_t t = tok0 + tl;
    // the source chunk does not depend on the slot: both loads go out together
    const int64_t src = (t * H + h) * (int64_t)D + (int64_t)c * kPerChunk;
    const u32x4 x = *reinterpret_cast<const u32x4*>(
        static_cast<const char*>(is_v ? a.v : a.k) + src * kInBytes);
    const int32_t slot = a.slots[t];
    if (slot < 0) continue;
    const int32_t blk = slot / bs;
    const int32_t off = slot - blk * bs;
    const int64_t dst = (((int64_t)blk * H + h) * bs + off) * (int64_t)D + (int64_t)c * kPerChunk;
    if constexpr (OUT == IN) {
      *reinterpret_cast<u32x4*>(static_cast<char*>(is_v ? a.vc : a.kc) + dst * kInBytes) = x;
    } else {
      const float inv = is_v ? a.inv_v : a.inv_k;
      uint8_t* out = static_cast<uint8_t*>(is_v ? a.vc : a.kc) + dst;
      if constexpr (IN == PKV_BF16) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = x[e >> 1];
          const uint32_t bits = (e & 1) ? (w >> 16) : (w & 0xffffu);
          lo |= e4m3_from_f32(f32_from_bf16_bits(bits) * inv) << (8 * e);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = x[2 + (e >> 1)];
          const uint32_t bits = (e & 1) ? (w >> 16) : (w & 0xffffu);
          hi |= e4m3_from_f32(f32_from_bf16_bits(bits) * inv) << (8 * e);
        }
        *reinterpret_cast<u32x2*>(out) = u32x2{lo, hi};
      } else {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) w |= e4m3_from_f32(__uint_as_float(x[e]) * inv) << (8 * e);
        *reinterpret_cast<uint32_t*>(out) = w;
      }
    }
  }
}

}  // namespace

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int in_bytes = a.in_dtype == PKV_F32 ? 4 : 2;
  const int per_token = 2 * a.num_heads * (a.head_dim * in_bytes / 16);
  int tpg = kThreads / per_token;
  if (tpg < 1) tpg = 1;
  const int64_t groups = (a.num_tokens + tpg - 1) / tpg;
  const dim3 grid((unsigned)groups), block(kThreads);
  if (a.in_dtype == PKV_F32 && a.cache_dtype == PKV_F32)
    hipLaunchKernelGGL((kv_write_kernel<PKV_F32, PKV_F32>), grid, block, 0, stream, a, tpg);
  else if (a.in_dtype == PKV_BF16 && a.cache_dtype == PKV_BF16)
    hipLaunchKernelGGL((kv_write_kernel<PKV_BF16, PKV_BF16>), grid, block, 0, stream, a, tpg);
  else if (a.in_dtype == PKV_BF16 && a.cache_dtype == PKV_FP8_E4M3)
    hipLaunchKernelGGL((kv_write_kernel<PKV_BF16, PKV_FP8_E4M3>), grid, block, 0, stream, a, tpg);
  else if (a.in_dtype == PKV_F32 && a.cache_dtype == PKV_FP8_E4M3)
    hipLaunchKernelGGL((kv_write_kernel<PKV_F32, PKV_FP8_E4M3>), grid, block, 0, stream, a, tpg);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
