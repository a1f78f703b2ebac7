// Slot-mapped KV-cache write for gfx950.
//
// Source: "PagedAttention, clearly explained" (a block holds the K/V of a fixed
// number of consecutive tokens; a token's logical position maps to a physical
// block recorded in the block table) and "What problem does PagedAttention
// solve...", section "The paging idea".  The caller hands each token's slot
// (physical block * block_size + offset); the kernel stores the token's rows for
// every KV head at that slot of the [NB, Hkv, bs, D] pools and nothing else.
//
// Work split: a thread moves 16-byte chunks of tokens' K or V rows, one or four
// per thread (four for large writes, all loads issued before any store).  A
// token's K row for all heads is contiguous in the source, so adjacent threads
// read adjacent 16 bytes; each (head, chunk) lands in a D-element row of the
// pool.  The work is pure HBM traffic, so there is no LDS staging.  E4M3 codes
// come from the hardware pack-convert (clamped first, so it saturates; NaN set
// to 0x7F), equal to the bit-level encoder in every case.
#include "e4m3.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
#ifndef PKV_WRITE_U
#define PKV_WRITE_U 4  // chunks per thread in large writes
#endif

__device__ __forceinline__ float f32_from_bf16_bits(uint32_t b) { return __uint_as_float(b << 16); }

template <int IN, int OUT, int U>
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

  // U chunks per thread: every source load and slot load of the round is
  // issued before the first conversion or store, so U x 16 bytes per thread
  // are in flight at once.
  for (int base = 0; base < n_local; base += kThreads * U) {
    u32x4 x[U];
    int32_t slot[U];
    int h[U], c[U], is_v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int i = base + threadIdx.x + j * kThreads;
      slot[j] = -1;
      if (i < n_local) {
        const int tl = i / per_token;
        const int r = i - tl * per_token;
        is_v[j] = r >= per_kv;
        const int r2 = r - is_v[j] * per_kv;
        h[j] = r2 / per_row;
        c[j] = r2 - h[j] * per_row;
        const int64_t t = tok0 + tl;
        const int64_t src = (t * H + h[j]) * (int64_t)D + (int64_t)c[j] * kPerChunk;
        x[j] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(is_v[j] ? a.v : a.k) +
                                               src * kInBytes);
        slot[j] = a.slots[t];
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (slot[j] < 0) continue;  // padding token, or past the group's chunks
      const int32_t blk = slot[j] / bs;
      const int32_t off = slot[j] - blk * bs;
      const int64_t dst =
          (((int64_t)blk * H + h[j]) * bs + off) * (int64_t)D + (int64_t)c[j] * kPerChunk;
      if constexpr (OUT == IN) {
        *reinterpret_cast<u32x4*>(static_cast<char*>(is_v[j] ? a.vc : a.kc) + dst * kInBytes) = x[j];
      } else {
        const float inv = is_v[j] ? a.inv_v : a.inv_k;
        uint8_t* out = static_cast<uint8_t*>(is_v[j] ? a.vc : a.kc) + dst;
        if constexpr (IN == PKV_BF16) {
          const u32x4 w = x[j];
          const uint32_t lo = e4m3x4_cvt(f32_from_bf16_bits(w[0] & 0xffffu) * inv,
                                         f32_from_bf16_bits(w[0] >> 16) * inv,
                                         f32_from_bf16_bits(w[1] & 0xffffu) * inv,
                                         f32_from_bf16_bits(w[1] >> 16) * inv);
          const uint32_t hi = e4m3x4_cvt(f32_from_bf16_bits(w[2] & 0xffffu) * inv,
                                         f32_from_bf16_bits(w[2] >> 16) * inv,
                                         f32_from_bf16_bits(w[3] & 0xffffu) * inv,
                                         f32_from_bf16_bits(w[3] >> 16) * inv);
          *reinterpret_cast<u32x2*>(out) = u32x2{lo, hi};
        } else {
          *reinterpret_cast<uint32_t*>(out) =
              e4m3x4_cvt(__uint_as_float(x[j][0]) * inv, __uint_as_float(x[j][1]) * inv,
                         __uint_as_float(x[j][2]) * inv, __uint_as_float(x[j][3]) * inv);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int in_bytes = a.in_dtype == PKV_F32 ? 4 : 2;
  const int64_t per_token = 2 * (int64_t)a.num_heads * (a.head_dim * in_bytes / 16);
  // Four chunks per thread once the launch still has at least ~2 workgroups
  // per compute unit that way (a 4,096-token prefill chunk of 8 heads: 1,024
  // workgroups); smaller writes (one token per sequence of a decode step) keep
  // one chunk per thread and more workgroups.
  const int64_t chunks = a.num_tokens * per_token;
  const bool wide = chunks >= (int64_t)512 * kThreads * 4;
  const int U = wide ? PKV_WRITE_U : 1;
  int tpg = (int)((int64_t)kThreads * U / per_token);
  if (tpg < 1) tpg = 1;
  const int64_t groups = (a.num_tokens + tpg - 1) / tpg;
  const dim3 grid((unsigned)groups), block(kThreads);
#define PKV_WRITE(IN, OUT)                                                                       \
  do {                                                                                           \
    if (wide) hipLaunchKernelGGL((kv_write_kernel<IN, OUT, PKV_WRITE_U>), grid, block, 0, stream, a, tpg); \
    else hipLaunchKernelGGL((kv_write_kernel<IN, OUT, 1>), grid, block, 0, stream, a, tpg);      \
  } while (0)
  if (a.in_dtype == PKV_F32 && a.cache_dtype == PKV_F32) PKV_WRITE(PKV_F32, PKV_F32);
  else if (a.in_dtype == PKV_BF16 && a.cache_dtype == PKV_BF16) PKV_WRITE(PKV_BF16, PKV_BF16);
  else if (a.in_dtype == PKV_BF16 && a.cache_dtype == PKV_FP8_E4M3) PKV_WRITE(PKV_BF16, PKV_FP8_E4M3);
  else if (a.in_dtype == PKV_F32 && a.cache_dtype == PKV_FP8_E4M3) PKV_WRITE(PKV_F32, PKV_FP8_E4M3);
  else return hipErrorInvalidValue;
#undef PKV_WRITE
  return hipGetLastError();
}

}  // namespace pkv
