// Slot-mapped KV-cache write for gfx950.
//
// Source: "PagedAttention, clearly explained" (a block holds the K/V of a fixed
// number of consecutive tokens; a token's logical position maps to a physical
// block recorded in the block table) and "What problem does PagedAttention
// solve...", section "The paging idea".  The caller hands each token's slot
// (physical block * block_size + offset); the kernel stores the token's rows for
// every KV head at that slot of the [NB, Hkv, bs, D] pools and nothing else.
//
// Work split.  Head dims 64, 128 and 256 take the row kernel: workgroup
// (x, y) writes row y (K or V of one head: y < H is K of head y) of a run of
// tokens, a row's 16-byte chunks spread over adjacent lanes, so a thread's
// chunk, head and K/V choice are constants and its token a simple stride --
// no per-chunk division.  (The index divisions of the general kernel below
// made the 4,096-token E4M3 chunk VALU-bound: about 185 VALU instructions per
// 16-byte chunk.)  Other head dims take the general kernel, which walks the
// flattened (token, K/V, head, chunk) index.  Both issue every load of a
// round (one or four chunks per thread) before the first store.  The work is
// pure HBM traffic, so there is no LDS staging.  E4M3 codes come from the
// hardware pack-convert (clamped first, so it saturates; NaN set to 0x7F),
// equal to the bit-level encoder in every case.
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

template <int IN, int OUT, int U>
__global__ __launch_bounds__(kThreads) void kv_write_any_kernel(WriteArgs a, int tokens_per_group) {
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
          *reinterpret_cast<u32x2*>(out) = u32x2{e4m3x4_cvt_bf16(x[j][0], x[j][1], inv),
                                                 e4m3x4_cvt_bf16(x[j][2], x[j][3], inv)};
        } else {
          *reinterpret_cast<uint32_t*>(out) =
              e4m3x4_cvt(__uint_as_float(x[j][0]) * inv, __uint_as_float(x[j][1]) * inv,
                         __uint_as_float(x[j][2]) * inv, __uint_as_float(x[j][3]) * inv);
        }
      }
    }
  }
}

// Row kernel: D / (16 / in bytes) lanes per row, kRows = 256 / that rows
// (tokens) per pass, U passes per workgroup with every load issued first.
// (Measured on the 4,096-token E4M3 chunk, replayed from a graph: two passes
// and the row-fastest order 4.6 us, against 4.8 us for rows in grid y.)
#ifndef PKV_WRITE_ROWS_U
#define PKV_WRITE_ROWS_U 2  // passes per workgroup in large writes
#endif
template <int IN, int OUT, int D, int U, bool POW2>
__global__ __launch_bounds__(kThreads) void kv_write_kernel(WriteArgs a, int bs_shift) {
  constexpr int kInBytes = IN == PKV_F32 ? 4 : 2;
  constexpr int kOutBytes = OUT == PKV_FP8_E4M3 ? 1 : kInBytes;
  constexpr int kPerChunk = 16 / kInBytes;     // elements per 16-byte source chunk
  constexpr int kLanesPerRow = D / kPerChunk;  // 8, 16, 32 or 64
  constexpr int kRows = kThreads / kLanesPerRow;
  const int H = a.num_heads, bs = a.block_size;
  // workgroup id = token run * 2H + row: the row varies fastest, so the
  // workgroups running together read whole tokens (all heads' K and V)
  const int rows = 2 * H;
  const int y = (int)(blockIdx.x % (unsigned)rows);
  const int64_t bx = blockIdx.x / (unsigned)rows;
  const bool is_v = y >= H;
  const int h = is_v ? y - H : y;
  const int c = threadIdx.x % kLanesPerRow;
  const int64_t t0 = bx * (kRows * U) + threadIdx.x / kLanesPerRow;
  const char* src = static_cast<const char*>(is_v ? a.v : a.k) +
                    ((int64_t)h * D + (int64_t)c * kPerChunk) * kInBytes;
  char* dst = static_cast<char*>(is_v ? a.vc : a.kc) +
              ((int64_t)h * bs * D + (int64_t)c * kPerChunk) * kOutBytes;
  const int64_t src_tok = (int64_t)H * D * kInBytes;  // source bytes per token
  const int64_t dst_blk = (int64_t)H * bs * D * kOutBytes;

  // Loads without branches (a token past the end re-reads the last one and
  // is dropped below), so the first store waits only for its own chunk.
  // The slots go first: then the first store waits for them and its own
  // chunk only.
  u32x4 x[U];
  int32_t slot[U];
  int64_t tc[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int64_t t = t0 + (int64_t)j * kRows;
    tc[j] = t < a.num_tokens ? t : a.num_tokens - 1;
    slot[j] = a.slots[tc[j]];
  }
  asm volatile("" ::: "memory");
#pragma unroll
  for (int j = 0; j < U; ++j) x[j] = *reinterpret_cast<const u32x4*>(src + tc[j] * src_tok);
  asm volatile("" ::: "memory");  // keep the loads here, ahead of every store
#pragma unroll
  for (int j = 0; j < U; ++j) {
    if (t0 + (int64_t)j * kRows >= a.num_tokens || slot[j] < 0) continue;  // past the end, or padding
    const int32_t blk = POW2 ? slot[j] >> bs_shift : slot[j] / bs;
    const int32_t off = POW2 ? slot[j] & (bs - 1) : slot[j] - blk * bs;
    char* o = dst + (int64_t)blk * dst_blk + (int64_t)off * D * kOutBytes;
    if constexpr (OUT == IN) {
      *reinterpret_cast<u32x4*>(o) = x[j];
    } else {
      const float inv = is_v ? a.inv_v : a.inv_k;
      if constexpr (IN == PKV_BF16) {
        *reinterpret_cast<u32x2*>(o) = u32x2{e4m3x4_cvt_bf16(x[j][0], x[j][1], inv),
                                             e4m3x4_cvt_bf16(x[j][2], x[j][3], inv)};
      } else {
        *reinterpret_cast<uint32_t*>(o) =
            e4m3x4_cvt(__uint_as_float(x[j][0]) * inv, __uint_as_float(x[j][1]) * inv,
                       __uint_as_float(x[j][2]) * inv, __uint_as_float(x[j][3]) * inv);
      }
    }
  }
}

template <int IN, int OUT>
hipError_t launch_any(const WriteArgs& a, hipStream_t stream) {
  const int in_bytes = IN == PKV_F32 ? 4 : 2;
  const int64_t per_token = 2 * (int64_t)a.num_heads * (a.head_dim * in_bytes / 16);
  // Four chunks per thread once the launch still has at least ~2 workgroups
  // per compute unit that way, else one chunk per thread and more workgroups.
  const int64_t chunks = a.num_tokens * per_token;
  const bool wide = chunks >= (int64_t)512 * kThreads * 4;
  const int U = wide ? PKV_WRITE_U : 1;
  int tpg = (int)((int64_t)kThreads * U / per_token);
  if (tpg < 1) tpg = 1;
  const int64_t groups = (a.num_tokens + tpg - 1) / tpg;
  const dim3 grid((unsigned)groups), block(kThreads);
  if (wide) hipLaunchKernelGGL((kv_write_any_kernel<IN, OUT, PKV_WRITE_U>), grid, block, 0, stream, a, tpg);
  else hipLaunchKernelGGL((kv_write_any_kernel<IN, OUT, 1>), grid, block, 0, stream, a, tpg);
  return hipGetLastError();
}

template <int IN, int OUT, int D>
hipError_t launch_rows(const WriteArgs& a, hipStream_t stream) {
  constexpr int kLanesPerRow = D / (16 / (IN == PKV_F32 ? 4 : 2));
  constexpr int kRows = kThreads / kLanesPerRow;
  const int bs = a.block_size;
  const bool pow2 = (bs & (bs - 1)) == 0;
  const int bs_shift = __builtin_ctz((unsigned)bs);
  // Two passes per workgroup while that still leaves at least ~2 workgroups
  // per compute unit (a 4,096-token chunk of 8 heads: 2,048), else one.
  const int64_t rows = 2 * (int64_t)a.num_heads;
  const bool wide = a.num_tokens * rows >= (int64_t)512 * kRows * PKV_WRITE_ROWS_U;
  constexpr int kU = PKV_WRITE_ROWS_U;
  const int U = wide ? kU : 1;
  const int64_t groups = (a.num_tokens + kRows * U - 1) / (kRows * U) * rows;
  if (groups > INT32_MAX) return launch_any<IN, OUT>(a, stream);
  const dim3 grid((unsigned)groups), block(kThreads);
  if (wide && pow2)
    hipLaunchKernelGGL((kv_write_kernel<IN, OUT, D, kU, true>), grid, block, 0, stream, a, bs_shift);
  else if (wide)
    hipLaunchKernelGGL((kv_write_kernel<IN, OUT, D, kU, false>), grid, block, 0, stream, a, bs_shift);
  else if (pow2)
    hipLaunchKernelGGL((kv_write_kernel<IN, OUT, D, 1, true>), grid, block, 0, stream, a, bs_shift);
  else
    hipLaunchKernelGGL((kv_write_kernel<IN, OUT, D, 1, false>), grid, block, 0, stream, a, bs_shift);
  return hipGetLastError();
}

template <int IN, int OUT>
hipError_t launch_io(const WriteArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_rows<IN, OUT, 128>(a, stream);
  if (a.head_dim == 64) return launch_rows<IN, OUT, 64>(a, stream);
  if (a.head_dim == 256) return launch_rows<IN, OUT, 256>(a, stream);
  return launch_any<IN, OUT>(a, stream);
}

}  // namespace

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  if (a.in_dtype == PKV_F32 && a.cache_dtype == PKV_F32) return launch_io<PKV_F32, PKV_F32>(a, stream);
  if (a.in_dtype == PKV_BF16 && a.cache_dtype == PKV_BF16) return launch_io<PKV_BF16, PKV_BF16>(a, stream);
  if (a.in_dtype == PKV_BF16 && a.cache_dtype == PKV_FP8_E4M3)
    return launch_io<PKV_BF16, PKV_FP8_E4M3>(a, stream);
  if (a.in_dtype == PKV_F32 && a.cache_dtype == PKV_FP8_E4M3)
    return launch_io<PKV_F32, PKV_FP8_E4M3>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
