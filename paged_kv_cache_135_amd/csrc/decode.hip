// Paged decode attention for gfx950 (CDNA4): one query token per sequence,
// keys and values gathered through the sequence's block table.
//
// Source: "PagedAttention, clearly explained" (at each decode step the kernel
// reads the block table and gathers K/V from whichever physical blocks they
// landed in) and "pipe-paged-block-allocation-kv-cache", sections "In and out"
// (the table is handed to the attention kernel, which gathers through that
// indirection; every read costs one indirection) and "Concept" (a weighted sum
// over logically ordered positions; physical adjacency is irrelevant).
//
// Design
// ------
// * Work unit: one workgroup per (partition, KV head, sequence).  All G = Hq/Hkv
//   query heads of the KV head are served by the same loaded K/V bytes.  A
//   partition is a run of 16-token tiles; in single-pass mode it is the whole
//   context.  The workgroup's wavefronts take tiles round-robin.
// * Tile = 16 consecutive tokens of one KV head: rows [t0, t0+16) of one
//   physical block (block_size is a multiple of 16), one table lookup.
// * Scores on the matrix cores: S^T[t][g] = sum_d K[t][d] Q[g][d] with
//   A = the K tile (16 tokens x 32 d per MFMA, read straight from HBM, 16 bytes
//   per lane) and B = Q^T (G heads padded to 16 columns).  The MFMA result puts
//   head g = lane % 16 and tokens 4*(lane/16)+i in each lane, which is also the
//   B-operand layout of the P.V product, so the probabilities never leave their
//   registers.
// * P.V on the matrix cores: out^T[d][g] = sum_t V^T[d][t] P[t][g].  V arrives
//   row-major (8 contiguous d per lane per token); pairs of tokens are packed
//   with v_perm into the A operand, assigning MFMA row m to d = VE*m + r, so no
//   LDS transpose is needed.  Accumulators stay in registers (fp32).
// * Online softmax in log2 units with a running max per head; tokens past the
//   context are removed by select (scores -> -inf, V rows -> 0), never by a
//   multiply, so stale or NaN bits in unwritten slots cannot leak.
// * Wavefront partials merge through LDS in a fixed order; split-K partials
//   merge in a second kernel in a fixed order: results are deterministic and
//   independent of physical block placement.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr uint32_t kSelLo = 0x05040100u;  // v_perm: low halves of two dwords
constexpr uint32_t kSelHi = 0x07060302u;  // v_perm: high halves of two dwords

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// E4M3 pairs -> f32 (exact): bytes 0,1 or 2,3 of a dword.
__device__ __forceinline__ f32x2 fp8x2_lo(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8(w, false); }
__device__ __forceinline__ f32x2 fp8x2_hi(uint32_t w) { return __builtin_amdgcn_cvt_pk_f32_fp8(w, true); }
// two f32 holding bf16-exact values -> packed bf16 pair (truncation is exact)
__device__ __forceinline__ uint32_t pack_exact(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), kSelHi);
}

__device__ __forceinline__ f32x4 mfma_bf16_k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16_k16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                   __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Per-element-type tile fragments.  `row0` is the pool row (token row of one
// KV head) of the tile's first token; rows are D elements long.
//
// K fragment, lane l: token t = l % 16 of the tile, 8 (bf16, E4M3 half-loads)
// or 4 (f32) consecutive d.  V fragment, lane l: tokens 4*(l/16) + j, j = 0..3,
// VE = D/16 consecutive d starting at VE*(l % 16).
// ---------------------------------------------------------------------------
template <int CT, int D>
struct Tile;

template <int D>
struct Tile<PKV_BF16, D> {
  static constexpr int VE = D / 16;
  static constexpr int KC = D / 32;  // 16x16x32 MFMAs per tile for q.K
  using VRow = typename std::conditional<VE == 8, u32x4, u32x2>::type;
  u32x4 k[KC];
  VRow v[4];

  __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t row0, int lane) {
    const uint16_t* kb = static_cast<const uint16_t*>(kc) + row0 * D;
    const uint16_t* vb = static_cast<const uint16_t*>(vc) + row0 * D;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      k[c] = *reinterpret_cast<const u32x4*>(kb + (lane & 15) * D + c * 32 + (lane >> 4) * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = *reinterpret_cast<const VRow*>(vb + (4 * (lane >> 4) + j) * D + VE * (lane & 15));
  }
  // B operand of the q.K MFMAs: Q row g = lane % 16 with the same d mapping as k[]
  struct QFrag {
    u32x4 q[KC];
  };
  __device__ static QFrag load_q(const uint16_t* qrow, bool valid, int lane) {
    QFrag f;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      f.q[c] = valid ? *reinterpret_cast<const u32x4*>(qrow + c * 32 + (lane >> 4) * 8)
                     : u32x4{0, 0, 0, 0};
    return f;
  }
  __device__ __forceinline__ f32x4 scores(const QFrag& qf) const {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) s = mfma_bf16_k32(k[c], qf.q[c], s);
    return s;
  }
  __device__ __forceinline__ void mask_rows(const bool ok[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < VE / 2; ++w) v[j][w] = ok[j] ? v[j][w] : 0u;
  }
  // acc[r] += V^T(rows d = VE*m + r) . P ; returns the sum of the rounded p
  __device__ __forceinline__ float pv(const float p[4], f32x4 acc[VE]) const {
    const uint32_t p01 = pack_bf16(p[0], p[1]);
    const uint32_t p23 = pack_bf16(p[2], p[3]);
    const u32x2 pb = {p01, p23};
#pragma unroll
    for (int r = 0; r < VE; ++r) {
      const uint32_t sel = (r & 1) ? kSelHi : kSelLo;
      const u32x2 a = {__builtin_amdgcn_perm(v[1][r >> 1], v[0][r >> 1], sel),
                       __builtin_amdgcn_perm(v[3][r >> 1], v[2][r >> 1], sel)};
      acc[r] = mfma_bf16_k16(a, pb, acc[r]);
    }
    return (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
  }
};

template <int D>
struct Tile<PKV_FP8_E4M3, D> {
  static constexpr int VE = D / 16;
  static constexpr int KC = D / 64;  // 16-byte K loads; each feeds two 16x16x32 MFMAs
  using VRow = typename std::conditional<VE == 8, u32x2, uint32_t>::type;
  u32x4 k[KC];
  VRow v[4];

  __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t row0, int lane) {
    const uint8_t* kb = static_cast<const uint8_t*>(kc) + row0 * D;
    const uint8_t* vb = static_cast<const uint8_t*>(vc) + row0 * D;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      k[c] = *reinterpret_cast<const u32x4*>(kb + (lane & 15) * D + 16 * ((lane >> 4) + 4 * c));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = *reinterpret_cast<const VRow*>(vb + (4 * (lane >> 4) + j) * D + VE * (lane & 15));
  }
  struct QFrag {
    u32x4 q[2 * KC];
  };
  __device__ static QFrag load_q(const uint16_t* qrow, bool valid, int lane) {
    QFrag f;
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        f.q[2 * c + h] =
            valid ? *reinterpret_cast<const u32x4*>(qrow + 16 * ((lane >> 4) + 4 * c) + 8 * h)
                  : u32x4{0, 0, 0, 0};
    return f;
  }
  __device__ __forceinline__ f32x4 scores(const QFrag& qf) const {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t w0 = k[c][2 * h], w1 = k[c][2 * h + 1];
        const f32x2 a = fp8x2_lo(w0), b = fp8x2_hi(w0), e = fp8x2_lo(w1), f = fp8x2_hi(w1);
        const u32x4 kb = {pack_exact(a[0], a[1]), pack_exact(b[0], b[1]),
                          pack_exact(e[0], e[1]), pack_exact(f[0], f[1])};
        s = mfma_bf16_k32(kb, qf.q[2 * c + h], s);
      }
    }
    return s;
  }
  __device__ __forceinline__ void mask_rows(const bool ok[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (VE == 8) {
        v[j][0] = ok[j] ? v[j][0] : 0u;
        v[j][1] = ok[j] ? v[j][1] : 0u;
      } else {
        v[j] = ok[j] ? v[j] : 0u;
      }
    }
  }
  __device__ __forceinline__ float pv(const float p[4], f32x4 acc[VE]) const {
    const uint32_t p01 = pack_bf16(p[0], p[1]);
    const uint32_t p23 = pack_bf16(p[2], p[3]);
    const u32x2 pb = {p01, p23};
    float fv[4][VE];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int w = 0; w < VE / 4; ++w) {
        uint32_t word;
        if constexpr (VE == 8) word = v[j][w]; else word = v[j];
        const f32x2 a = fp8x2_lo(word), b = fp8x2_hi(word);
        fv[j][4 * w + 0] = a[0];
        fv[j][4 * w + 1] = a[1];
        fv[j][4 * w + 2] = b[0];
        fv[j][4 * w + 3] = b[1];
      }
    }
#pragma unroll
    for (int r = 0; r < VE; ++r) {
      const u32x2 a = {pack_exact(fv[0][r], fv[1][r]), pack_exact(fv[2][r], fv[3][r])};
      acc[r] = mfma_bf16_k16(a, pb, acc[r]);
    }
    return (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23));
  }
};

template <int D>
struct Tile<PKV_F32, D> {
  static constexpr int VE = D / 16;
  static constexpr int KC = D / 16;  // float4 K loads; each feeds four 16x16x4 MFMAs
  f32x4 k[KC];
  f32x4 v[4][VE / 4];

  __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t row0, int lane) {
    const float* kb = static_cast<const float*>(kc) + row0 * D;
    const float* vb = static_cast<const float*>(vc) + row0 * D;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      k[c] = *reinterpret_cast<const f32x4*>(kb + (lane & 15) * D + 4 * (4 * c + (lane >> 4)));
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < VE / 4; ++w)
        v[j][w] = *reinterpret_cast<const f32x4*>(vb + (4 * (lane >> 4) + j) * D + VE * (lane & 15) + 4 * w);
  }
  struct QFrag {
    f32x4 q[KC];
  };
  __device__ static QFrag load_q(const float* qrow, bool valid, int lane) {
    QFrag f;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      f.q[c] = valid ? *reinterpret_cast<const f32x4*>(qrow + 4 * (4 * c + (lane >> 4)))
                     : f32x4{0.f, 0.f, 0.f, 0.f};
    return f;
  }
  __device__ __forceinline__ f32x4 scores(const QFrag& qf) const {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) s = mfma_f32_k4(k[c][e], qf.q[c][e], s);
    return s;
  }
  __device__ __forceinline__ void mask_rows(const bool ok[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < VE / 4; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[j][w][e] = ok[j] ? v[j][w][e] : 0.f;
  }
  __device__ __forceinline__ float pv(const float p[4], f32x4 acc[VE]) const {
#pragma unroll
    for (int r = 0; r < VE; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[r] = mfma_f32_k4(v[i][r >> 2][r & 3], p[i], acc[r]);
    return (p[0] + p[1]) + (p[2] + p[3]);
  }
};

template <int CT>
using QElem = typename std::conditional<CT == PKV_F32, float, uint16_t>::type;

// Store VE consecutive outputs (one lane's d-run) as f32 or bf16.
template <int CT, int VE>
__device__ __forceinline__ void store_run(void* out, int64_t idx, const float* x) {
  if constexpr (CT == PKV_F32) {
    float* o = static_cast<float*>(out) + idx;
#pragma unroll
    for (int w = 0; w < VE / 4; ++w)
      *reinterpret_cast<f32x4*>(o + 4 * w) = f32x4{x[4 * w], x[4 * w + 1], x[4 * w + 2], x[4 * w + 3]};
  } else {
    uint16_t* o = static_cast<uint16_t*>(out) + idx;
    if constexpr (VE == 8) {
      *reinterpret_cast<u32x4*>(o) = u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]),
                                           pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
    } else {
      *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
    }
  }
}

template <int CT, int D, int NW>
__global__ __launch_bounds__(NW * 64) void decode_partition_kernel(DecodeArgs a) {
  using T = Tile<CT, D>;
  constexpr int VE = T::VE;
  const int part = blockIdx.x, hk = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ctx = a.lens[s];
  const int ntiles = (ctx + 15) >> 4;
  const int tile_begin = part * a.part_tiles;
  if (part > 0 && tile_begin >= ntiles) return;  // whole workgroup: past this sequence
  const int tile_end = min(ntiles, tile_begin + a.part_tiles);
  const bool final_out = ntiles <= a.part_tiles;  // one partition holds the whole context

  const int G = a.group;
  const int g = lane & 15;
  const bool g_ok = g < G;
  const int qh = hk * G + g;  // query head of this lane's column
  const QElem<CT>* qrow = static_cast<const QElem<CT>*>(a.q) +
                          ((int64_t)s * a.num_q_heads + (g_ok ? qh : 0)) * D;
  const typename T::QFrag qf = T::load_q(qrow, g_ok, lane);

  const int32_t* table = a.tables + (int64_t)s * a.max_blocks;
  const int bs = a.block_size;
  const int64_t head_rows = (int64_t)hk * bs;  // row offset of this KV head inside a block
  const int64_t block_rows = (int64_t)a.num_kv_heads * bs;

  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[VE];
#pragma unroll
  for (int r = 0; r < VE; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline: the next tile's loads are in flight while this tile is
  // computed.  Past the end the load repeats the wave's last tile (in bounds,
  // result unused) so every iteration issues the same loads.
  T cur, nxt;
  int tile = tile_begin + wave;
  auto row_of = [&](int t_idx) -> int64_t {
    const int t0 = t_idx * 16;
    const int32_t blk = table[t0 / bs];
    return (int64_t)blk * block_rows + head_rows + (t0 % bs);
  };
  if (tile < tile_end) cur.load(a.kc, a.vc, row_of(tile), lane);
  for (; tile < tile_end; tile += NW) {
    const int nt = tile + NW < tile_end ? tile + NW : tile;
    nxt.load(a.kc, a.vc, row_of(nt), lane);

    const int t0 = tile * 16;
    const f32x4 sacc = cur.scores(qf);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = sacc[i] * a.qk_scale;
    if (t0 + 16 > ctx) {  // ragged last tile: drop tokens >= ctx by select
      bool ok[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ok[i] = t0 + 4 * (lane >> 4) + i < ctx;
        sc[i] = ok[i] ? sc[i] : kNegInf;
      }
      cur.mask_rows(ok);
    }
    float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float m_new = fmaxf(m_run, bm);  // finite: every tile holds >= 1 live token
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
#pragma unroll
    for (int r = 0; r < VE; ++r) acc[r] *= alpha;
    l_run = l_run * alpha + cur.pv(p, acc);
    m_run = m_new;
    cur = nxt;
  }
  // per-lane sums cover tokens 4*(lane/16)+i only; add the four lane groups
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);

  if constexpr (NW > 1) {
    // Merge the wavefronts' states in wave order.  Lane-indexed layout: every
    // lane reads back exactly the positions it owns.
    __shared__ float sm_acc[NW - 1][VE * 4][64];
    __shared__ float sm_ml[NW - 1][2][64];
    if (wave > 0) {
#pragma unroll
      for (int r = 0; r < VE; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm_acc[wave - 1][r * 4 + i][lane] = acc[r][i];
      sm_ml[wave - 1][0][lane] = m_run;
      sm_ml[wave - 1][1][lane] = l_run;
    }
    __syncthreads();
    if (wave > 0) return;
    float M = m_run;
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) M = fmaxf(M, sm_ml[w][0][lane]);
    if (M == kNegInf) {  // no tokens anywhere (empty context)
      l_run = 0.f;
    } else {
      const float f0 = __builtin_amdgcn_exp2f(m_run - M);
      l_run *= f0;
#pragma unroll
      for (int r = 0; r < VE; ++r) acc[r] *= f0;
#pragma unroll
      for (int w = 0; w < NW - 1; ++w) {
        const float fw = __builtin_amdgcn_exp2f(sm_ml[w][0][lane] - M);
        l_run += fw * sm_ml[w][1][lane];
#pragma unroll
        for (int r = 0; r < VE; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[r][i] += fw * sm_acc[w][r * 4 + i][lane];
      }
    }
    m_run = M;
  }

  if (!g_ok) return;
  const int64_t row = (int64_t)s * a.num_q_heads + qh;
  if (final_out) {
    const float inv = l_run > 0.f ? a.v_scale / l_run : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x[VE];
#pragma unroll
      for (int r = 0; r < VE; ++r) x[r] = acc[r][i] * inv;
      store_run<CT, VE>(a.out, row * D + VE * (4 * (lane >> 4) + i), x);
    }
  } else {
    const int64_t prow = row * a.num_parts + part;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* o = a.ws_acc + prow * D + VE * (4 * (lane >> 4) + i);
#pragma unroll
      for (int w = 0; w < VE / 4; ++w)
        *reinterpret_cast<f32x4*>(o + 4 * w) =
            f32x4{acc[4 * w][i], acc[4 * w + 1][i], acc[4 * w + 2][i], acc[4 * w + 3][i]};
    }
    if (lane < 16) *reinterpret_cast<f32x2*>(a.ws_ml + prow * 2) = f32x2{m_run, l_run};
  }
}

// Merge the partitions of one (sequence, query head) in partition order.
template <int CT, int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;
  const int h = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  const int ctx = a.lens[s];
  const int ntiles = (ctx + 15) >> 4;
  if (ntiles <= a.part_tiles) return;  // written directly by its only partition
  const int np = (ntiles + a.part_tiles - 1) / a.part_tiles;
  const int64_t prow0 = ((int64_t)s * a.num_q_heads + h) * a.num_parts;
  const float* ml = a.ws_ml + prow0 * 2;
  float M = kNegInf;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ml[2 * p]);
  float L = 0.f, o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int p = 0; p < np; ++p) {
    const float f = __builtin_amdgcn_exp2f(ml[2 * p] - M);
    L += f * ml[2 * p + 1];
    const float* src = a.ws_acc + (prow0 + p) * D + PER * lane;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] += f * src[e];
  }
  const float inv = a.v_scale / L;
  const int64_t oi = ((int64_t)s * a.num_q_heads + h) * D + PER * lane;
  if constexpr (CT == PKV_F32) {
#pragma unroll
    for (int e = 0; e < PER; ++e) static_cast<float*>(a.out)[oi + e] = o[e] * inv;
  } else {
    uint16_t* out = static_cast<uint16_t*>(a.out) + oi;
    if constexpr (PER == 2) {
      *reinterpret_cast<uint32_t*>(out) = pack_bf16(o[0] * inv, o[1] * inv);
    } else {
      out[0] = (uint16_t)(pack_bf16(o[0] * inv, 0.f) & 0xffffu);
    }
  }
}

template <int CT, int D, int NW>
hipError_t launch_nw(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.num_parts, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
  hipLaunchKernelGGL((decode_partition_kernel<CT, D, NW>), grid, dim3(NW * 64), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_parts == 1) return e;
  const dim3 rgrid((unsigned)a.num_q_heads, (unsigned)a.num_seqs);
  hipLaunchKernelGGL((decode_reduce_kernel<CT, D>), rgrid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int CT, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  switch (a.waves) {
    case 1: return launch_nw<CT, D, 1>(a, stream);
    case 2: return launch_nw<CT, D, 2>(a, stream);
    case 4: return launch_nw<CT, D, 4>(a, stream);
    case 8: return launch_nw<CT, D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int CT>
hipError_t launch_ct(const DecodeArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<CT, 128>(a, stream);
  if (a.head_dim == 64) return launch_d<CT, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  switch (a.cache_dtype) {
    case PKV_F32: return launch_ct<PKV_F32>(a, stream);
    case PKV_BF16: return launch_ct<PKV_BF16>(a, stream);
    case PKV_FP8_E4M3: return launch_ct<PKV_FP8_E4M3>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
