// Wave64 tile fragments shared by the attention kernels of libpagedkv.so:
// one 16-token tile of one KV head in the MFMA operand layouts, the q
// fragments, the online-softmax state and the output stores.  Device code
// only: include from .hip sources.
//
// A tile holds tokens [t0, t0+16) of one KV head (rows of one physical block).
// Scores are S^T = K . Q^T on the matrix cores with A = the K tile (16 tokens
// x 32 d per MFMA, read straight from memory, 16 bytes per lane) and B = Q^T
// (16 query columns).  The result leaves column c = lane % 16 and tokens
// 4 * (lane / 16) + i in each lane, which is the B-operand layout of the P.V
// product, so probabilities never leave their registers.  V arrives row-major;
// pairs of tokens are packed with v_perm into the A operand of
// out^T = V^T . P with MFMA row m standing for d = VE * m + r.  The f32 tile
// also reads from a padded LDS copy (load_pitched) for the chunked prefill,
// whose bf16 and E4M3 path builds its own operand images in LDS instead.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "e4m3.h"
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
// E4M3 pairs -> packed bf16 pairs in one instruction (gfx950's scaled convert
// with scale 1: every E4M3 value is a bf16 value, so it is exact).
__device__ __forceinline__ uint32_t bf16x2_from_fp8x2_lo(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}
__device__ __forceinline__ uint32_t bf16x2_from_fp8x2_hi(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}
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

// K/V tile reads from the pool.  NT: every block is read once in the call,
// so the loads carry the non-temporal hint and stream past L2 and the MALL,
// which keep the small per-call data (lengths, block tables, q) instead.
template <bool NT, typename V>
__device__ __forceinline__ V pool_load(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(static_cast<const V*>(p));
  else return *static_cast<const V*>(p);
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

  template <bool NT = false>
  __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t row0, int lane) {
    const uint16_t* kb = static_cast<const uint16_t*>(kc) + row0 * D;
    const uint16_t* vb = static_cast<const uint16_t*>(vc) + row0 * D;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      k[c] = pool_load<NT, u32x4>(kb + (lane & 15) * D + c * 32 + (lane >> 4) * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = pool_load<NT, VRow>(vb + (4 * (lane >> 4) + j) * D + VE * (lane & 15));
  }
  // load() with token r of the tile read from the rows kn / vn instead (r < 0: none)
  template <bool NT = false>
  __device__ __forceinline__ void load_sub(const void* kc, const void* vc, int64_t row0, int lane,
                                           int r, const void* kn, const void* vn, float, float) {
    const uint16_t* kb = static_cast<const uint16_t*>(kc) + row0 * D;
    const uint16_t* vb = static_cast<const uint16_t*>(vc) + row0 * D;
    const uint16_t* kr = (lane & 15) == r ? static_cast<const uint16_t*>(kn) : kb + (lane & 15) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) k[c] = pool_load<NT, u32x4>(kr + c * 32 + (lane >> 4) * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * (lane >> 4) + j;
      const uint16_t* vr = t == r ? static_cast<const uint16_t*>(vn) : vb + t * D;
      v[j] = pool_load<NT, VRow>(vr + VE * (lane & 15));
    }
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

  template <bool NT = false>
  __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t row0, int lane) {
    const uint8_t* kb = static_cast<const uint8_t*>(kc) + row0 * D;
    const uint8_t* vb = static_cast<const uint8_t*>(vc) + row0 * D;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      k[c] = pool_load<NT, u32x4>(kb + (lane & 15) * D + 16 * ((lane >> 4) + 4 * c));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = pool_load<NT, VRow>(vb + (4 * (lane >> 4) + j) * D + VE * (lane & 15));
  }
  // load() with token r replaced by the bf16 rows kn / vn, quantized as the
  // KV write quantizes them (the conversion waits for those loads); r < 0: none
  template <bool NT = false>
  __device__ __forceinline__ void load_sub(const void* kc, const void* vc, int64_t row0, int lane,
                                           int r, const void* kn, const void* vn, float inv_k,
                                           float inv_v) {
    load<NT>(kc, vc, row0, lane);
    if (r < 0) return;
    if ((lane & 15) == r) {
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const uint16_t* src = static_cast<const uint16_t*>(kn) + 16 * ((lane >> 4) + 4 * c);
        const u32x4 lo = *reinterpret_cast<const u32x4*>(src);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(src + 8);
        k[c] = u32x4{e4m3x4_from_bf16x4(lo[0], lo[1], inv_k), e4m3x4_from_bf16x4(lo[2], lo[3], inv_k),
                     e4m3x4_from_bf16x4(hi[0], hi[1], inv_k), e4m3x4_from_bf16x4(hi[2], hi[3], inv_k)};
      }
    }
    if ((lane >> 4) == (r >> 2)) {
      const uint16_t* src = static_cast<const uint16_t*>(vn) + VE * (lane & 15);
      VRow x;
      if constexpr (VE == 8) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(src);
        x = VRow{e4m3x4_from_bf16x4(w[0], w[1], inv_v), e4m3x4_from_bf16x4(w[2], w[3], inv_v)};
      } else {
        const u32x2 w = *reinterpret_cast<const u32x2*>(src);
        x = e4m3x4_from_bf16x4(w[0], w[1], inv_v);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == (r & 3)) v[j] = x;
    }
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
        const u32x4 kb = {bf16x2_from_fp8x2_lo(w0), bf16x2_from_fp8x2_hi(w0),
                          bf16x2_from_fp8x2_lo(w1), bf16x2_from_fp8x2_hi(w1)};
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

  __device__ __forceinline__ void load_pitched(const char* kb, const char* vb, int pitch, int lane) {
#pragma unroll
    for (int c = 0; c < KC; ++c)
      k[c] = *reinterpret_cast<const f32x4*>(kb + (lane & 15) * pitch + 16 * (4 * c + (lane >> 4)));
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < VE / 4; ++w)
        v[j][w] = *reinterpret_cast<const f32x4*>(vb + (4 * (lane >> 4) + j) * pitch +
                                                  4 * (VE * (lane & 15) + 4 * w));
  }
  template <bool NT = false>
  __device__ __forceinline__ void load(const void* kc, const void* vc, int64_t row0, int lane) {
    const float* kb = static_cast<const float*>(kc) + row0 * D;
    const float* vb = static_cast<const float*>(vc) + row0 * D;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      k[c] = pool_load<NT, f32x4>(kb + (lane & 15) * D + 4 * (4 * c + (lane >> 4)));
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < VE / 4; ++w)
        v[j][w] = pool_load<NT, f32x4>(vb + (4 * (lane >> 4) + j) * D + VE * (lane & 15) + 4 * w);
  }
  template <bool NT = false>
  __device__ __forceinline__ void load_sub(const void* kc, const void* vc, int64_t row0, int lane,
                                           int r, const void* kn, const void* vn, float, float) {
    const float* kb = static_cast<const float*>(kc) + row0 * D;
    const float* vb = static_cast<const float*>(vc) + row0 * D;
    const float* kr = (lane & 15) == r ? static_cast<const float*>(kn) : kb + (lane & 15) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) k[c] = pool_load<NT, f32x4>(kr + 4 * (4 * c + (lane >> 4)));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * (lane >> 4) + j;
      const float* vr = t == r ? static_cast<const float*>(vn) : vb + t * D;
#pragma unroll
      for (int w = 0; w < VE / 4; ++w)
        v[j][w] = pool_load<NT, f32x4>(vr + VE * (lane & 15) + 4 * w);
    }
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
  struct PV {
    f32x4 v[4][VE / 4];
  };
  __device__ __forceinline__ PV pack_v() const {
    PV o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int w = 0; w < VE / 4; ++w) o.v[j][w] = v[j][w];
    return o;
  }
  __device__ static __forceinline__ float pv_packed(const PV& o, const float p[4], f32x4 acc[VE]) {
#pragma unroll
    for (int r = 0; r < VE; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[r] = mfma_f32_k4(o.v[i][r >> 2][r & 3], p[i], acc[r]);
    return (p[0] + p[1]) + (p[2] + p[3]);
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

// Max over the four lanes l, l^16, l^32, l^48 (the lanes holding one head's
// scores) with the gfx950 row-swap permutes: VALU only, no LDS round trip.
__device__ __forceinline__ float max_over_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Whole-wavefront reductions and scans in VALU: DPP moves within each row of
// 16 lanes (quad permutes, mirrors, row shifts), then across rows either the
// gfx950 row-swap permutes or the row broadcasts.  No LDS round trip.
// DPP controls (gfx9 encoding): quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_shr:n = 0x110 + n, row_mirror = 0x140, row_half_mirror = 0x141,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143.
template <int CTRL, int ROW_MASK = 0xF, bool BOUND = false>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, BOUND);
}
template <typename Op>
__device__ __forceinline__ uint32_t wave_all_reduce(uint32_t x, Op op) {
  x = op(x, dpp_u32<0xB1>(x));   // lane ^ 1
  x = op(x, dpp_u32<0x4E>(x));   // lane ^ 2
  x = op(x, dpp_u32<0x141>(x));  // lane i with 7 - i of its half row
  x = op(x, dpp_u32<0x140>(x));  // lane i with 15 - i of its row
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);  // lane ^ 16
  x = op(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);  // lane ^ 32
  return op(b[0], b[1]);
}
// Sum over the 64 lanes, in every lane.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return wave_all_reduce(x, [](uint32_t u, uint32_t v) { return u + v; });
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  return __uint_as_float(wave_all_reduce(__float_as_uint(x), [](uint32_t u, uint32_t v) {
    return __float_as_uint(__uint_as_float(u) + __uint_as_float(v));
  }));
}
__device__ __forceinline__ float wave_max_f32(float x) {
  return __uint_as_float(wave_all_reduce(__float_as_uint(x), [](uint32_t u, uint32_t v) {
    return __float_as_uint(fmaxf(__uint_as_float(u), __uint_as_float(v)));
  }));
}
// x + the value of lane ^ 16, then + the value of lane ^ 32 (the four lane groups).
__device__ __forceinline__ float sum_over_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Inclusive prefix sum over the 64 lanes: row shifts by 1, 2, 4, 8 (lanes
// past a row's start add 0), then rows 1 and 3 add the total of the row
// before them and rows 2 and 3 the total of rows 0 and 1.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += dpp_u32<0x111, 0xF, true>(x);
  x += dpp_u32<0x112, 0xF, true>(x);
  x += dpp_u32<0x114, 0xF, true>(x);
  x += dpp_u32<0x118, 0xF, true>(x);
  x += dpp_u32<0x142, 0xA>(x);
  x += dpp_u32<0x143, 0xC>(x);
  return x;
}

// Online-softmax state of one wavefront: per lane, head g = lane % 16.
template <int VE>
struct Softmax {
  float m = kNegInf;  // running max (log2 units), identical in the 4 lane groups
  float l = 0.f;      // this lane's share of the running sum
  f32x4 acc[VE];
};

}  // namespace
}  // namespace pkv
