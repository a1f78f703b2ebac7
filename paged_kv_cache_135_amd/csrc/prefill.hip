// Chunked-prefill paged attention for gfx950 (CDNA4): many new query tokens
// per sequence, each attending causally to its cached prefix (read through the
// block table) and to the chunk's earlier tokens.
//
// Source: "What problem does PagedAttention solve for the KV cache in vLLM?",
// section "Sharing, the second dividend" (blocks already holding a prompt
// prefix are reused and that part of prefill is skipped, so the remaining
// tokens attend over the cached prefix through the table) and
// "pipe-paged-block-allocation-kv-cache", section "Effect" (the boundary
// between reused and freshly prefilled blocks only changes how the attention
// reduction is tiled).  The chunk's own K/V are written first (the KV write),
// so query i of a chunk of n tokens sits at position len - n + i.
//
// Design
// ------
// * Rows: for one KV head, the chunk's (query token, query head) pairs in
//   token-major order, row = token * G + g, so one K/V tile feeds all G heads.
//   A wavefront owns R blocks of 16 rows (the B operand's 16 columns); a
//   workgroup of NW wavefronts owns 16 R NW consecutive rows.
// * Keys: 16-token tiles from position 0 up to the last position among the
//   wavefront's rows, loaded straight from the pool in the MFMA operand layout
//   (the decode tile fragments); V is packed once per tile and reused by the R
//   row blocks.  Block ids of the workgroup's tiles are staged in LDS.
// * Causal mask by select (scores of keys past a row's position -> -inf) only
//   on tiles that reach past the wavefront's first position; V rows past the
//   context are zeroed by select.  Tiles are visited in increasing order, so
//   key 0 (visible to every row) comes first and every running max is finite
//   from the first tile on.
// * Each row's result is finalised in place: no workspace, no second kernel.
// * The same machinery serves the shared-prefix part of a cascade decode
//   (shared_prefix_kernel): all sequences' query heads against one prefix,
//   split over keys, leaving partial states for the decode's merge.
#include "pkv_internal.h"
#include "tile.h"

namespace pkv {
namespace {

constexpr int kPrefillWaves = 8;
constexpr int kPrefillChunkTiles = 1024;  // block ids staged in LDS per pass

// A column keeps its running max until a score exceeds it by more than
// kLazyMax (log2 units): its probabilities then stay below 2^kLazyMax and the
// accumulators need no rescale (an unchanged max rescales by exactly 1).
constexpr float kLazyMax = 8.0f;

// Online-softmax update of one 16-row block with one tile.
template <int CT, int D>
__device__ __forceinline__ void prefill_update(const f32x4 sacc, const typename Tile<CT, D>::PV& pv,
                                               Softmax<D / 16>& st, int t0, int pos, bool causal,
                                               float qk_scale, int lane) {
  constexpr int VE = D / 16;
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = sacc[i] * qk_scale;
    if (causal) sc[i] = t0 + 4 * (lane >> 4) + i <= pos ? sc[i] : kNegInf;
  }
  const float bm = max_over_lane_groups(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
  // the first tile a column sees holds a visible key (tile 0 holds key 0), so
  // its running max is finite from then on
  const bool grow = bm > st.m + kLazyMax;
  const float m_new = grow ? bm : st.m;
  if (__ballot(grow) != 0) {  // wave-uniform: some column's max moved
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
#pragma unroll
    for (int r = 0; r < VE; ++r) st.acc[r] *= alpha;
    st.l *= alpha;
  }
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
  st.l += Tile<CT, D>::pv_packed(pv, p, st.acc);
  st.m = m_new;
}

// K/V of kStageKeys keys of one KV head staged in LDS, rows padded by 32
// bytes: the lanes reading one 16-byte column of 16 different rows then meet
// the fewest bank conflicts (measured against 0, 16, 48, 64 and 96 bytes).
constexpr int kStageKeys = 128;
constexpr int kStageTiles = kStageKeys / 16;
template <int CT, int D>
constexpr int row_bytes() {
  return D * (CT == PKV_F32 ? 4 : CT == PKV_BF16 ? 2 : 1);
}
template <int CT, int D>
constexpr int lds_pitch() {
  return row_bytes<CT, D>() + 32;
}

enum RowsJob : int { kPrefillJob = 0, kPrefixJob = 1 };

// Query rows against paged keys on the matrix cores, K/V streamed through LDS.
//   kPrefillJob: rows = a chunk's (query token, head) pairs of one KV head,
//     causal, final outputs (PrefillArgs).
//   kPrefixJob: rows = every sequence's query heads of one KV head against one
//     key split of a shared prefix, no mask, partial states (PrefixArgs).
// Per stage the workgroup's 256 threads copy kStageKeys keys of K and V from
// the pool into LDS (16 bytes per thread and piece), then every wavefront
// reads its MFMA fragments from LDS.  The next stage's global loads are issued
// before the current stage is computed, so they are in flight meanwhile.
// The same update for two tiles at once (keys t0 .. t0+31): one max, one
// rescale, and P.V on the double-rate K=32 MFMA.  A second tile that is out of
// range has all its scores at -inf (and its V rows zeroed by the caller).
template <int CT, int D>
__device__ __forceinline__ void prefill_update2(const f32x4 sa, const f32x4 sb,
                                                const typename Tile<CT, D>::PV2& pv,
                                                Softmax<D / 16>& st, int t0, int pos, bool causal,
                                                bool b_live, float qk_scale, int lane) {
  constexpr int VE = D / 16;
  float pa[4], pb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = t0 + 4 * (lane >> 4) + i;
    pa[i] = sa[i] * qk_scale;
    pb[i] = sb[i] * qk_scale;
    if (causal) {
      pa[i] = key <= pos ? pa[i] : kNegInf;
      pb[i] = key + 16 <= pos ? pb[i] : kNegInf;
    }
    pb[i] = b_live ? pb[i] : kNegInf;
  }
  const float bm = max_over_lane_groups(fmaxf(fmaxf(fmaxf(pa[0], pa[1]), fmaxf(pa[2], pa[3])),
                                              fmaxf(fmaxf(pb[0], pb[1]), fmaxf(pb[2], pb[3]))));
  const bool grow = bm > st.m + kLazyMax;
  const float m_new = grow ? bm : st.m;
  if (__ballot(grow) != 0) {
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
#pragma unroll
    for (int r = 0; r < VE; ++r) st.acc[r] *= alpha;
    st.l *= alpha;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pa[i] = __builtin_amdgcn_exp2f(pa[i] - m_new);
    pb[i] = __builtin_amdgcn_exp2f(pb[i] - m_new);
  }
  st.l += Tile<CT, D>::pv2(pv, pa, pb, st.acc);
  st.m = m_new;
}

template <int CT, int D, int R, int JOB, typename Args>
__global__ __launch_bounds__(kPrefillWaves * 64) void rows_kernel(Args a) {
  using T = Tile<CT, D>;
  constexpr int VE = T::VE;
  constexpr int NW = kPrefillWaves;
  constexpr int ROWS_W = 16 * R;
  constexpr int ROWS_G = ROWS_W * NW;
  constexpr int RB = row_bytes<CT, D>();
  constexpr int PITCH = lds_pitch<CT, D>();
  constexpr int PER_ROW = RB / 16;                          // 16-byte pieces per key row
  constexpr int TOTAL = kStageKeys * PER_ROW;               // pieces per stage and pool
  constexpr int PIECES = (TOTAL + NW * 64 - 1) / (NW * 64);  // per thread and pool
  static_assert(TOTAL % (NW * 64) == 0 || TOTAL < NW * 64, "stage split");
  const int hk = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group, Hq = a.num_q_heads, bs = a.block_size;
  const int64_t head_rows = (int64_t)hk * bs;
  const int64_t block_rows = (int64_t)a.num_kv_heads * bs;

  // what this workgroup works on
  int rows, ctx, first_pos = 0, q0 = 0, k_lo, k_hi_all;
  const int32_t* table;
  if constexpr (JOB == kPrefillJob) {
    const int s = blockIdx.z;
    q0 = a.qstart[s];
    const int nq = a.qstart[s + 1] - q0;
    rows = nq * G;
    ctx = a.lens[s];
    first_pos = ctx - nq;
    table = a.tables + (int64_t)s * a.max_blocks;
    k_lo = 0;
    k_hi_all = 0;  // per row group below
  } else {
    const int split = blockIdx.z;
    const int ntiles = a.prefix_len / 16;
    rows = a.num_seqs * G;
    ctx = a.prefix_len;
    table = a.blocks;
    k_lo = (int)((int64_t)split * ntiles / a.splits);
    k_hi_all = (int)((int64_t)(split + 1) * ntiles / a.splits);
  }

  __shared__ int32_t sm_blk[kPrefillChunkTiles];
  __shared__ __attribute__((aligned(16))) char sm_k[kStageKeys * PITCH];
  __shared__ __attribute__((aligned(16))) char sm_v[kStageKeys * PITCH];

  for (int row_g0 = blockIdx.x * ROWS_G; row_g0 < rows; row_g0 += gridDim.x * ROWS_G) {
    const int row_w0 = row_g0 + wave * ROWS_W;
    const bool live = row_w0 < rows;
    const int last_row_g = min(rows, row_g0 + ROWS_G) - 1;
    const int last_row_w = min(rows, row_w0 + ROWS_W) - 1;
    // key tiles: [k_lo, k_hi) for the workgroup, [k_lo, k_hi_w) for this wavefront
    int k_hi, k_hi_w, minpos_w = 0;
    if constexpr (JOB == kPrefillJob) {
      k_hi = (first_pos + last_row_g / G) / 16 + 1;
      k_hi_w = live ? (first_pos + last_row_w / G) / 16 + 1 : 0;
      minpos_w = first_pos + row_w0 / G;
    } else {
      k_hi = k_hi_all;
      k_hi_w = live ? k_hi_all : k_lo;
    }

    typename T::QFrag qf[R];
    int pos[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
      const int rr = row_w0 + 16 * rb + (lane & 15);
      const bool valid = rr < rows;
      const int t = valid ? rr / G : 0;  // query token (prefill) or sequence (prefix)
      const int g = valid ? rr - t * G : 0;
      qf[rb] = T::load_q(static_cast<const QElem<CT>*>(a.q) + ((int64_t)(q0 + t) * Hq + hk * G + g) * D,
                         valid, lane);
      pos[rb] = valid ? first_pos + t : ctx - 1;  // padding columns see every key
    }
    Softmax<VE> st[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb)
#pragma unroll
      for (int r = 0; r < VE; ++r) st[rb].acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = k_lo; c0 < k_hi; c0 += kPrefillChunkTiles) {
      const int c1 = min(k_hi, c0 + kPrefillChunkTiles);
      __syncthreads();  // the previous pass is done with the ids and the stage
      for (int i = threadIdx.x; i < c1 - c0; i += NW * 64) sm_blk[i] = table[((c0 + i) * 16) / bs];
      __syncthreads();

      // staged copy of stage [t0, t0 + kStageTiles): piece p of a pool is key
      // p / PER_ROW, 16-byte column p % PER_ROW
      u32x4 rk[PIECES], rv[PIECES];
      auto fetch = [&](int tile0) {
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
          const int p = threadIdx.x + i * NW * 64;
          if (TOTAL < NW * 64 && p >= TOTAL) break;  // fewer pieces than threads
          const int key = p / PER_ROW, col = p - key * PER_ROW;
          const int t = min(tile0 + key / 16, c1 - 1);  // past the end: a valid tile, unused
          const int64_t row = (int64_t)sm_blk[t - c0] * block_rows + head_rows + ((t * 16) % bs) + (key & 15);
          rk[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.kc) + row * RB + col * 16);
          rv[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.vc) + row * RB + col * 16);
        }
      };
      fetch(c0);
      for (int t0s = c0; t0s < c1; t0s += kStageTiles) {
        __syncthreads();  // every wave has finished reading the previous stage
#pragma unroll
        for (int i = 0; i < PIECES; ++i) {
          const int p = threadIdx.x + i * NW * 64;
          if (TOTAL < NW * 64 && p >= TOTAL) break;
          const int key = p / PER_ROW, col = p - key * PER_ROW;
          *reinterpret_cast<u32x4*>(sm_k + key * PITCH + col * 16) = rk[i];
          *reinterpret_cast<u32x4*>(sm_v + key * PITCH + col * 16) = rv[i];
        }
        __syncthreads();
        if (t0s + kStageTiles < c1) fetch(t0s + kStageTiles);  // in flight during the compute
        auto load_masked = [&](T& tl, int j, bool in_range) {
          const int t0 = (t0s + j) * 16;
          tl.load_pitched(sm_k + j * 16 * PITCH, sm_v + j * 16 * PITCH, PITCH, lane);
          if (!in_range || t0 + 16 > ctx) {  // V rows past the context may hold any bits
            bool ok[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ok[i] = in_range && t0 + 4 * (lane >> 4) + i < ctx;
            tl.mask_rows(ok);
          }
        };
        if constexpr (CT == PKV_F32) {  // no K=32 f32 MFMA: one tile at a time
#pragma unroll
          for (int j = 0; j < kStageTiles; ++j) {
            const int tile = t0s + j;
            if (tile >= k_hi_w) break;  // wave-uniform
            const int t0 = tile * 16;
            T tl;
            load_masked(tl, j, true);
            const typename T::PV pv = tl.pack_v();
            const bool causal = JOB == kPrefillJob && t0 + 15 > minpos_w;
#pragma unroll
            for (int rb = 0; rb < R; ++rb)
              prefill_update<CT, D>(tl.scores(qf[rb]), pv, st[rb], t0, pos[rb], causal, a.qk_scale,
                                    lane);
          }
        } else {  // tile pairs on the double-rate MFMA
#pragma unroll
          for (int j = 0; j < kStageTiles; j += 2) {
            const int tile = t0s + j;
            if (tile >= k_hi_w) break;  // wave-uniform
            const bool b_live = tile + 1 < k_hi_w;
            const int t0 = tile * 16;
            T ta, tb;
            load_masked(ta, j, true);
            load_masked(tb, j + 1, b_live);
            const typename T::PV2 pv = T::pack_v2(ta, tb);
            const bool causal = JOB == kPrefillJob && t0 + 31 > minpos_w;
#pragma unroll
            for (int rb = 0; rb < R; ++rb)
              prefill_update2<CT, D>(ta.scores(qf[rb]), tb.scores(qf[rb]), pv, st[rb], t0, pos[rb],
                                     causal, b_live, a.qk_scale, lane);
          }
        }
      }
    }

    if (live) {
#pragma unroll
      for (int rb = 0; rb < R; ++rb) {
        float l_run = st[rb].l;
        l_run += __shfl_xor(l_run, 16);
        l_run += __shfl_xor(l_run, 32);
        const int rr = row_w0 + 16 * rb + (lane & 15);
        if (rr >= rows) continue;
        const int t = rr / G, g = rr - t * G;
        if constexpr (JOB == kPrefillJob) {
          const int64_t orow = (int64_t)(q0 + t) * Hq + hk * G + g;
          const float inv = a.v_scale / l_run;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x[VE];
#pragma unroll
            for (int r = 0; r < VE; ++r) x[r] = st[rb].acc[r][i] * inv;
            store_run<CT, VE>(a.out, orow * D + VE * (4 * (lane >> 4) + i), x);
          }
        } else {
          const int64_t slot = a.slot0 + ((int64_t)t * a.num_kv_heads + hk) * a.splits + blockIdx.z;
          float* o = a.ws_acc + (slot * G + g) * D;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q4 = 0; q4 < VE / 4; ++q4)
              *reinterpret_cast<f32x4*>(o + VE * (4 * (lane >> 4) + i) + 4 * q4) =
                  f32x4{st[rb].acc[4 * q4][i], st[rb].acc[4 * q4 + 1][i], st[rb].acc[4 * q4 + 2][i],
                        st[rb].acc[4 * q4 + 3][i]};
          if (lane < 16) *reinterpret_cast<f32x2*>(a.ws_ml + (slot * G + g) * 2) = f32x2{st[rb].m, l_run};
        }
      }
    }
  }
}

template <int CT, int D>
hipError_t launch_prefix_d(const PrefixArgs& a, hipStream_t stream) {
  constexpr int ROWS_G = 32 * kPrefillWaves;
  int64_t gx = ((int64_t)a.num_seqs * a.group + ROWS_G - 1) / ROWS_G;
  gx = gx < 1 ? 1 : gx > 65535 ? 65535 : gx;
  const dim3 grid((unsigned)gx, (unsigned)a.num_kv_heads, (unsigned)a.splits);
  hipLaunchKernelGGL((rows_kernel<CT, D, 2, kPrefixJob, PrefixArgs>), grid, dim3(kPrefillWaves * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <int CT>
hipError_t launch_prefix_ct(const PrefixArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_prefix_d<CT, 128>(a, stream);
  if (a.head_dim == 64) return launch_prefix_d<CT, 64>(a, stream);
  return hipErrorInvalidValue;
}

template <int CT, int D, int R>
hipError_t launch_r(const PrefillArgs& a, hipStream_t stream) {
  constexpr int ROWS_G = 16 * R * kPrefillWaves;
  const int64_t rows = (int64_t)a.max_query_len * a.group;
  int64_t gx = (rows + ROWS_G - 1) / ROWS_G;
  gx = gx < 1 ? 1 : gx > 65535 ? 65535 : gx;
  const dim3 grid((unsigned)gx, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
  hipLaunchKernelGGL((rows_kernel<CT, D, R, kPrefillJob, PrefillArgs>), grid, dim3(kPrefillWaves * 64), 0,
                     stream, a);
  return hipGetLastError();
}

template <int CT, int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
  switch (a.rows_per_wave) {
    case 16: return launch_r<CT, D, 1>(a, stream);
    case 32: return launch_r<CT, D, 2>(a, stream);
    case 64:  // with head_dim 128 or f32 fragments, 64 rows per wavefront would spill
      if constexpr (CT != PKV_F32 && D == 64) return launch_r<CT, D, 4>(a, stream);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int CT>
hipError_t launch_ct(const PrefillArgs& a, hipStream_t stream) {
  if (a.head_dim == 128) return launch_d<CT, 128>(a, stream);
  if (a.head_dim == 64) return launch_d<CT, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_shared_prefix(const PrefixArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  switch (a.cache_dtype) {
    case PKV_F32: return launch_prefix_ct<PKV_F32>(a, stream);
    case PKV_BF16: return launch_prefix_ct<PKV_BF16>(a, stream);
    case PKV_FP8_E4M3: return launch_prefix_ct<PKV_FP8_E4M3>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.max_query_len == 0) return hipSuccess;
  switch (a.cache_dtype) {
    case PKV_F32: return launch_ct<PKV_F32>(a, stream);
    case PKV_BF16: return launch_ct<PKV_BF16>(a, stream);
    case PKV_FP8_E4M3: return launch_ct<PKV_FP8_E4M3>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
