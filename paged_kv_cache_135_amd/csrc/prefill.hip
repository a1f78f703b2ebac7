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

constexpr int kPrefillWaves = 4;
constexpr int kPrefillChunkTiles = 1024;  // block ids staged in LDS per pass

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
  const float m_new = fmaxf(st.m, bm);  // finite: tile 0 holds key 0, visible to every row
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
#pragma unroll
  for (int r = 0; r < VE; ++r) st.acc[r] *= alpha;
  st.l = st.l * alpha + Tile<CT, D>::pv_packed(pv, p, st.acc);
  st.m = m_new;
}

template <int CT, int D, int R, int NBUF>
__global__ __launch_bounds__(kPrefillWaves * 64) void prefill_kernel(PrefillArgs a) {
  using T = Tile<CT, D>;
  constexpr int VE = T::VE;
  constexpr int NW = kPrefillWaves;
  constexpr int ROWS_W = 16 * R;
  constexpr int ROWS_G = ROWS_W * NW;
  const int s = blockIdx.z, hk = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group, Hq = a.num_q_heads, bs = a.block_size;
  const int q0 = a.qstart[s];
  const int nq = a.qstart[s + 1] - q0;
  const int rows = nq * G;
  const int ctx = a.lens[s];
  const int first_pos = ctx - nq;  // position of the chunk's first query
  const int32_t* table = a.tables + (int64_t)s * a.max_blocks;
  const int64_t head_rows = (int64_t)hk * bs;
  const int64_t block_rows = (int64_t)a.num_kv_heads * bs;
  __shared__ int32_t sm_blk[kPrefillChunkTiles];

  for (int row_g0 = blockIdx.x * ROWS_G; row_g0 < rows; row_g0 += gridDim.x * ROWS_G) {
    const int last_row_g = min(rows, row_g0 + ROWS_G) - 1;
    const int ntiles_g = (first_pos + last_row_g / G) / 16 + 1;
    const int row_w0 = row_g0 + wave * ROWS_W;
    const bool live = row_w0 < rows;
    const int last_row_w = min(rows, row_w0 + ROWS_W) - 1;
    const int ntiles_w = live ? (first_pos + last_row_w / G) / 16 + 1 : 0;
    const int minpos_w = first_pos + row_w0 / G;

    // q fragments and positions of this lane's column in each row block
    typename T::QFrag qf[R];
    int pos[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
      const int rr = row_w0 + 16 * rb + (lane & 15);
      const bool valid = rr < rows;
      const int tok = valid ? rr / G : 0;
      const int g = valid ? rr - tok * G : 0;
      const QElem<CT>* qrow = static_cast<const QElem<CT>*>(a.q) +
                              ((int64_t)(q0 + tok) * Hq + hk * G + g) * D;
      qf[rb] = T::load_q(qrow, valid, lane);
      pos[rb] = valid ? first_pos + tok : ctx - 1;  // padding columns see every key
    }
    Softmax<VE> st[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb)
#pragma unroll
      for (int r = 0; r < VE; ++r) st[rb].acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = 0; c0 < ntiles_g; c0 += kPrefillChunkTiles) {
      const int c1 = min(ntiles_g, c0 + kPrefillChunkTiles);
      __syncthreads();  // every wave is done with the previous ids
      for (int i = threadIdx.x; i < c1 - c0; i += NW * 64) sm_blk[i] = table[((c0 + i) * 16) / bs];
      __syncthreads();
      const int end = min(c1, ntiles_w);
      // batches of NBUF tiles: loads issued back to back, then computed in order
      for (int k = c0; k < end; k += NBUF) {
        T buf[NBUF];
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          const int t = min(k + j, end - 1);
          buf[j].load(a.kc, a.vc, (int64_t)sm_blk[t - c0] * block_rows + head_rows + ((t * 16) % bs),
                      lane);
        }
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          if (k + j >= end) break;
          const int t0 = (k + j) * 16;
          if (t0 + 16 > ctx) {  // V rows past the context may hold any bits
            bool ok[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ok[i] = t0 + 4 * (lane >> 4) + i < ctx;
            buf[j].mask_rows(ok);
          }
          const typename T::PV pv = buf[j].pack_v();
          const bool causal = t0 + 15 > minpos_w;
#pragma unroll
          for (int rb = 0; rb < R; ++rb)
            prefill_update<CT, D>(buf[j].scores(qf[rb]), pv, st[rb], t0, pos[rb], causal,
                                  a.qk_scale, lane);
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
        if (rr < rows) {
          const int tok = rr / G, g = rr - tok * G;
          const int64_t orow = (int64_t)(q0 + tok) * Hq + hk * G + g;
          const float inv = a.v_scale / l_run;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x[VE];
#pragma unroll
            for (int r = 0; r < VE; ++r) x[r] = st[rb].acc[r][i] * inv;
            store_run<CT, VE>(a.out, orow * D + VE * (4 * (lane >> 4) + i), x);
          }
        }
      }
    }
  }
}

// The shared-prefix part of a cascade decode: every sequence's query heads
// (rows s * G + g of one KV head) against one split of the prefix's tiles, no
// mask (every query sits past the whole prefix).  Each row leaves its partial
// state (running max in log2 units, sum, unnormalised accumulator) in the
// balanced merge's slot layout; the merge adds the sequence's own tail.
template <int CT, int D, int R, int NBUF>
__global__ __launch_bounds__(kPrefillWaves * 64) void shared_prefix_kernel(PrefixArgs a) {
  using T = Tile<CT, D>;
  constexpr int VE = T::VE;
  constexpr int NW = kPrefillWaves;
  constexpr int ROWS_W = 16 * R;
  constexpr int ROWS_G = ROWS_W * NW;
  const int split = blockIdx.z, hk = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group, Hq = a.num_q_heads, bs = a.block_size;
  const int rows = a.num_seqs * G;
  const int ntiles = a.prefix_len / 16;
  const int k0 = (int)((int64_t)split * ntiles / a.splits);
  const int k1 = (int)((int64_t)(split + 1) * ntiles / a.splits);
  const int64_t head_rows = (int64_t)hk * bs;
  const int64_t block_rows = (int64_t)a.num_kv_heads * bs;
  __shared__ int32_t sm_blk[kPrefillChunkTiles];

  for (int row_g0 = blockIdx.x * ROWS_G; row_g0 < rows; row_g0 += gridDim.x * ROWS_G) {
    const int row_w0 = row_g0 + wave * ROWS_W;
    const bool live = row_w0 < rows;
    typename T::QFrag qf[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
      const int rr = row_w0 + 16 * rb + (lane & 15);
      const bool valid = rr < rows;
      const int s = valid ? rr / G : 0;
      const int g = valid ? rr - s * G : 0;
      qf[rb] = T::load_q(static_cast<const QElem<CT>*>(a.q) + ((int64_t)s * Hq + hk * G + g) * D,
                         valid, lane);
    }
    Softmax<VE> st[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb)
#pragma unroll
      for (int r = 0; r < VE; ++r) st[rb].acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c0 = k0; c0 < k1; c0 += kPrefillChunkTiles) {
      const int c1 = min(k1, c0 + kPrefillChunkTiles);
      __syncthreads();
      for (int i = threadIdx.x; i < c1 - c0; i += NW * 64) sm_blk[i] = a.blocks[((c0 + i) * 16) / bs];
      __syncthreads();
      if (!live) continue;
      for (int k = c0; k < c1; k += NBUF) {
        T buf[NBUF];
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          const int t = min(k + j, c1 - 1);
          buf[j].load(a.kc, a.vc, (int64_t)sm_blk[t - c0] * block_rows + head_rows + ((t * 16) % bs),
                      lane);
        }
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          if (k + j >= c1) break;
          const typename T::PV pv = buf[j].pack_v();
#pragma unroll
          for (int rb = 0; rb < R; ++rb)
            prefill_update<CT, D>(buf[j].scores(qf[rb]), pv, st[rb], 0, 0, false, a.qk_scale, lane);
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
        if (rr < rows) {
          const int s = rr / G, g = rr - s * G;
          const int64_t slot = a.slot0 + ((int64_t)s * a.num_kv_heads + hk) * a.splits + split;
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
  hipLaunchKernelGGL((shared_prefix_kernel<CT, D, 2, 2>), grid, dim3(kPrefillWaves * 64), 0, stream, a);
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
  hipLaunchKernelGGL((prefill_kernel<CT, D, R, 2>), grid, dim3(kPrefillWaves * 64), 0, stream, a);
  return hipGetLastError();
}

template <int CT, int D>
hipError_t launch_d(const PrefillArgs& a, hipStream_t stream) {
  switch (a.rows_per_wave) {
    case 16: return launch_r<CT, D, 1>(a, stream);
    case 32: return launch_r<CT, D, 2>(a, stream);
    case 64:  // f32 fragments are twice as large: 64 rows would spill
      if constexpr (CT != PKV_F32) return launch_r<CT, D, 4>(a, stream);
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
