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
// * Append (the step's KV write folded into the decode): the wavefront that
//   holds a (sequence, KV head) pair's last tile reads the new token's rows
//   from k / v instead of the pool (a per-lane address choice, no extra
//   latency) and also stores them to their slot.
#include "e4m3.h"
#include "pkv_internal.h"
#include "tile.h"

namespace pkv {
namespace {

#ifndef PKV_DECODE_RING
#define PKV_DECODE_RING 2
#endif

constexpr int kChunkTiles = 1024;  // block ids staged in LDS per pass (4 KiB)

// Split-K partial rows in the workspace: a lane holds, for each i, the VE
// consecutive columns d = VE (4 q + i) .. + VE - 1 (q = lane / 16).  They are
// stored permuted so that the four lanes of a row write 64 contiguous bytes
// per store instruction (four of them, one per q, at float 4 P, P = (i VE/4 +
// q4) 4 + q) instead of four 16-byte pieces 128 bytes apart: partial-line
// writes behind which the next loads of the wavefront wait.  part_pos is the
// float offset of the chunk (i, q4) of lane group q; part_d0 the first column
// of chunk P.
template <int VE>
__device__ __forceinline__ int part_pos(int i, int q4, int q) {
  return ((i * (VE / 4) + q4) * 4 + q) * 4;
}
template <int VE>
__device__ __forceinline__ int part_d0(int P) {
  const int q = P & 3, t = P >> 2, q4 = t % (VE / 4), i = t / (VE / 4);
  return VE * (4 * q + i) + 4 * q4;
}
// Block tables read as constant memory (uniform indices: scalar loads).
typedef const __attribute__((address_space(4))) int32_t* ctab;
// Balanced split: work units charged for starting a piece, in tiles.  A piece
// start (q rows, block ids, the partial write) costs two to three bf16 tile
// times on MI355X; an E4M3 tile streams in half the time, so the same start
// costs about four of them.  bf16 takes 3 (Qwen-shaped call: 1 -> 51.2 us,
// 2 -> 49.8, 3 -> 49.5, 4 -> 50.7), but 2 for the tails of a shared-prefix
// call, whose many short pairs all end in pieces (256-sequence batch: 110.1 us
// at 2, 112.1 at 3).
__host__ __device__ constexpr int piece_cost(int ct, bool cascade) {
  return ct == PKV_FP8_E4M3 ? 4 : ct == PKV_BF16 ? (cascade ? 2 : 3) : 1;
}

// The new token's K and V rows of one KV head, one 16-byte chunk per lane
// (lanes [0, CH) carry K, [CH, 2 CH) carry V): the KV write of one row, split
// into its load and its store so the load can be issued early.
template <int CT, int D>
struct NewRow {
  static constexpr int IB = CT == PKV_F32 ? 4 : 2;  // new rows: f32 for f32 pools, else bf16
  static constexpr int CH = D * IB / 16;            // 16-byte chunks per row, <= 32
  u32x4 x;

  __device__ __forceinline__ void load(const DecodeArgs& a, int s, int h, int lane) {
    const int64_t src = (int64_t)s * a.num_kv_heads + h;
    const int is_v = lane >= CH;
    const int c = lane - is_v * CH;
    if (lane < 2 * CH)
      x = *reinterpret_cast<const u32x4*>(static_cast<const char*>(is_v ? a.vn : a.kn) +
                                          src * D * IB + c * 16);
  }
  __device__ __forceinline__ void store(const DecodeArgs& a, int32_t slot, int h, int lane) const {
    const int64_t blk = slot / a.block_size;
    const int64_t dst = (blk * a.num_kv_heads + h) * a.block_size + (slot - blk * a.block_size);
    const int is_v = lane >= CH;
    const int c = lane - is_v * CH;
    if (lane >= 2 * CH) return;
    char* pool = static_cast<char*>(const_cast<void*>(is_v ? a.vc : a.kc));
    if constexpr (CT == PKV_FP8_E4M3) {
      const float inv = is_v ? a.inv_v : a.inv_k;
      *reinterpret_cast<u32x2*>(pool + dst * D + c * 8) =
          u32x2{e4m3x4_from_bf16x4(x[0], x[1], inv), e4m3x4_from_bf16x4(x[2], x[3], inv)};
    } else {
      *reinterpret_cast<u32x4*>(pool + dst * D * IB + c * 16) = x;
    }
  }
};

// The KV write of sequence s's new token, KV head h, when nothing attends it
// in this call (an empty sequence).
template <int CT, int D>
__device__ __forceinline__ void append_row(const DecodeArgs& a, int s, int h, int lane) {
  const int32_t slot = a.slots[s];
  if (slot < 0) return;
  NewRow<CT, D> r;
  r.load(a, s, h, lane);
  r.store(a, slot, h, lane);
}

// One 16-token tile: scores, masking of tokens >= ctx, online-softmax update, P.V.
template <int CT, int D>
__device__ __forceinline__ void process_tile(Tile<CT, D>& t, const typename Tile<CT, D>::QFrag& qf,
                                             Softmax<D / 16>& st, int t0, int ctx, float qk_scale,
                                             int lane) {
  constexpr int VE = D / 16;
  const f32x4 sacc = t.scores(qf);
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = sacc[i] * qk_scale;
  if (t0 + 16 > ctx) {  // ragged last tile: drop tokens >= ctx by select
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ok[i] = t0 + 4 * (lane >> 4) + i < ctx;
      sc[i] = ok[i] ? sc[i] : kNegInf;
    }
    t.mask_rows(ok);
  }
  const float bm = max_over_lane_groups(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
  const float m_new = fmaxf(st.m, bm);  // finite: every tile holds >= 1 live token
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
#pragma unroll
  for (int r = 0; r < VE; ++r) st.acc[r] *= alpha;
  st.l = st.l * alpha + t.pv(p, st.acc);
  st.m = m_new;
}

// E4M3 (without the folded write) at four wavefronts per SIMD: one more
// workgroup resident per CU for the many short pairs auto mode sends here
// (512-sequence E4M3 batch: 194.0 -> 192.6 us); the other variants would spill.
template <int CT, int D, int NW, int NBUF, bool APPEND, bool NT>
__global__ __launch_bounds__(NW * 64, (CT == PKV_FP8_E4M3 && !APPEND) ? 4 : 1) void decode_partition_kernel(DecodeArgs a) {
  using T = Tile<CT, D>;
  constexpr int VE = T::VE;
  const int part = blockIdx.x, hk = blockIdx.y;
  // grid row z takes sequence seq_order[z] (e.g. longest first), or z
  const int s = a.seq_order ? a.seq_order[blockIdx.z] : (int)blockIdx.z;
  if (s < 0 || s >= a.num_seqs) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
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

  Softmax<VE> st;
#pragma unroll
  for (int r = 0; r < VE; ++r) st.acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Append: the wavefront holding tile ntiles-1 writes the new token's rows to
  // their slot (loaded now, stored at the end) and, when that slot is position
  // ctx-1 (found through the tile's block id), reads the rows from k / v.
  const int32_t slot_new = APPEND && tile_end == ntiles && ntiles > 0 ? a.slots[s] : -1;
  const bool owns_last = slot_new >= 0 && wave == ((ntiles - 1 - tile_begin) % kChunkTiles) % NW;
  const int r_new = (ctx - 1) & 15;
  const int64_t off_new = ctx > 0 ? (ctx - 1) % bs : 0;
  const int64_t new_row = (int64_t)s * a.num_kv_heads + hk;
  const void* kn = static_cast<const QElem<CT>*>(a.kn) + new_row * D;
  const void* vn = static_cast<const QElem<CT>*>(a.vn) + new_row * D;
  NewRow<CT, D> nrow;
  if (owns_last) nrow.load(a, s, hk, lane);

  // The partition's tiles are taken in chunks of up to kChunkTiles.  For each
  // chunk the workgroup first copies the block id of every tile into LDS (one
  // cooperative pass over the table), so inside the loop an address costs an
  // LDS read, whose wait does not touch the in-flight K/V loads.  Wave w takes
  // tiles c0 + w + NW*k.  Past the wave's last tile, indices clamp to it (in
  // bounds, result unused), so every batch issues the same loads.
  __shared__ int32_t sm_blk[kChunkTiles];
  for (int c0 = tile_begin; c0 < tile_end; c0 += kChunkTiles) {
    const int c1 = min(tile_end, c0 + kChunkTiles);
    if (c0 > tile_begin) __syncthreads();  // every wave is done with the previous chunk
    for (int i = threadIdx.x; i < c1 - c0; i += NW * 64) sm_blk[i] = table[((c0 + i) * 16) / bs];
    __syncthreads();
    const int first = c0 + wave;
    const int n_my = first < c1 ? (c1 - first + NW - 1) / NW : 0;
    auto tile_of = [&](int k) { return first + NW * min(k, n_my - 1); };
    // Batches of NBUF tiles: all their loads are issued back to back, then the
    // tiles are computed in order, each waiting only for its own loads.  No
    // load is in flight across the loop's back edge.
    for (int k = 0; k < n_my; k += NBUF) {
      T buf[NBUF];
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        const int t = tile_of(k + j);
        const int32_t blk = sm_blk[t - c0];
        const int64_t row = (int64_t)blk * block_rows + head_rows + ((t * 16) % bs);
        const int rsub = owns_last && k + j < n_my && t == ntiles - 1 &&
                                 (int64_t)blk * bs + off_new == slot_new ? r_new : -1;
        buf[j].template load_sub<NT>(a.kc, a.vc, row, lane, rsub, kn, vn, a.inv_k, a.inv_v);
      }
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        if (k + j >= n_my) break;
        process_tile<CT, D>(buf[j], qf, st, tile_of(k + j) * 16, ctx, a.qk_scale, lane);
      }
    }
  }
  if (owns_last) nrow.store(a, slot_new, hk, lane);
  if (APPEND && ntiles == 0 && part == 0 && wave == 0) append_row<CT, D>(a, s, hk, lane);
  float m_run = st.m, l_run = st.l;
  f32x4* acc = st.acc;
  // per-lane sums cover tokens 4*(lane/16)+i only; add the four lane groups
  l_run = sum_over_lane_groups(l_run);

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
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int w = 0; w < VE / 4; ++w)
        *reinterpret_cast<f32x4*>(a.ws_acc + prow * D + part_pos<VE>(i, w, lane >> 4)) =
            f32x4{acc[4 * w][i], acc[4 * w + 1][i], acc[4 * w + 2][i], acc[4 * w + 3][i]};
    if (lane < 16) *reinterpret_cast<f32x2*>(a.ws_ml + prow * 2) = f32x2{m_run, l_run};
  }
}

// Merge the partitions of one (sequence, query head).  256 threads: thread t
// owns the four columns 4 (t % CW) .. of the rows (partitions) t / CW,
// t / CW + RS, ... (CW = D / 4 column quads, RS = 256 / CW row sets), with
// kRows of them loaded before any is used; the common max M and the total L
// come from a block reduction over the (max, sum) pairs, and the RS partial
// rows are added in row-set order, so the result does not depend on timing.
template <int CT, int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  constexpr int CW = D / 4, RS = 256 / CW, kRows = 8;
  __shared__ float red[2][4];
  __shared__ f32x4 part[RS][CW];
  const int h = blockIdx.x, s = blockIdx.y, t = threadIdx.x;
  const int wv = t >> 6, c = t % CW, r = t / CW;
  const int ctx = a.lens[s];
  const int ntiles = (ctx + 15) >> 4;
  if (ntiles <= a.part_tiles) return;  // written directly by its only partition
  const int np = (ntiles + a.part_tiles - 1) / a.part_tiles;
  const int64_t prow0 = ((int64_t)s * a.num_q_heads + h) * a.num_parts;
  const float* ml = a.ws_ml + prow0 * 2;
  const float* acc = a.ws_acc + prow0 * D + 4 * c;

  // the first batch of rows goes out before the reductions that need M
  f32x4 v[kRows];
  float mr[kRows];
  auto load_rows = [&](int p0) {
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const int p = p0 + j * RS;
      v[j] = p < np ? *reinterpret_cast<const f32x4*>(acc + (int64_t)p * D) : f32x4{0.f, 0.f, 0.f, 0.f};
      mr[j] = p < np ? ml[2 * p] : kNegInf;
    }
  };
  load_rows(r);

  float m = kNegInf;
  for (int p = t; p < np; p += 256) m = fmaxf(m, ml[2 * p]);
  m = wave_max_f32(m);
  if ((t & 63) == 0) red[0][wv] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float l = 0.f;
  for (int p = t; p < np; p += 256) l += __builtin_amdgcn_exp2f(ml[2 * p] - M) * ml[2 * p + 1];
  l = wave_sum_f32(l);
  if ((t & 63) == 0) red[1][wv] = l;

  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = r;; p0 += kRows * RS) {
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const int p = p0 + j * RS;
      if (p < np) o += __builtin_amdgcn_exp2f(mr[j] - M) * v[j];
    }
    if (p0 + kRows * RS >= np) break;
    load_rows(p0 + kRows * RS);
  }
  part[r][c] = o;
  __syncthreads();
  if (t >= CW) return;
  f32x4 sum = part[0][c];
#pragma unroll
  for (int i = 1; i < RS; ++i) sum += part[i][c];
  const float L = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  const float inv = a.v_scale / L;
  const float x[4] = {sum[0] * inv, sum[1] * inv, sum[2] * inv, sum[3] * inv};
  store_run<CT, 4>(a.out, ((int64_t)s * a.num_q_heads + h) * D + part_d0<D / 16>(c), x);
}

// ---------------------------------------------------------------------------
// Balanced split.  The work of one call is the flattened list of tiles of all
// segments (sequence s, KV head h) in (s, h, tile) order.  num_workers
// wavefronts each take an equal contiguous run of it, so every wavefront
// streams the same number of bytes and they finish together, whatever the
// spread of context lengths.  A run covers parts of one or more segments; a
// segment covered by a single run is finalised in place, otherwise each run's
// piece leaves its partial state in slot (worker + segment) and the merge
// kernel combines the pieces in worker order.
// ---------------------------------------------------------------------------

template <int CT, int D>
__device__ void write_zero_rows(const DecodeArgs& a, int s, int lane) {
  constexpr int EB = CT == PKV_F32 ? 4 : 2;
  char* o = static_cast<char*>(a.out) + (int64_t)s * a.num_q_heads * D * EB;
  const int n16 = a.num_q_heads * D * EB / 16;
  for (int i = lane; i < n16; i += 64) reinterpret_cast<u32x4*>(o)[i] = u32x4{0, 0, 0, 0};
}

// Orders one wavefront's LDS accesses across its lanes: what any lane wrote
// before is visible to every lane after, and no access moves across it.
// Emits no barrier instruction (a wavefront's LDS operations already complete
// in issue order); it only fixes the compiler's order.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// At most two wavefronts per SIMD (the split runs 4 or 8 workers per CU): with
// the tighter three-per-SIMD budget the loop lost its load scheduling (the
// Qwen-shaped batch: 44.5 us per launch at two, 52 us when it spilled at three).
template <int CT, int D, int NBUF, bool APPEND, bool NT>
__global__ __launch_bounds__(256, 2) void decode_balanced_kernel(DecodeArgs a) {
  using T = Tile<CT, D>;
  constexpr int VE = T::VE;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = a.num_workers;
  if (w >= W) return;
  const int S = a.num_seqs, Hkv = a.num_kv_heads, G = a.group, bs = a.block_size;

  // The split is made in work units: a (sequence, KV head) pair with n tiles
  // costs n + kPieceCost units, the first kPieceCost standing for the fixed
  // cost of starting a piece (its q rows, block ids and partial state), so a
  // run that crosses into a new pair gets fewer tiles.
  // Lengths of up to kScanRegs * 64 sequences stay in registers (lane l
  // holds sequences l, l+64, ...), so a piece start reads its length with a
  // readlane instead of a dependent load; longer batches re-read the rest.
  // Sequences with no tokens have no tiles: worker s % W writes their zero rows.
  constexpr int kScanRegs = 8;
  const int kPieceCost = piece_cost(CT, a.cascade != 0);
  auto units = [kPieceCost](uint32_t n) { return n ? n + (uint32_t)kPieceCost : 0u; };
  int creg[kScanRegs];
#pragma unroll
  for (int i = 0; i < kScanRegs; ++i) creg[i] = 0;
  int64_t total = 0;
  for (int c = 0, r = 0; c < S; c += 64, ++r) {
    const int s = c + lane;
    const int ctx = s < S ? max(0, a.lens[s] - a.len_offset) : 0;
    const uint32_t n = (uint32_t)((ctx + 15) >> 4);
    if (r < kScanRegs) creg[r] = ctx;
    total += wave_sum_u32(units(n));
    uint64_t zmask = __ballot(s < S && ctx == 0 && s % W == w);
    while (zmask) {
      const int l = __builtin_ctzll(zmask);
      zmask &= zmask - 1;
      write_zero_rows<CT, D>(a, c + l, lane);
      if constexpr (APPEND)
        for (int h = 0; h < Hkv; ++h) append_row<CT, D>(a, c + l, h, lane);
      if (lane < Hkv) {
        a.ws_meta[2 * ((int64_t)(c + l) * Hkv + lane)] = -1;
        a.ws_meta[2 * ((int64_t)(c + l) * Hkv + lane) + 1] = -1;
      }
      for (int h = 64; h < Hkv; ++h) {  // more than 64 KV heads: rest by lane 0
        if (lane == 0) {
          a.ws_meta[2 * ((int64_t)(c + l) * Hkv + h)] = -1;
          a.ws_meta[2 * ((int64_t)(c + l) * Hkv + h) + 1] = -1;
        }
      }
    }
  }
  total *= Hkv;
  if (total == 0) return;
  const int64_t chunk = (total + W - 1) / W;
  const int64_t x0 = (int64_t)w * chunk;
  const int64_t x1 = min(total, x0 + chunk);
  if (x0 >= x1) return;

  // Sequence holding unit x0, and the units before it.
  int s_cur = 0;
  int64_t p_cur = 0;
  {
    int64_t base = 0;
    for (int c = 0, r = 0; c < S; c += 64, ++r) {
      const int s = c + lane;
      uint32_t n;
      if (r < kScanRegs) n = (uint32_t)((creg[r] + 15) >> 4);
      else n = s < S ? (uint32_t)((max(0, a.lens[s] - a.len_offset) + 15) >> 4) : 0u;
      const uint32_t u = units(n);
      const uint32_t incl = wave_incl_scan_u32(u);
      const int64_t tot = (int64_t)Hkv * __builtin_amdgcn_readlane(incl, 63);
      if (x0 < base + tot) {
        const uint64_t hit = __ballot(x0 < base + (int64_t)Hkv * incl);
        const int l = __builtin_ctzll(hit);
        s_cur = c + l;
        p_cur = base + (int64_t)Hkv * __builtin_amdgcn_readlane(incl - u, l);
        break;
      }
      base += tot;
    }
  }

  const int g = lane & 15;
  const bool g_ok = g < G;
  // States of this run's pieces (partial states, or the final rows of a pair
  // the run holds whole), staged in LDS and written out at the end of the run
  // (or when the buffer is full): a global store in the middle of the run
  // would hold up the next piece's loads until it completes.  Slot: G rows of
  // D floats, then G (max, sum) pairs; meta: (workspace slot, or -1 for final
  // rows; segment; the segment's piece record when this is its last piece).
  constexpr int kPendFloats = 4096;  // 16 KiB per wavefront
  __shared__ __attribute__((aligned(16))) float sm_pend[4][kPendFloats];
  __shared__ int4 sm_pend_meta[4][16];
  const int wv = threadIdx.x >> 6;
  float* const pend = sm_pend[wv];
  int4* const pend_meta = sm_pend_meta[wv];
  const int kSlotFloats = (G * (D + 2) + 3) & ~3;
  const int kPendSlots = min(16, kPendFloats / kSlotFloats);
  int npend = 0;
  auto flush = [&]() {
    wave_lds_sync();  // slots and meta were written by other lanes
    for (int j = 0; j < npend; ++j) {
      const int4 meta = pend_meta[j];
      const float* slot = pend + j * kSlotFloats;
      if (meta.x < 0) {  // a whole pair: G consecutive output rows
        const int sj = meta.y / Hkv, hj = meta.y - sj * Hkv;
        const int64_t row0 = (int64_t)sj * a.num_q_heads + hj * G;
        for (int u = lane; u < G * D / 4; u += 64) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(slot + 4 * u);
          const float xv[4] = {v[0], v[1], v[2], v[3]};
          store_run<CT, 4>(a.out, row0 * D + 4 * u, xv);
        }
        if (lane == 0) {
          a.ws_meta[2 * (int64_t)meta.y] = meta.z;
          a.ws_meta[2 * (int64_t)meta.y + 1] = meta.w;
        }
        continue;
      }
      float* dst = a.ws_acc + (int64_t)meta.x * G * D;
      for (int u = lane; u < G * D / 4; u += 64)
        *reinterpret_cast<f32x4*>(dst + 4 * u) = *reinterpret_cast<const f32x4*>(slot + 4 * u);
      if (lane < G)
        *reinterpret_cast<f32x2*>(a.ws_ml + ((int64_t)meta.x * G + lane) * 2) =
            *reinterpret_cast<const f32x2*>(slot + G * D + 2 * lane);
      if (lane == 0 && meta.z != INT32_MIN) {
        a.ws_meta[2 * (int64_t)meta.y] = meta.z;
        a.ws_meta[2 * (int64_t)meta.y + 1] = meta.w;
      }
    }
    wave_lds_sync();  // every lane is done reading before the slots are reused
    npend = 0;
  };
  int64_t x = x0;
  int32_t carry[NBUF] = {};  // first-batch block ids of the next piece, loaded ahead
  bool has_carry = false;
  // the run's sequences lie in the 64-sequence chunk of s_cur and, for runs
  // that cross it, the next one: keep those two registers
  const int r0 = s_cur >> 6;
  int cw0 = 0, cw1 = 0;
#pragma unroll
  for (int i = 0; i < kScanRegs; ++i) {
    if (i == r0) cw0 = creg[i];
    if (i == r0 + 1) cw1 = creg[i];
  }
  auto ctx_of = [&](int sq) -> int {  // sq wave-uniform
    const int r = sq >> 6;
    if (r == r0 && r < kScanRegs) return __builtin_amdgcn_readlane(cw0, sq & 63);
    if (r == r0 + 1 && r < kScanRegs) return __builtin_amdgcn_readlane(cw1, sq & 63);
    return max(0, a.lens[sq] - a.len_offset);
  };
  while (x < x1 && s_cur < S) {
    const int ctx = ctx_of(s_cur);
    const int n = (ctx + 15) >> 4;
    if (n == 0) {
      ++s_cur;
      continue;
    }
    const int u = n + kPieceCost;
    const int64_t rel = x - p_cur;
    const int h = (int)(rel / u);
    if (h >= Hkv) break;  // cannot happen: x lies inside sequence s_cur's units
    const int vt = (int)(rel - (int64_t)h * u);          // unit range of this run
    const int ve = (int)min((int64_t)u, vt + (x1 - x));  // inside the pair: [vt, ve)
    const int tl = max(0, vt - kPieceCost);               // its tiles: [tl, te)
    const int te = max(0, ve - kPieceCost);
    const int seg = s_cur * Hkv + h;
    if (te <= tl) {  // the run holds only the pair's start-up units: no tiles here
      x += ve - vt;
      if (ve == u && h == Hkv - 1) {
        p_cur += (int64_t)Hkv * u;
        ++s_cur;
      }
      continue;
    }

    const int qh = h * G + g;
    const QElem<CT>* qrow = static_cast<const QElem<CT>*>(a.q) +
                            ((int64_t)s_cur * a.num_q_heads + (g_ok ? qh : 0)) * D;
    const typename T::QFrag qf = T::load_q(qrow, g_ok, lane);
    const int32_t* table = a.tables + (int64_t)s_cur * a.max_blocks;
    const int64_t head_rows = (int64_t)h * bs;
    const int64_t block_rows = (int64_t)Hkv * bs;

    Softmax<VE> st;
#pragma unroll
    for (int r = 0; r < VE; ++r) st.acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Append: the piece holding the pair's last tile writes the new token's rows
    // to their slot (loaded now, stored at the end) and, when that slot is
    // position ctx-1, reads them from k / v.
    const int32_t slot_new = APPEND && te == n ? a.slots[s_cur] : -1;
    const int r_new = (ctx - 1) & 15;
    const int64_t off_new = (ctx - 1) % bs;
    const int64_t new_row = (int64_t)s_cur * Hkv + h;
    const void* kn = static_cast<const QElem<CT>*>(a.kn) + new_row * D;
    const void* vn = static_cast<const QElem<CT>*>(a.vn) + new_row * D;
    NewRow<CT, D> nrow;
    if (slot_new >= 0) nrow.load(a, s_cur, h, lane);
    // Block ids of the next batch arrive one batch ahead, through scalar loads
    // (the tables are read-only here, so they are read as constant memory:
    // the ids never wait in the vector-memory queue behind the tile loads);
    // tiles past the piece clamp to its last tile (in bounds, result unused).
    const ctab ctable = (ctab)table;  // address-space cast: C-style only
    auto entry = [&](int t) { return ctable[(min(t, te - 1) * 16) / bs]; };
    int32_t ent_next[NBUF];
#pragma unroll
    for (int j = 0; j < NBUF; ++j) ent_next[j] = has_carry ? carry[j] : entry(tl + j);
    // When the run goes on into the next pair (the next KV head of this
    // sequence, or the next sequence with tokens), that piece starts at tile 0
    // of its table row: fetch its first block ids now, so the piece change
    // costs no dependent table read.
    const int64_t after = x + (ve - vt);
    has_carry = ve == u && x1 - after > kPieceCost;
    int s_next = s_cur;
    if (has_carry && h + 1 >= Hkv) {
      do ++s_next; while (s_next < S && ctx_of(s_next) == 0);
      has_carry = s_next < S;
    }
    const int te_next =
        has_carry ? (int)min((int64_t)((ctx_of(s_next) + 15) >> 4), x1 - after - kPieceCost) : 1;
    const int32_t* table_next = a.tables + (int64_t)s_next * a.max_blocks;
    for (int k = tl; k < te; k += NBUF) {
      int32_t ent[NBUF];
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        ent[j] = ent_next[j];
        ent_next[j] = entry(k + NBUF + j);
      }
      if (has_carry && k == tl) {
#pragma unroll
        for (int j = 0; j < NBUF; ++j)
          carry[j] = ((ctab)table_next)[(min(j, te_next - 1) * 16) / bs];
      }
      T buf[NBUF];
      if (APPEND && slot_new >= 0 && k + NBUF >= n) {
        // the batch holding the pair's last tile: its new token's rows come
        // from k / v (a per-lane address choice) when the slot is position ctx-1
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          const int t = min(k + j, te - 1);
          const int32_t blk = ent[j];
          const int64_t row = (int64_t)blk * block_rows + head_rows + ((t * 16) % bs);
          const int rsub = k + j == n - 1 && (int64_t)blk * bs + off_new == slot_new ? r_new : -1;
          buf[j].template load_sub<NT>(a.kc, a.vc, row, lane, rsub, kn, vn, a.inv_k, a.inv_v);
        }
      } else {
        // every other batch: plain tile loads, nothing computed in front of them
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          const int t = min(k + j, te - 1);
          const int64_t row = (int64_t)ent[j] * block_rows + head_rows + ((t * 16) % bs);
          buf[j].template load<NT>(a.kc, a.vc, row, lane);
        }
      }
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        if (k + j >= te) break;
        process_tile<CT, D>(buf[j], qf, st, (k + j) * 16, ctx, a.qk_scale, lane);
      }
    }
    if (slot_new >= 0) nrow.store(a, slot_new, h, lane);
    float l_run = st.l;
    l_run = sum_over_lane_groups(l_run);

    const bool whole = tl == 0 && te == n && !a.cascade;  // cascade: always pieces
    if (npend == kPendSlots) flush();
    float* slot = pend + npend * kSlotFloats;
    if (whole) {
      // finalised in place (the rows in column order); its record says so
      if (g_ok) {
        const float inv = a.v_scale / l_run;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q4 = 0; q4 < VE / 4; ++q4)
            *reinterpret_cast<f32x4*>(slot + g * D + VE * (4 * (lane >> 4) + i) + 4 * q4) =
                f32x4{st.acc[4 * q4][i] * inv, st.acc[4 * q4 + 1][i] * inv, st.acc[4 * q4 + 2][i] * inv,
                      st.acc[4 * q4 + 3][i] * inv};
      }
      if (lane == 0) pend_meta[npend] = int4{-1, seg, -1, -1};
      ++npend;
    } else {
      if (g_ok) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q4 = 0; q4 < VE / 4; ++q4)
            *reinterpret_cast<f32x4*>(slot + g * D + VE * (4 * (lane >> 4) + i) + 4 * q4) =
                f32x4{st.acc[4 * q4][i], st.acc[4 * q4 + 1][i], st.acc[4 * q4 + 2][i],
                      st.acc[4 * q4 + 3][i]};
        if (lane < 16) *reinterpret_cast<f32x2*>(slot + G * D + 2 * g) = f32x2{st.m, l_run};
      }
      if (lane == 0) {
        // the segment's last piece records where its pieces are
        const int64_t first_tile_unit = p_cur + (int64_t)h * u + kPieceCost;
        pend_meta[npend] = te == n ? int4{w + seg, seg, (int32_t)(first_tile_unit / chunk), w}
                                   : int4{w + seg, seg, INT32_MIN, 0};
      }
      ++npend;
    }
    x += ve - vt;
    if (ve == u && h == Hkv - 1) {
      p_cur += (int64_t)Hkv * u;
      ++s_cur;
    }
  }
  flush();
}

// ---------------------------------------------------------------------------
// Split-K partitions streamed by persistent wavefronts.  The tasks of a call
// are the (sequence, KV head, partition) triples in that order, a partition
// being part_tiles tiles of one pair (the last one shorter).  num_workers
// wavefronts each take an equal contiguous run of tasks and stream them back
// to back: the next task's first block ids are loaded during the current
// task's first batch, and q is reloaded only when the pair changes, so a
// partition boundary costs no dependent round trip.  Every partition's state
// is computed exactly as by decode_partition_kernel with one wavefront (same
// tiles, same order), so the partial states, and the reduce, are the same.
// ---------------------------------------------------------------------------
template <int CT, int D, int NBUF, bool APPEND, bool NT>
__global__ __launch_bounds__(256, 1) void decode_partition_run_kernel(DecodeArgs a) {
  using T = Tile<CT, D>;
  constexpr int VE = T::VE;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = a.num_workers;
  if (w >= W) return;
  const int S = a.num_seqs, Hkv = a.num_kv_heads, G = a.group, bs = a.block_size;
  const int PT = a.part_tiles;
  auto parts_of = [PT](int ctx) { return ctx > 0 ? (((ctx + 15) >> 4) + PT - 1) / PT : 0; };

  // Task count; sequences with no tokens have no task: worker s % W writes
  // their zero rows.
  int64_t total = 0;
  for (int c = 0; c < S; c += 64) {
    const int s = c + lane;
    const int ctx = s < S ? a.lens[s] : 0;
    total += wave_sum_u32((uint32_t)parts_of(ctx));
    uint64_t zmask = __ballot(s < S && ctx <= 0 && s % W == w);
    while (zmask) {
      const int l = __builtin_ctzll(zmask);
      zmask &= zmask - 1;
      write_zero_rows<CT, D>(a, c + l, lane);
      if constexpr (APPEND)
        for (int h = 0; h < Hkv; ++h) append_row<CT, D>(a, c + l, h, lane);
    }
  }
  total *= Hkv;
  if (total == 0) return;
  const int64_t chunk = (total + W - 1) / W;
  const int64_t t0 = (int64_t)w * chunk;
  const int64_t t1 = min(total, t0 + chunk);
  if (t0 >= t1) return;

  // Sequence holding task t0, and the tasks before it.
  int s_cur = 0;
  int64_t p_cur = 0;
  {
    int64_t base = 0;
    for (int c = 0; c < S; c += 64) {
      const int s = c + lane;
      const uint32_t u = s < S ? (uint32_t)parts_of(a.lens[s]) : 0u;
      const uint32_t incl = wave_incl_scan_u32(u);
      const int64_t tot = (int64_t)Hkv * __builtin_amdgcn_readlane(incl, 63);
      if (t0 < base + tot) {
        const uint64_t hit = __ballot(t0 < base + (int64_t)Hkv * incl);
        const int l = __builtin_ctzll(hit);
        s_cur = c + l;
        p_cur = base + (int64_t)Hkv * __builtin_amdgcn_readlane(incl - u, l);
        break;
      }
      base += tot;
    }
  }

  const int g = lane & 15;
  const bool g_ok = g < G;
  const int64_t block_rows = (int64_t)Hkv * bs;
  // States of this wavefront's partitions (partial states, or the final rows
  // of a pair held by one partition), staged in LDS and written out when the
  // buffer is full and at the end of the run, so that no store sits in front
  // of the next partition's loads.  Slot: G rows of D floats, then G (max,
  // sum) pairs.
  constexpr int kPendFloats = 8192;  // 32 KiB per wavefront
  __shared__ __attribute__((aligned(16))) float sm_pend[4][kPendFloats];
  __shared__ int2 sm_pend_meta[4][64];
  const int wv = threadIdx.x >> 6;
  float* const pend = sm_pend[wv];
  int2* const pend_meta = sm_pend_meta[wv];
  const int kSlotFloats = (G * (D + 2) + 3) & ~3;
  const int kPendSlots = min(64, kPendFloats / kSlotFloats);
  int npend = 0;
  auto flush = [&]() {
    wave_lds_sync();  // slots and meta were written by other lanes
    for (int j = 0; j < npend; ++j) {
      const int2 meta = pend_meta[j];  // (pair, partition or -1 for final rows)
      const int sj = meta.x / Hkv, hj = meta.x - sj * Hkv;
      const int64_t row0 = (int64_t)sj * a.num_q_heads + hj * G;
      const float* slot = pend + j * kSlotFloats;
      if (meta.y < 0) {  // the pair's final rows: G consecutive output rows
        for (int u = lane; u < G * D / 4; u += 64) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(slot + 4 * u);
          const float xv[4] = {v[0], v[1], v[2], v[3]};
          store_run<CT, 4>(a.out, row0 * D + 4 * u, xv);
        }
        continue;
      }
      for (int u = lane; u < G * D / 4; u += 64) {
        const int gg = u / (D / 4), c4 = u - gg * (D / 4);
        *reinterpret_cast<f32x4*>(a.ws_acc + ((row0 + gg) * a.num_parts + meta.y) * D + 4 * c4) =
            *reinterpret_cast<const f32x4*>(slot + 4 * u);
      }
      if (lane < G)
        *reinterpret_cast<f32x2*>(a.ws_ml + ((row0 + lane) * a.num_parts + meta.y) * 2) =
            *reinterpret_cast<const f32x2*>(slot + G * D + 2 * lane);
    }
    wave_lds_sync();  // every lane is done reading before the slots are reused
    npend = 0;
  };
  typename T::QFrag qf;
  int q_seg = -1;            // pair whose q rows qf holds
  int32_t carry[NBUF] = {};  // first-batch block ids of the next task, loaded ahead
  bool has_carry = false;
  for (int64_t t = t0; t < t1 && s_cur < S;) {
    const int ctx = max(0, a.lens[s_cur]);
    const int n = (ctx + 15) >> 4;
    const int np = (n + PT - 1) / PT;
    if (np == 0) {
      ++s_cur;
      continue;
    }
    const int64_t rel = t - p_cur;
    const int h = (int)(rel / np), part = (int)(rel - (int64_t)h * np);
    const int tl = part * PT, te = min(n, tl + PT);
    const int seg = s_cur * Hkv + h;
    const int qh = h * G + g;
    if (seg != q_seg) {
      const QElem<CT>* qrow = static_cast<const QElem<CT>*>(a.q) +
                              ((int64_t)s_cur * a.num_q_heads + (g_ok ? qh : 0)) * D;
      qf = T::load_q(qrow, g_ok, lane);
      q_seg = seg;
    }
    const int32_t* table = a.tables + (int64_t)s_cur * a.max_blocks;
    const int64_t head_rows = (int64_t)h * bs;
    const ctab ctable = (ctab)table;  // address-space cast: C-style only
    auto entry = [&](int tt) { return ctable[(min(tt, te - 1) * 16) / bs]; };
    int32_t ent_next[NBUF];
#pragma unroll
    for (int j = 0; j < NBUF; ++j) ent_next[j] = has_carry ? carry[j] : entry(tl + j);
    // the next task: the next partition of this pair, the next KV head, or
    // the next sequence with tokens; its first block ids come with the first
    // batch of this one
    int s_next = s_cur, tl_next = te, te_next = 0;
    if (te < n) {
      te_next = min(n, te + PT);
    } else if (h + 1 < Hkv) {
      tl_next = 0;
      te_next = min(n, PT);
    } else {
      do ++s_next; while (s_next < S && a.lens[s_next] <= 0);
      tl_next = 0;
      te_next = s_next < S ? min((a.lens[s_next] + 15) >> 4, PT) : 0;
    }
    has_carry = t + 1 < t1 && te_next > tl_next;
    const int32_t* table_next = a.tables + (int64_t)min(s_next, S - 1) * a.max_blocks;

    Softmax<VE> st;
#pragma unroll
    for (int r = 0; r < VE; ++r) st.acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Append: the partition holding the pair's last tile writes the new
    // token's rows to their slot (loaded now, stored at the end) and, when
    // that slot is position ctx-1, reads them from k / v.
    const int32_t slot_new = APPEND && te == n ? a.slots[s_cur] : -1;
    const int r_new = (ctx - 1) & 15;
    const int64_t off_new = (ctx - 1) % bs;
    const int64_t new_row = (int64_t)s_cur * Hkv + h;
    const void* kn = static_cast<const QElem<CT>*>(a.kn) + new_row * D;
    const void* vn = static_cast<const QElem<CT>*>(a.vn) + new_row * D;
    NewRow<CT, D> nrow;
    if (slot_new >= 0) nrow.load(a, s_cur, h, lane);
    for (int k = tl; k < te; k += NBUF) {
      int32_t ent[NBUF];
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        ent[j] = ent_next[j];
        ent_next[j] = entry(k + NBUF + j);
      }
      if (has_carry && k == tl) {
#pragma unroll
        for (int j = 0; j < NBUF; ++j)
          carry[j] = ((ctab)table_next)[(min(tl_next + j, te_next - 1) * 16) / bs];
      }
      T buf[NBUF];
      if (APPEND && slot_new >= 0 && k + NBUF >= n) {
        // the batch holding the pair's last tile: its new token's rows come
        // from k / v when the slot is position ctx-1
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          const int tt = min(k + j, te - 1);
          const int32_t blk = ent[j];
          const int64_t row = (int64_t)blk * block_rows + head_rows + ((tt * 16) % bs);
          const int rsub = k + j == n - 1 && (int64_t)blk * bs + off_new == slot_new ? r_new : -1;
          buf[j].template load_sub<NT>(a.kc, a.vc, row, lane, rsub, kn, vn, a.inv_k, a.inv_v);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          const int tt = min(k + j, te - 1);
          const int64_t row = (int64_t)ent[j] * block_rows + head_rows + ((tt * 16) % bs);
          buf[j].template load<NT>(a.kc, a.vc, row, lane);
        }
      }
#pragma unroll
      for (int j = 0; j < NBUF; ++j) {
        if (k + j >= te) break;
        process_tile<CT, D>(buf[j], qf, st, (k + j) * 16, ctx, a.qk_scale, lane);
      }
    }
    if (slot_new >= 0) nrow.store(a, slot_new, h, lane);
    const float m_run = st.m;
    const float l_run = sum_over_lane_groups(st.l);
    {
      // the state waits in LDS: a global store here would hold up the next
      // partition's loads until it completes
      if (npend == kPendSlots) flush();
      float* slot = pend + npend * kSlotFloats;
      if (np == 1) {  // one partition holds the whole context: the final rows, in column order
        const float inv = l_run > 0.f ? a.v_scale / l_run : 0.f;
        if (g_ok) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q4 = 0; q4 < VE / 4; ++q4)
              *reinterpret_cast<f32x4*>(slot + g * D + VE * (4 * (lane >> 4) + i) + 4 * q4) =
                  f32x4{st.acc[4 * q4][i] * inv, st.acc[4 * q4 + 1][i] * inv, st.acc[4 * q4 + 2][i] * inv,
                        st.acc[4 * q4 + 3][i] * inv};
        }
      } else if (g_ok) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q4 = 0; q4 < VE / 4; ++q4)
            *reinterpret_cast<f32x4*>(slot + g * D + part_pos<VE>(i, q4, lane >> 4)) =
                f32x4{st.acc[4 * q4][i], st.acc[4 * q4 + 1][i], st.acc[4 * q4 + 2][i], st.acc[4 * q4 + 3][i]};
        if (lane < 16) *reinterpret_cast<f32x2*>(slot + G * D + 2 * g) = f32x2{m_run, l_run};
      }
      if (lane == 0) pend_meta[npend] = int2{seg, np == 1 ? -1 : part};  // -1: final rows
      ++npend;
    }
    ++t;
    if (part == np - 1 && h == Hkv - 1) {
      p_cur += (int64_t)Hkv * np;
      ++s_cur;
    }
  }
  flush();
}

// Merge the pieces of one segment (sequence, KV head) for one query head.
// Pieces in order: the shared-prefix pieces (cascade only), then the
// workers' pieces of the segment's own tiles.  One wavefront: lanes first take
// the pieces' (max, sum) pairs (pieces strided over lanes) for the common max M
// and the total L; then lane (group p4 = lane / 16, column chunk c = lane % 16)
// sums pieces p4, p4+4, ... over its D/16 columns, and the four groups are
// added in a fixed order.
template <int CT, int D>
__global__ __launch_bounds__(64) void decode_balanced_merge_kernel(DecodeArgs a) {
  constexpr int VE = D / 16;
  const int seg = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
  const int w0 = a.ws_meta[2 * (int64_t)seg], w1 = a.ws_meta[2 * (int64_t)seg + 1];
  const int ns = a.cascade ? a.num_prefix_splits : 0;
  const int np = ns + (w0 < 0 ? 0 : w1 - w0 + 1);
  if (np == 0) return;  // finalised in place (or an empty context)
  const int G = a.group;
  auto slot_of = [&](int p) -> int64_t {
    return p < ns ? a.prefix_slot0 + (int64_t)seg * ns + p : (int64_t)w0 + seg + (p - ns);
  };
  auto ml = [&](int p) { return a.ws_ml + (slot_of(p) * G + g) * 2; };
  // Lane (p4 = lane / 16, c = lane % 16) sums pieces p4, p4 + 4, ... over
  // columns [VE c, VE c + VE).  Its first two pieces' columns are loaded now,
  // together with the (max, sum) pairs below, so the two latencies overlap.
  const int p4 = lane >> 4, c = lane & 15;
  f32x4 v0[VE / 4], v1[VE / 4];
  {
    const float* src0 = a.ws_acc + (slot_of(min(p4, np - 1)) * G + g) * D + VE * c;
    const float* src1 = a.ws_acc + (slot_of(min(p4 + 4, np - 1)) * G + g) * D + VE * c;
#pragma unroll
    for (int q = 0; q < VE / 4; ++q) {
      v0[q] = p4 < np ? *reinterpret_cast<const f32x4*>(src0 + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
      v1[q] = p4 + 4 < np ? *reinterpret_cast<const f32x4*>(src1 + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }

  float M = kNegInf;
  for (int p = lane; p < np; p += 64) M = fmaxf(M, ml(p)[0]);
  M = wave_max_f32(M);
  float L = 0.f;
  for (int p = lane; p < np; p += 64) L += __builtin_amdgcn_exp2f(ml(p)[0] - M) * ml(p)[1];
  L = wave_sum_f32(L);

  float o[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) o[e] = 0.f;
  auto add = [&](float f, const f32x4* v) {
#pragma unroll
    for (int q = 0; q < VE / 4; ++q) {
      o[4 * q] += f * v[q][0];
      o[4 * q + 1] += f * v[q][1];
      o[4 * q + 2] += f * v[q][2];
      o[4 * q + 3] += f * v[q][3];
    }
  };
  // pieces p4, p4 + 4, ... in order; the first two were loaded up front
  if (p4 < np) add(__builtin_amdgcn_exp2f(ml(p4)[0] - M), v0);
  if (p4 + 4 < np) add(__builtin_amdgcn_exp2f(ml(p4 + 4)[0] - M), v1);
  for (int p = p4 + 8; p < np; p += 4) {
    const float* src = a.ws_acc + (slot_of(p) * G + g) * D + VE * c;
    f32x4 v[VE / 4];
#pragma unroll
    for (int q = 0; q < VE / 4; ++q) v[q] = *reinterpret_cast<const f32x4*>(src + 4 * q);
    add(__builtin_amdgcn_exp2f(ml(p)[0] - M), v);
  }
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    o[e] = sum_over_lane_groups(o[e]);
  }
  if (p4 != 0) return;
  const float inv = a.v_scale / L;
  const int s = seg / a.num_kv_heads, h = seg - s * a.num_kv_heads;
  float x[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) x[e] = o[e] * inv;
  store_run<CT, VE>(a.out, ((int64_t)s * a.num_q_heads + h * G + g) * D + VE * c, x);
}

// Tiles loaded per batch.  More tiles put more bytes in flight per wavefront
// but cost VGPRs (32 per bf16 D=128 tile) and occupancy.
#ifndef PKV_DECODE_RING_FP8
#define PKV_DECODE_RING_FP8 PKV_DECODE_RING
#endif
template <int CT, int D>
constexpr int ring_depth() {
  return CT == PKV_FP8_E4M3 ? PKV_DECODE_RING_FP8 : PKV_DECODE_RING;
}

template <int CT, int D, int NW>
hipError_t launch_nw(const DecodeArgs& a, hipStream_t stream) {
  if (a.phase != kMergePhase && NW == 1 && a.num_workers > 0) {
    // one-wavefront partitions: persistent wavefronts stream runs of them
    constexpr int B = ring_depth<CT, D>();
    const dim3 grid((unsigned)((a.num_workers + 3) / 4));
    if (a.append && a.stream_kv)
      hipLaunchKernelGGL((decode_partition_run_kernel<CT, D, B, true, true>), grid, dim3(256), 0, stream, a);
    else if (a.append)
      hipLaunchKernelGGL((decode_partition_run_kernel<CT, D, B, true, false>), grid, dim3(256), 0, stream, a);
    else if (a.stream_kv)
      hipLaunchKernelGGL((decode_partition_run_kernel<CT, D, B, false, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_partition_run_kernel<CT, D, B, false, false>), grid, dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (a.phase != kMergePhase) {
    const dim3 grid((unsigned)a.num_parts, (unsigned)a.num_kv_heads, (unsigned)a.num_seqs);
    constexpr int B = ring_depth<CT, D>();
    const dim3 block(NW * 64);
    if (a.append && a.stream_kv)
      hipLaunchKernelGGL((decode_partition_kernel<CT, D, NW, B, true, true>), grid, block, 0, stream, a);
    else if (a.append)
      hipLaunchKernelGGL((decode_partition_kernel<CT, D, NW, B, true, false>), grid, block, 0, stream, a);
    else if (a.stream_kv)
      hipLaunchKernelGGL((decode_partition_kernel<CT, D, NW, B, false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_partition_kernel<CT, D, NW, B, false, false>), grid, block, 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.phase == kSplitPhase || a.num_parts == 1) return hipSuccess;
  const dim3 rgrid((unsigned)a.num_q_heads, (unsigned)a.num_seqs);
  hipLaunchKernelGGL((decode_reduce_kernel<CT, D>), rgrid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int CT, int D>
hipError_t launch_balanced(const DecodeArgs& a, hipStream_t stream) {
  if (a.phase != kMergePhase) {
    const dim3 grid((unsigned)((a.num_workers + 3) / 4));
    constexpr int B = ring_depth<CT, D>();
    if (a.append && a.stream_kv)
      hipLaunchKernelGGL((decode_balanced_kernel<CT, D, B, true, true>), grid, dim3(256), 0, stream, a);
    else if (a.append)
      hipLaunchKernelGGL((decode_balanced_kernel<CT, D, B, true, false>), grid, dim3(256), 0, stream, a);
    else if (a.stream_kv)
      hipLaunchKernelGGL((decode_balanced_kernel<CT, D, B, false, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_balanced_kernel<CT, D, B, false, false>), grid, dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.phase == kSplitPhase) return hipSuccess;
  const dim3 mgrid((unsigned)(a.num_seqs * a.num_kv_heads), (unsigned)a.group);
  hipLaunchKernelGGL((decode_balanced_merge_kernel<CT, D>), mgrid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

template <int CT, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t stream) {
  if (a.mode == kBalanced) return launch_balanced<CT, D>(a, stream);
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
