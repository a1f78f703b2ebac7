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
//   wavefront's rows, staged per workgroup through LDS.  bf16 and E4M3 caches
//   become bf16 images there: K row-major with an XOR swizzle of its 16-byte
//   chunks, V transposed into the A operand of V^T.P, so the wavefronts read
//   MFMA operands with plain 16-byte loads and no per-wavefront repacking or
//   conversion.  f32 caches are staged as they are.
// * Softmax per block of four tiles (one max and one lazy rescale per block);
//   the causal mask and the wavefront's range enter as -inf starting values of
//   the score accumulators on the few blocks that need them, and keys past the
//   context are zeroed in the staging.  Tiles are visited in increasing order,
//   so key 0 (visible to every row) comes first and every running max is
//   finite from the first tile on.
// * One workgroup per compute unit takes (sequence, row group, KV head) jobs
//   longest first, in snake order over the rounds (round_item), so the long
//   rows of sequences with long cached prefixes do not start last and short
//   jobs fill in behind them; one ranking in LDS plans several rounds
//   (plan_jobs).
// * Each row's result is finalised in place: no workspace, no second kernel.
// * The same machinery serves the shared-prefix part of a cascade decode
//   (shared_prefix_kernel): all sequences' query heads against one prefix,
//   split over keys, leaving partial states for the decode's merge.
#include "pkv_internal.h"
#include "tile.h"

namespace pkv {
namespace {

constexpr int kPrefillWaves = 8;
constexpr int kPrefillChunkTiles = 1024;  // tile row bases staged in LDS per pass

// A column keeps its running max until a score exceeds it by more than
// kLazyMax (log2 units): its probabilities then stay below 2^kLazyMax and the
// accumulators need no rescale (an unchanged max rescales by exactly 1).
constexpr float kLazyMax = 8.0f;

// Online-softmax state of one 16-row block, per lane: column g = lane % 16.
// Scores enter raw (q.k) and the positive factor qs (scale * log2 e) is
// applied inside the exponent's FMA, so m is in log2 units of scaled scores.
template <int VE>
struct RowState {
  float m;       // running max reference, identical in the 4 lane groups
  f32x4 l;       // running sum of the rounded probabilities (see the updates)
  f32x4 acc[VE];
};

// Max over the four lanes l, l^16, l^32, l^48 (one column's lane groups).
// IEEE maximum: no input canonicalisation, and a NaN score propagates.
__device__ __forceinline__ float column_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float m = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Max of one raw-score column over the lane's keys and the other lane groups,
// scaled into log2 units, and the lazy rescale it may call for.
template <int VE>
__device__ __forceinline__ float raise_max(RowState<VE>& st, float local_max, float qs) {
  const float bm = column_max(local_max) * qs;
  // a column's first tile holds a visible key (tile 0 holds key 0), so its
  // running max is finite from then on; a fully masked tile leaves bm = -inf
  const bool grow = bm > st.m + kLazyMax;
  const float m_new = grow ? bm : st.m;
  if (__ballot(grow) != 0) {  // wave-uniform: some column's max moved
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
#pragma unroll
    for (int r = 0; r < VE; ++r) st.acc[r] *= alpha;
    st.l *= alpha;
  }
  st.m = m_new;
  return m_new;
}

// Keys pass through LDS in stages: kStageKeys at a time for f32 caches, one
// softmax block (kBlockTiles tiles, double-buffered) for the bf16 images.
constexpr int kStageKeys = 128;
constexpr int kStageTiles = kStageKeys / 16;
constexpr int kBlockTiles = 4;

// f32 caches: K and V rows copied as they are, padded by 32 bytes so that the
// lanes reading one 16-byte column of 16 different rows meet the fewest bank
// conflicts (measured against 0, 16, 48, 64 and 96 bytes).
template <int D>
constexpr int f32_pitch() {
  return 4 * D + 32;
}
// bf16 and E4M3 caches: bf16 images of K and V.
// K: rows of 2D bytes, the 16-byte chunk n of key row k stored at chunk
// n ^ k_swizzle(k), so that the 16 rows one MFMA operand read touches (one
// chunk each) fall in distinct banks.
// V: column-chunk major.  Region r (d = 16 r .. 16 r + 15, 32 bytes per key)
// holds the stage's keys in order, key k at byte 32 k of the region, so the
// 16 keys of a tile make 512 contiguous bytes.  The A operand of V^T.P comes
// from gfx950's LDS transpose read: lane l reads the 8 bytes at 8 l of a
// tile's 512 bytes, and within each 16-lane group the hardware hands lane
// 4 b + e element j of the lane 4 j + b read, i.e. lane l receives d = 16 r +
// l % 16 of keys 4 (l / 16) .. 4 (l / 16) + 3, the key order of the scores'
// P.  Two such reads (tiles a and b of a pair) make one 16-byte operand.  This
// replaces a transposing copy through registers (per-element permutes in the
// staging) with a plain 16-byte copy.
template <int D>
__device__ __forceinline__ int k_swizzle(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);  // rows 256 / 128 bytes long
}
constexpr int kVRegion = 16 * kBlockTiles * 32;  // one 32-byte column chunk of a stage's 64 keys

// gfx950 LDS transpose read of four bf16 (see the V layout above).
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
}

// Probabilities of one column from raw scores x (dropped keys at -inf).
template <int VE, int N>
__device__ __forceinline__ void probabilities(RowState<VE>& st, const float (&x)[N], float qs, float (&p)[N]) {
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mx = __builtin_elementwise_maximum(mx, x[i]);
  const float m = raise_max(st, mx, qs);
#pragma unroll
  for (int i = 0; i < N; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], qs, -m));
}

// f32 caches, one tile (keys t0 .. t0+15) for the R row blocks on the
// 16x16x4 f32 MFMA; l[0] holds this lane's share of the column sum.
// MASKED: keys past lim[rb] (the column's position - t0 - 4 * lane group)
// are dropped.
template <int D, int R, bool MASKED>
__device__ __forceinline__ void update_tile_f32(const Tile<PKV_F32, D>& tl,
                                                const typename Tile<PKV_F32, D>::QFrag (&qf)[R],
                                                RowState<D / 16> (&st)[R], const int (&lim)[R], float qs) {
  f32x4 s[R];
#pragma unroll
  for (int rb = 0; rb < R; ++rb) s[rb] = tl.scores(qf[rb]);
  const typename Tile<PKV_F32, D>::PV pv = tl.pack_v();
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    float x[4], p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = !MASKED || i <= lim[rb] ? s[rb][i] : kNegInf;
    probabilities(st[rb], x, qs, p);
    st[rb].l[0] += Tile<PKV_F32, D>::pv_packed(pv, p, st[rb].acc);
  }
}

// bf16 images (bf16 and E4M3 caches): a block of NT tiles (keys t0 ..
// t0 + 16 NT - 1) for the R row blocks, with one max and one rescale per row
// block for the whole block, in two halves: block_probs (scores, max,
// rescale, probabilities) and block_pv (P.V and the row sums).  Scores come from the K image (kt: the block's
// first tile, ko: the lane's chunk offsets); P.V runs per tile pair a, b on the
// double-rate K=32 MFMA, lane group q carrying keys 4q..4q+3 of a, then of b,
// in P and in V^T alike.  V^T is read from the V image one group of 16 d (r)
// and tile pair at a time and feeds every row block.  The column
// sums come from one more MFMA against an all-ones A operand, so every lane's
// l[0] is its column's full sum of the rounded probabilities.
// masked: tiles from `live` on and keys past lim[rb] (the column's position -
// t0 - 4 * lane group) are dropped (score -inf); the staging zeroes V past
// the context, so no stray bits reach the sums.
template <int D, int R, int NT>
__device__ __forceinline__ void block_probs(const char* kt, const int (&ko)[D / 32],
                                            const typename Tile<PKV_BF16, D>::QFrag (&qf)[R],
                                            RowState<D / 16> (&st)[R], bool masked, const int (&lim)[R],
                                            int live, float qs, u32x4 (&pk)[R][NT / 2]) {
  f32x4 sc[R][NT];
#pragma unroll
  for (int rb = 0; rb < R; ++rb)
#pragma unroll
    for (int t = 0; t < NT; ++t) sc[rb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {  // 32 d at a time, every tile and row block
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 k = *reinterpret_cast<const u32x4*>(kt + t * 32 * D + ko[c]);
#pragma unroll
      for (int rb = 0; rb < R; ++rb) sc[rb][t] = mfma_bf16_k32(k, qf[rb].q[c], sc[rb][t]);
    }
  }
  if (masked) {  // wave-uniform and rare: a real branch, not selects on every block
#pragma unroll
    for (int rb = 0; rb < R; ++rb)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!(t < live && 16 * t + i <= lim[rb])) sc[rb][t][i] = kNegInf;
  }
#pragma unroll
  for (int rb = 0; rb < R; ++rb) {
    float x[4 * NT], p[4 * NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * t + i] = sc[rb][t][i];
    probabilities(st[rb], x, qs, p);
#pragma unroll
    for (int h = 0; h < NT / 2; ++h)
      pk[rb][h] = u32x4{pack_bf16(p[8 * h], p[8 * h + 1]), pack_bf16(p[8 * h + 2], p[8 * h + 3]),
                        pack_bf16(p[8 * h + 4], p[8 * h + 5]), pack_bf16(p[8 * h + 6], p[8 * h + 7])};
  }
}

// P.V of one block: V^T from its LDS image (vt: the stage's V image plus 8
// lane bytes) against the probabilities pk, plus the row sums.  acc[r] row m
// is d = 16 r + m.
template <int D, int R, int NT>
__device__ __forceinline__ void block_pv(const char* vt, const u32x4 (&pk)[R][NT / 2],
                                         RowState<D / 16> (&st)[R]) {
  constexpr int VE = D / 16;
  constexpr uint32_t kOnes = 0x3f803f80u;  // two bf16 1.0
#pragma unroll
  for (int h = 0; h < NT / 2; ++h) {
#pragma unroll
    for (int r = 0; r < VE; ++r) {
      const u32x2 va = lds_read_tr16(vt + r * kVRegion + 2 * h * 512);
      const u32x2 vb = lds_read_tr16(vt + r * kVRegion + (2 * h + 1) * 512);
      const u32x4 v = {va[0], va[1], vb[0], vb[1]};
#pragma unroll
      for (int rb = 0; rb < R; ++rb) st[rb].acc[r] = mfma_bf16_k32(v, pk[rb][h], st[rb].acc[r]);
    }
#pragma unroll
    for (int rb = 0; rb < R; ++rb)
      st[rb].l = mfma_bf16_k32(u32x4{kOnes, kOnes, kOnes, kOnes}, pk[rb][h], st[rb].l);
  }
}

// q fragments prepared for a positive factor: a negative scale flips the sign
// bits of q (exact) and a zero scale zeroes q and uses factor 1; scores, max
// and probabilities are then those of the signed scale.
__device__ __forceinline__ void condition_q(u32x4& q, uint32_t sign, bool zero) {
  q = zero ? u32x4{0, 0, 0, 0} : (q ^ sign);
}
__device__ __forceinline__ void condition_q(f32x4& q, uint32_t sign, bool zero) {
  const u32x4 w = __builtin_bit_cast(u32x4, q);
  q = __builtin_bit_cast(f32x4, zero ? u32x4{0, 0, 0, 0} : (w ^ sign));
}

// Exclusive prefix sum of one value per thread over a workgroup of NT
// threads; scratch holds NT / 64 ints.  Every thread calls it.
template <int NT>
__device__ int block_exclusive_scan(int v, int* scratch, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = (int)wave_incl_scan_u32((uint32_t)v);
  if (lane == 63) scratch[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int t = scratch[i];
    base += i < w ? t : 0;
    tot += t;
  }
  __syncthreads();  // scratch free again
  total = tot;
  return base + x - v;
}

// Longest-first order of a chunked-prefill grid.  A job is (sequence s, row
// group rg) and costs its key tile count, which grows with the position of the
// group's last row; workgroups take jobs in decreasing cost (in buckets of
// 2^shift tiles, at most kRankBuckets of them), then by s, then by rg, so the
// long jobs start first and the short ones fill in behind them.  Every
// workgroup computes the same counting sort over the lengths and keeps the
// job of its own rank.
constexpr int kRankBuckets = 2 * kPrefillWaves * 64;

struct PrefillJob {
  int s, rg;        // sequence (-1: none), row group
  int q0, nq, ctx;  // its first query token, query count and context length
  int hk;           // KV head
};

__device__ __forceinline__ int job_cost(int first, int rows, int rg, int rows_g, int G) {
  return (first + (min(rows, (rg + 1) * rows_g) - 1) / G) / 16 + 1;
}

// The ranking for any batch size: thread t owns a contiguous run of sequences
// and reads their lengths from global memory in every pass.  false: no job of
// that rank.  scratch: kRankBuckets + 16 ints of LDS.
__device__ bool ranked_job_by_seq(const PrefillArgs& a, int rows_g, int rank, int* scratch, int& s_out,
                                  int& rg_out) {
  constexpr int NT = kPrefillWaves * 64;
  const int S = a.num_seqs, G = a.group, tid = threadIdx.x;
  int* hist = scratch;
  int* tmp = scratch + kRankBuckets;  // [0, 8): scan, [8, 12): results
  auto cost = [&](int first, int rows, int rg) { return job_cost(first, rows, rg, rows_g, G); };
  // the largest cost (every sequence's last row group) sets the bucket width
  int mx = 0;
  for (int s = tid; s < S; s += NT) {
    const int nq = a.qstart[s + 1] - a.qstart[s];
    if (nq > 0) mx = max(mx, cost(a.lens[s] - nq, nq * G, (nq * G - 1) / rows_g));
  }
  mx = (int)wave_all_reduce((uint32_t)mx, [](uint32_t u, uint32_t v) { return u > v ? u : v; });  // mx >= 0
  if ((tid & 63) == 0) tmp[tid >> 6] = mx;
  for (int i = tid; i < kRankBuckets; i += NT) hist[i] = 0;
  __syncthreads();
  mx = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) mx = max(mx, tmp[i]);
  int shift = 0;
  while ((mx >> shift) >= kRankBuckets) ++shift;
  __syncthreads();  // tmp read before the scans reuse it
  for (int s = tid; s < S; s += NT) {
    const int nq = a.qstart[s + 1] - a.qstart[s], rows = nq * G, first = a.lens[s] - nq;
    for (int rg = 0; rg * rows_g < rows; ++rg) atomicAdd(&hist[cost(first, rows, rg) >> shift], 1);
  }
  __syncthreads();
  // thread t owns buckets kRankBuckets-1-2t and kRankBuckets-2-2t (descending)
  const int b0 = kRankBuckets - 1 - 2 * tid, h0 = hist[b0], h1 = hist[b0 - 1];
  int total;
  const int above = block_exclusive_scan<NT>(h0 + h1, tmp, total);
  if (rank >= total) return false;  // workgroup-uniform
  if (rank >= above && rank < above + h0) {
    tmp[8] = b0;
    tmp[9] = rank - above;
  } else if (rank >= above + h0 && rank < above + h0 + h1) {
    tmp[8] = b0 - 1;
    tmp[9] = rank - above - h0;
  }
  __syncthreads();
  const int bucket = tmp[8], off = tmp[9];
  // the off-th job of that bucket in (s, rg) order: sequences in contiguous
  // runs per thread
  const int per = (S + NT - 1) / NT, s_lo = min(S, tid * per), s_hi = min(S, s_lo + per);
  int cnt = 0;
  for (int s = s_lo; s < s_hi; ++s) {
    const int nq = a.qstart[s + 1] - a.qstart[s], rows = nq * G, first = a.lens[s] - nq;
    for (int rg = 0; rg * rows_g < rows; ++rg) cnt += (cost(first, rows, rg) >> shift) == bucket;
  }
  int total2;
  const int before = block_exclusive_scan<NT>(cnt, tmp, total2);
  if (off >= before && off < before + cnt) {
    int k = off - before;
    for (int s = s_lo; s < s_hi && k >= 0; ++s) {
      const int nq = a.qstart[s + 1] - a.qstart[s], rows = nq * G, first = a.lens[s] - nq;
      for (int rg = 0; rg * rows_g < rows && k >= 0; ++rg) {
        if ((cost(first, rows, rg) >> shift) != bucket) continue;
        if (k == 0) {
          tmp[10] = s;
          tmp[11] = rg;
        }
        --k;
      }
    }
  }
  __syncthreads();
  s_out = tmp[10];
  rg_out = tmp[11];
  return true;
}

// Item i of the prefill grid: the job of rank i / Hkv on KV head i % Hkv.  Of
// W workgroups, workgroup w takes item it * W + w in even rounds it and
// (it + 1) * W - 1 - w in odd ones (snake order), so the one that drew the
// shortest job of a round draws the longest of the next.  Items only grow
// from round to round.
__device__ __forceinline__ int64_t round_item(int it) {
  const int64_t W = gridDim.x;
  return (it & 1) ? (int64_t)(it + 1) * W - 1 - blockIdx.x : (int64_t)it * W + blockIdx.x;
}

// Rounds ranked together: one ranking serves this many of a workgroup's jobs.
constexpr int kPlanRounds = 4;

// This workgroup's jobs of rounds it0 .. it0 + kPlanRounds - 1 into jobs[]
// (LDS; s = -1: no job), for batches whose sequence table fits the scratch.
// The sequences' lengths are read from global memory once, into LDS with each
// sequence's first job index; the passes split the flat job list evenly over
// the threads (a batch of a few long chunks has many row groups per sequence;
// one thread per sequence would walk them alone).  Up to one job per thread,
// every job's rank is counted directly against the others' buckets; beyond
// that the counting sort finds each round's rank.  Same order as
// ranked_job_by_seq.  scratch: kRankBuckets + 16 + 4 * num_seqs + 1 + NT
// ints of LDS.
template <int NT>
__device__ void plan_staged(const PrefillArgs& a, int rows_g, int it0, int* scratch, PrefillJob* jobs) {
  const int S = a.num_seqs, G = a.group, Hkv = a.num_kv_heads, tid = threadIdx.x;
  int* hist = scratch;
  int* tmp = scratch + kRankBuckets;  // [0, 8): scans, [8, 16): maxima, then results
  int* seq = tmp + 16;                // q0, nq, ctx of sequence s at 3 s
  int* joff = seq + 3 * S;            // first job index of sequence s; joff[S]: job count
  int* ord = joff + S + 1;            // job index of each rank (one job per thread)
  for (int i = tid; i < kRankBuckets; i += NT) hist[i] = 0;
  // pass 1: per-sequence data, job counts and the largest cost
  const int ps = (S + NT - 1) / NT, s_lo = min(S, tid * ps), s_hi = min(S, s_lo + ps);
  int njobs = 0, mx = 0;
  for (int s = s_lo; s < s_hi; ++s) {
    const int q0 = a.qstart[s], nq = a.qstart[s + 1] - q0, ctx = a.lens[s];
    seq[3 * s] = q0;
    seq[3 * s + 1] = nq;
    seq[3 * s + 2] = ctx;
    const int rows = nq * G, n = (rows + rows_g - 1) / rows_g;
    if (n > 0) mx = max(mx, job_cost(ctx - nq, rows, n - 1, rows_g, G));
    njobs += n;
  }
  mx = (int)wave_all_reduce((uint32_t)mx, [](uint32_t u, uint32_t v) { return u > v ? u : v; });  // mx >= 0
  if ((tid & 63) == 0) tmp[8 + (tid >> 6)] = mx;
  int J;
  int j = block_exclusive_scan<NT>(njobs, tmp, J);  // its syncs publish seq and the maxima
  for (int s = s_lo; s < s_hi; ++s) {
    joff[s] = j;
    j += (seq[3 * s + 1] * G + rows_g - 1) / rows_g;
  }
  if (tid == 0) joff[S] = J;
  mx = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) mx = max(mx, tmp[8 + i]);
  int shift = 0;
  while ((mx >> shift) >= kRankBuckets) ++shift;
  __syncthreads();
  // the last s with joff[s] <= j (j < J)
  auto seq_of = [&](int jj) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (joff[mid] <= jj) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  auto put = [&](int k, int s, int rg, int hk) {
    jobs[k] = PrefillJob{s, rg, seq[3 * s], seq[3 * s + 1], seq[3 * s + 2], hk};
  };
  // rank of round it0 + k (-1: none)
  auto round_rank = [&](int k) {
    const int64_t r = round_item(it0 + k) / Hkv;
    return r < J ? (int)r : -1;
  };

  if (J <= NT) {
    // one job per thread: its rank is the number of jobs of a larger bucket,
    // or of the same bucket and a smaller index
    int b = 0;
    if (tid < J) {
      const int s = seq_of(tid);
      b = job_cost(seq[3 * s + 2] - seq[3 * s + 1], seq[3 * s + 1] * G, tid - joff[s], rows_g, G) >> shift;
    }
    hist[tid] = tid < J ? b : -1;  // -1: no job, below every bucket
    __syncthreads();
    if (tid < J) {
      int r = 0;
      for (int j0 = 0; j0 < J; j0 += 16) {  // 16 buckets a step, 4 reads in flight
        int4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const int4*>(hist + j0 + 4 * u);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int jj = j0 + 4 * u;
          r += (v[u].x > b || (v[u].x == b && jj < tid)) + (v[u].y > b || (v[u].y == b && jj + 1 < tid)) +
               (v[u].z > b || (v[u].z == b && jj + 2 < tid)) + (v[u].w > b || (v[u].w == b && jj + 3 < tid));
        }
      }
      ord[r] = tid;
    }
    __syncthreads();
    if (tid < kPlanRounds) {
      const int r = round_rank(tid);
      if (r < 0) {
        jobs[tid].s = -1;
      } else {
        const int jj = ord[r], s = seq_of(jj);
        put(tid, s, jj - joff[s], (int)(round_item(it0 + tid) % Hkv));
      }
    }
    __syncthreads();
    return;
  }

  // this thread's jobs [j_lo, j_hi) and the sequence holding j_lo
  const int pj = (J + NT - 1) / NT, j_lo = min(J, tid * pj), j_hi = min(J, j_lo + pj);
  const int s0 = j_lo < j_hi ? seq_of(j_lo) : 0;
  // fn(s, rg, bucket) over this thread's jobs in order; stops when fn is false
  auto walk = [&](auto&& fn) {
    int s = s0, first = 0, rows = 0, end = 0, rg = 0;
    for (int jj = j_lo; jj < j_hi; ++jj, ++rg) {
      if (jj == j_lo || jj == end) {
        while (joff[s + 1] <= jj) ++s;
        rg = jj - joff[s];
        end = joff[s + 1];
        rows = seq[3 * s + 1] * G;
        first = seq[3 * s + 2] - seq[3 * s + 1];
      }
      if (!fn(s, rg, job_cost(first, rows, rg, rows_g, G) >> shift)) return;
    }
  };
  walk([&](int, int, int bk) {
    atomicAdd(&hist[bk], 1);
    return true;
  });
  __syncthreads();
  // thread t owns buckets kRankBuckets-1-2t and kRankBuckets-2-2t (descending)
  const int b0 = kRankBuckets - 1 - 2 * tid, h0 = hist[b0], h1 = hist[b0 - 1];
  int total;
  const int above = block_exclusive_scan<NT>(h0 + h1, tmp, total);
  for (int k = 0; k < kPlanRounds; ++k) {
    const int rank = round_rank(k);  // workgroup-uniform
    if (rank < 0) {
      if (tid == 0) jobs[k].s = -1;
      continue;
    }
    if (rank >= above && rank < above + h0) {
      tmp[8] = b0;
      tmp[9] = rank - above;
    } else if (rank >= above + h0 && rank < above + h0 + h1) {
      tmp[8] = b0 - 1;
      tmp[9] = rank - above - h0;
    }
    __syncthreads();
    const int bucket = tmp[8], off = tmp[9];
    // the off-th job of that bucket in (s, rg) order
    int cnt = 0;
    walk([&](int, int, int bk) {
      cnt += bk == bucket;
      return true;
    });
    int total2;
    const int before = block_exclusive_scan<NT>(cnt, tmp, total2);  // its first sync: tmp[8, 10) read
    if (off >= before && off < before + cnt) {
      int left = off - before;
      const int hk = (int)(round_item(it0 + k) % Hkv);
      walk([&](int s, int rg, int bk) {
        if (bk != bucket) return true;
        if (left-- > 0) return true;
        put(k, s, rg, hk);
        return false;
      });
    }
  }
  __syncthreads();
}

// This workgroup's jobs from round it0 on into jobs[] (LDS; s = -1: no job);
// returns how many rounds were planned.  scratch_ints: LDS ints available at
// scratch (at least kRankBuckets + 16).
__device__ int plan_jobs(const PrefillArgs& a, int rows_g, int it0, int* scratch, int scratch_ints,
                         PrefillJob* jobs) {
  constexpr int NT = kPrefillWaves * 64;
  if ((int64_t)kRankBuckets + 17 + 4 * (int64_t)a.num_seqs + NT <= scratch_ints) {
    plan_staged<NT>(a, rows_g, it0, scratch, jobs);
    return kPlanRounds;
  }
  const int64_t item = round_item(it0), rank = item / a.num_kv_heads;
  int s = -1, rg = 0;
  if (rank > 0x7fffffff || !ranked_job_by_seq(a, rows_g, (int)rank, scratch, s, rg)) s = -1;
  if (threadIdx.x == 0) {
    if (s < 0) {
      jobs[0].s = -1;
    } else {
      const int q0 = a.qstart[s];
      jobs[0] = PrefillJob{s, rg, q0, a.qstart[s + 1] - q0, a.lens[s], (int)(item % a.num_kv_heads)};
    }
  }
  __syncthreads();
  return 1;
}

enum RowsJob : int { kPrefillJob = 0, kPrefixJob = 1 };

// Query rows against paged keys on the matrix cores, K/V streamed through LDS.
//   kPrefillJob: rows = a chunk's (query token, head) pairs of one KV head,
//     causal, final outputs (PrefillArgs).
//   kPrefixJob: rows = every sequence's query heads of one KV head against one
//     key split of a shared prefix, no mask, partial states (PrefixArgs).
// Per stage the workgroup's threads copy the stage's K and V from the pool
// into LDS, then every wavefront reads its MFMA fragments from there.  The
// next stage's global loads are issued before the current stage is computed,
// so they are in flight meanwhile.
template <int CT, int D, int R, int JOB, typename Args>
__global__ __launch_bounds__(kPrefillWaves * 64, 8 / kPrefillWaves) void rows_kernel(Args a) {
  constexpr bool F32 = CT == PKV_F32;
  using T = Tile<F32 ? PKV_F32 : PKV_BF16, D>;  // fragments read from LDS
  constexpr int VE = D / 16;
  constexpr int NW = kPrefillWaves;
  constexpr int ROWS_W = 16 * R;
  constexpr int ROWS_G = ROWS_W * NW;
  constexpr int EB = CT == PKV_F32 ? 4 : CT == PKV_BF16 ? 2 : 1;  // cache bytes per element
  constexpr int RB = D * EB;                                     // cache bytes per key row
  constexpr int PER_ROW = RB / 16;                               // 16-byte pieces per key row
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.group, Hq = a.num_q_heads, bs = a.block_size, Hkv = a.num_kv_heads;
  const int64_t block_rows = (int64_t)Hkv * bs;
  // the factor applied to raw scores, made positive (condition_q)
  const float qs_in = a.qk_scale;
  const bool q_zero = qs_in == 0.f;
  const uint32_t q_sign = qs_in < 0.f ? (F32 ? 0x80000000u : 0x80008000u) : 0u;
  const float qs = q_zero ? 1.f : fabsf(qs_in);

  __shared__ int64_t sm_row[kPrefillChunkTiles];  // pool row of each tile's first key
  // bf16 images: stage buffers for K (two: one read, the next written) and V
  // (three: the lagging half of the wavefronts still reads the previous one)
  constexpr int K_STAGE = 16 * kBlockTiles * 2 * D, V_STAGE = 16 * kBlockTiles * 2 * D;
  constexpr int K_BYTES = F32 ? kStageKeys * f32_pitch<D>() : 2 * K_STAGE;
  constexpr int V_BYTES = F32 ? kStageKeys * f32_pitch<D>() : 3 * V_STAGE;
  __shared__ __attribute__((aligned(16))) char sm_k[K_BYTES];
  __shared__ __attribute__((aligned(16))) char sm_v[V_BYTES];
  static_assert(K_BYTES >= 4 * (kRankBuckets + 16), "ranking scratch");

  // Jobs: prefill: items in round_item's order, ranked kPlanRounds rounds at
  // a time into sm_jobs; prefix: x = KV head, y = key split, z = row group,
  // from the last row group down.
  __shared__ PrefillJob sm_jobs[kPlanRounds];
  int plan0 = 0, planned = 0;  // sm_jobs holds rounds plan0 .. plan0 + planned - 1
  int hk = JOB == kPrefillJob ? 0 : (int)blockIdx.x;
  int64_t head_rows = (int64_t)hk * bs;
  int rows = 0, ctx = 0, first_pos = 0, q0 = 0, k_lo = 0, k_hi_all = 0;
  const int32_t* table = nullptr;
  if constexpr (JOB == kPrefixJob) {
    const int split = blockIdx.y;
    const int ntiles = a.prefix_len / 16;
    rows = a.num_seqs * G;
    ctx = a.prefix_len;
    table = a.blocks;
    k_lo = (int)((int64_t)split * ntiles / a.splits);
    k_hi_all = (int)((int64_t)(split + 1) * ntiles / a.splits);
  }

  for (int it = 0;; ++it) {
    int rg;
    if constexpr (JOB == kPrefillJob) {
      if (it == plan0 + planned) {
        __syncthreads();  // the ranking scratch aliases the K stage
        plan0 = it;
        planned = plan_jobs(a, ROWS_G, it, reinterpret_cast<int*>(sm_k), K_BYTES / 4, sm_jobs);
      }
      const PrefillJob job = sm_jobs[it - plan0];
      if (job.s < 0) break;  // workgroup-uniform; items only grow from round to round
      hk = job.hk;
      head_rows = (int64_t)hk * bs;
      rg = job.rg;
      q0 = job.q0;
      rows = job.nq * G;
      ctx = job.ctx;
      first_pos = ctx - job.nq;
      table = a.tables + (int64_t)job.s * a.max_blocks;
    } else {
      rg = (int)(gridDim.z - 1 - blockIdx.z) + it * (int)gridDim.z;
      if (rg * ROWS_G >= rows) break;
    }
    const int row_g0 = rg * ROWS_G;
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
    int pos4[R];  // the column's position minus 4 * lane group
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
      const int rr = row_w0 + 16 * rb + (lane & 15);
      const bool valid = rr < rows;
      const int t = valid ? rr / G : 0;  // query token (prefill) or sequence (prefix)
      const int g = valid ? rr - t * G : 0;
      qf[rb] = T::load_q(static_cast<const QElem<CT>*>(a.q) + ((int64_t)(q0 + t) * Hq + hk * G + g) * D,
                         valid, lane);
#pragma unroll
      for (int c = 0; c < (int)(sizeof(qf[rb].q) / sizeof(qf[rb].q[0])); ++c)
        condition_q(qf[rb].q[c], q_sign, q_zero);
      // the prefix job's rows and padding columns see every key
      pos4[rb] = (JOB == kPrefillJob && valid ? first_pos + t : ctx - 1) - 4 * (lane >> 4);
    }
    RowState<VE> st[R];
#pragma unroll
    for (int rb = 0; rb < R; ++rb) {
      st[rb].m = kNegInf;
      st[rb].l = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < VE; ++r) st[rb].acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int c0 = k_lo; c0 < k_hi; c0 += kPrefillChunkTiles) {
      const int c1 = min(k_hi, c0 + kPrefillChunkTiles);
      __syncthreads();  // the previous pass is done with the ids and the stage
      for (int i = threadIdx.x; i < c1 - c0; i += NW * 64) {
        const int key0 = (c0 + i) * 16;
        sm_row[i] = (int64_t)table[key0 / bs] * block_rows + head_rows + key0 % bs;
      }
      __syncthreads();

      if constexpr (F32) {
        // piece p of a pool is key p / PER_ROW, 16-byte column p % PER_ROW
        constexpr int PITCH = f32_pitch<D>();
        constexpr int TOTAL = kStageKeys * PER_ROW;
        constexpr int PIECES = (TOTAL + NW * 64 - 1) / (NW * 64);
        static_assert(TOTAL % (NW * 64) == 0 || TOTAL < NW * 64, "stage split");
        u32x4 rk[PIECES], rv[PIECES];
        auto fetch = [&](int tile0) {
#pragma unroll
          for (int i = 0; i < PIECES; ++i) {
            const int p = threadIdx.x + i * NW * 64;
            if (TOTAL < NW * 64 && p >= TOTAL) break;  // fewer pieces than threads
            const int key = p / PER_ROW, col = p - key * PER_ROW;
            const int t = min(tile0 + key / 16, c1 - 1);  // past the end: a valid tile, unused
            const int64_t row =
                sm_row[t - c0] + (key & 15);
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
#pragma unroll
          for (int j = 0; j < kStageTiles; ++j) {
            const int tile = t0s + j;
            if (tile >= k_hi_w) break;  // wave-uniform
            const int t0 = tile * 16;
            T tl;
            tl.load_pitched(sm_k + j * 16 * PITCH, sm_v + j * 16 * PITCH, PITCH, lane);
            if (t0 + 16 > ctx) {  // V rows past the context may hold any bits
              bool ok[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) ok[i] = t0 + 4 * (lane >> 4) + i < ctx;
              tl.mask_rows(ok);
            }
            int lim[R];
#pragma unroll
            for (int rb = 0; rb < R; ++rb) lim[rb] = pos4[rb] - t0;
            if (JOB == kPrefillJob && t0 + 15 > minpos_w)  // causal tile, wave-uniform
              update_tile_f32<D, R, true>(tl, qf, st, lim, qs);
            else
              update_tile_f32<D, R, false>(tl, qf, st, lim, qs);
          }
        }
      } else {
        // Stages of one softmax block (kBlockTiles tiles).  Every thread
        // copies up to KP 16-byte K pieces and VP V pieces of the stage.  K
        // piece p: key p / PER_ROW, column p % PER_ROW.  V piece p (bf16): key
        // (p / 2) % SK, 16-byte half p % 2 of column chunk p / (2 SK), which
        // lands at byte 16 p of the V image; V piece p (E4M3, 16 codes = one
        // column chunk): key p % SK, chunk p / SK, at byte 32 p.  A wavefront's
        // writes then cover contiguous LDS bytes.
        constexpr int NT = kBlockTiles;
        constexpr int SK = 16 * NT;           // keys per stage
        constexpr int NTH = NW * 64;
        constexpr int KTOTAL = SK * PER_ROW;  // 16-byte cache pieces per stage, K and V alike
        constexpr int KP = (KTOTAL + NTH - 1) / NTH;
        static_assert(KP <= 2 && (KTOTAL % NTH == 0 || KTOTAL < NTH), "staging split");
        u32x4 pre_k[KP], pre_v[KP];
        auto fetch = [&](int tile0) {
#pragma unroll
          for (int i = 0; i < KP; ++i) {
            const int p = threadIdx.x + NTH * i;
            if (KTOTAL < NTH && p >= KTOTAL) break;  // fewer pieces than threads
            const int key = p / PER_ROW, kcol = p - key * PER_ROW;
            const int tk = min(tile0 + key / 16, c1 - 1);  // past the end: a valid tile, zeroed
            pre_k[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.kc) +
                                                       (sm_row[tk - c0] + (key & 15)) * RB + kcol * 16);
            const int vkey = EB == 2 ? (p >> 1) & (SK - 1) : p & (SK - 1);
            const int vcol = EB == 2 ? 2 * (p / (2 * SK)) + (p & 1) : p / SK;
            const int tv = min(tile0 + vkey / 16, c1 - 1);
            pre_v[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.vc) +
                                                       (sm_row[tv - c0] + (vkey & 15)) * RB + vcol * 16);
          }
        };
        // lane's K chunk offsets within a tile: row lane % 16, d = 32 c + 8 (lane / 16) + 0..7
        int ko[D / 32];
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
          ko[c] = (lane & 15) * 2 * D + (((lane >> 4) + 4 * c) ^ k_swizzle<D>(lane & 15)) * 16;
        // the fetched stage (tiles t0s .. t0s + NT - 1) into the buffers kd0 / vd0
        auto stage_write = [&](int t0s, char* kd0, char* vd0) {
          // keys past the context or the range: zero (finite K, so that a
          // score accumulator started at -inf stays -inf; V as its
          // probabilities, so that no stray bits reach the sums)
          if (t0s * 16 + SK > ctx || t0s + NT > c1) {  // workgroup-uniform
#pragma unroll
            for (int i = 0; i < KP; ++i) {
              const int p = threadIdx.x + NTH * i;
              if (KTOTAL < NTH && p >= KTOTAL) break;
              const int key = p / PER_ROW, tk = t0s + key / 16;
              if (tk >= c1 || tk * 16 + (key & 15) >= ctx) pre_k[i] = u32x4{0, 0, 0, 0};
              const int vkey = EB == 2 ? (p >> 1) & (SK - 1) : p & (SK - 1), tv = t0s + vkey / 16;
              if (tv >= c1 || tv * 16 + (vkey & 15) >= ctx) pre_v[i] = u32x4{0, 0, 0, 0};
            }
          }
#pragma unroll
          for (int i = 0; i < KP; ++i) {
            const int p = threadIdx.x + NTH * i;
            if (KTOTAL < NTH && p >= KTOTAL) break;
            const int key = p / PER_ROW, kcol = p - key * PER_ROW;
            char* kd = kd0 + key * 2 * D;
            const int sw = k_swizzle<D>(key);
            if constexpr (CT == PKV_BF16) {
              *reinterpret_cast<u32x4*>(kd + ((kcol ^ sw) * 16)) = pre_k[i];
              *reinterpret_cast<u32x4*>(vd0 + 16 * p) = pre_v[i];
            } else {  // E4M3 codes -> bf16 (exact): K chunks 2 kcol, 2 kcol + 1; V one column chunk
              uint32_t b[8], c[8];  // bf16 pairs of elements 2n, 2n+1
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                b[2 * w] = bf16x2_from_fp8x2_lo(pre_k[i][w]);
                b[2 * w + 1] = bf16x2_from_fp8x2_hi(pre_k[i][w]);
                c[2 * w] = bf16x2_from_fp8x2_lo(pre_v[i][w]);
                c[2 * w + 1] = bf16x2_from_fp8x2_hi(pre_v[i][w]);
              }
              *reinterpret_cast<u32x4*>(kd + (((2 * kcol) ^ sw) * 16)) = u32x4{b[0], b[1], b[2], b[3]};
              *reinterpret_cast<u32x4*>(kd + (((2 * kcol + 1) ^ sw) * 16)) = u32x4{b[4], b[5], b[6], b[7]};
              *reinterpret_cast<u32x4*>(vd0 + 32 * p) = u32x4{c[0], c[1], c[2], c[3]};
              *reinterpret_cast<u32x4*>(vd0 + 32 * p + 16) = u32x4{c[4], c[5], c[6], c[7]};
            }
          }
        };
        // Stage n's K sits in K buffer n % 2 and its V in V buffer n % 3; the
        // write of stage n + 1 and the loads of stage n + 2 overlap the compute
        // of stage n, one barrier per stage.  The second half of the
        // wavefronts runs each block's P.V one stage late (ping-pong): while
        // the first half issues a block's score MFMAs, the second half issues
        // the previous block's P.V MFMAs, and each half's softmax VALU work then
        // meets the other half's MFMAs instead of its own partner's softmax.
        const bool lagging = wave >= NW / 2;
        const int voff = 8 * lane;
        u32x4 pk[R][NT / 2];  // a block's probabilities (lagging waves: until the next stage)
        int late_buf = -1;    // lagging waves: the V buffer pk goes with (-1: none)
        fetch(c0);
        stage_write(c0, sm_k, sm_v);
        if (c0 + NT < c1) fetch(c0 + NT);
        __syncthreads();
        for (int t0s = c0, n = 0; t0s < c1; t0s += NT, ++n) {
          const int kb = n & 1, vb = n % 3;
          if (t0s + NT < c1) {
            stage_write(t0s + NT, sm_k + (kb ^ 1) * K_STAGE, sm_v + ((n + 1) % 3) * V_STAGE);
            if (t0s + 2 * NT < c1) fetch(t0s + 2 * NT);  // in flight during the compute
          }
          if (lagging && late_buf >= 0) {  // wave-uniform
            block_pv<D, R, NT>(sm_v + late_buf * V_STAGE + voff, pk, st);
            late_buf = -1;
          }
          if (t0s < k_hi_w) {  // wave-uniform
            const int t0 = t0s * 16;
            int lim[R];
#pragma unroll
            for (int rb = 0; rb < R; ++rb) lim[rb] = pos4[rb] - t0;
            // a block reaching past the first row's position, or with tiles
            // past the wavefront's range, is masked
            const int live_tiles = k_hi_w - t0s;
            const bool masked = (JOB == kPrefillJob && t0 + SK - 1 > minpos_w) || live_tiles < NT;
            block_probs<D, R, NT>(sm_k + kb * K_STAGE, ko, qf, st, masked, lim, live_tiles, qs, pk);
            if (lagging)
              late_buf = vb;
            else
              block_pv<D, R, NT>(sm_v + vb * V_STAGE + voff, pk, st);
          }
          __syncthreads();  // stage n read and stage n + 1 written by every wave
        }
        if (late_buf >= 0) block_pv<D, R, NT>(sm_v + late_buf * V_STAGE + voff, pk, st);
      }
    }

    if (live) {
#pragma unroll
      for (int rb = 0; rb < R; ++rb) {
        float l_run = st[rb].l[0];
        if constexpr (F32) {  // lane shares -> column sum
          l_run = sum_over_lane_groups(l_run);
        }
        const int rr = row_w0 + 16 * rb + (lane & 15);
        if (rr >= rows) continue;
        const int t = rr / G, g = rr - t * G;
        // the lane's outputs: d = VE m + r (f32 fragments) or d = 16 r + m
        // (bf16 images), m = 4 (lane / 16) + i
        if constexpr (JOB == kPrefillJob) {
          const int64_t orow = (int64_t)(q0 + t) * Hq + hk * G + g;
          const float inv = a.v_scale / l_run;
          if constexpr (F32) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float x[VE];
#pragma unroll
              for (int r = 0; r < VE; ++r) x[r] = st[rb].acc[r][i] * inv;
              store_run<CT, VE>(a.out, orow * D + VE * (4 * (lane >> 4) + i), x);
            }
          } else {
#pragma unroll
            for (int r = 0; r < VE; ++r) {
              const float x[4] = {st[rb].acc[r][0] * inv, st[rb].acc[r][1] * inv, st[rb].acc[r][2] * inv,
                                  st[rb].acc[r][3] * inv};
              store_run<CT, 4>(a.out, orow * D + 16 * r + 4 * (lane >> 4), x);
            }
          }
        } else {
          const int64_t slot = a.slot0 + ((int64_t)t * a.num_kv_heads + hk) * a.splits + blockIdx.y;
          float* o = a.ws_acc + (slot * G + g) * D;
          if constexpr (F32) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int q4 = 0; q4 < VE / 4; ++q4)
                *reinterpret_cast<f32x4*>(o + VE * (4 * (lane >> 4) + i) + 4 * q4) =
                    f32x4{st[rb].acc[4 * q4][i], st[rb].acc[4 * q4 + 1][i], st[rb].acc[4 * q4 + 2][i],
                          st[rb].acc[4 * q4 + 3][i]};
          } else {
#pragma unroll
            for (int r = 0; r < VE; ++r)
              *reinterpret_cast<f32x4*>(o + 16 * r + 4 * (lane >> 4)) = st[rb].acc[r];
          }
          if (lane < 16) *reinterpret_cast<f32x2*>(a.ws_ml + (slot * G + g) * 2) = f32x2{st[rb].m, l_run};
        }
      }
    }
  }
}

template <int CT, int D>
hipError_t launch_prefix_d(const PrefixArgs& a, hipStream_t stream) {
  // 16 rows per wavefront (128 per workgroup): each workgroup sees only its
  // key split, so more, smaller workgroups beat fuller ones (measured on the
  // 256-sequence batch: 110.5 us per call against 115.3 us with 32 rows)
  constexpr int ROWS_G = 16 * kPrefillWaves;
  int64_t gz = ((int64_t)a.num_seqs * a.group + ROWS_G - 1) / ROWS_G;
  gz = gz < 1 ? 1 : gz > 65535 ? 65535 : gz;
  const dim3 grid((unsigned)a.num_kv_heads, (unsigned)a.splits, (unsigned)gz);
  hipLaunchKernelGGL((rows_kernel<CT, D, 1, kPrefixJob, PrefixArgs>), grid, dim3(kPrefillWaves * 64), 0,
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
  // one workgroup per compute unit, fewer if max_query_len-long chunks have
  // fewer items; every workgroup keeps taking items while jobs remain
  const int64_t per_seq = ((int64_t)a.max_query_len * a.group + ROWS_G - 1) / ROWS_G;
  const int64_t items = (int64_t)a.num_seqs * (per_seq < 1 ? 1 : per_seq) * a.num_kv_heads;
  const int64_t cap = a.workgroups > 0 ? a.workgroups : 256;
  const dim3 grid((unsigned)(items < cap ? items : cap));
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
