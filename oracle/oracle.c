/*
 * oracle.c -- plain, slow, fp64 CPU oracle for the paged KV cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP kernels behind include/pagedkv.h) never links, calls or includes
 * anything from here, and nothing here is shared with it.
 *
 * What is computed, and where the pages define it:
 *
 *  - The KV-cache write (orc_paged_kv_write).  "PagedAttention, clearly
 *    explained" (x thread, DexRobotics): a block holds the keys and values of a
 *    fixed number of consecutive tokens, a logical block is only an index into
 *    the sequence, and each one is paired with a physical block recorded in the
 *    block table.  A token's slot therefore names (physical block, offset
 *    inside it); the write stores the token's K and V for every KV head there
 *    and touches nothing else.  Layout reading: one layer's cache is
 *    [num_blocks][num_kv_heads][block_size][head_dim].
 *
 *  - Decode attention (orc_paged_attention_decode).  Same thread: at each
 *    decode step the kernel reads the block table and gathers keys and values
 *    from whichever physical blocks they landed in.  "pipe-paged-block-
 *    allocation-kv-cache" (foundry), sections "In and out" and "Concept":
 *    attention needs its keys and values logically ordered, not physically
 *    adjacent, and the kernel computes a weighted sum over positions.  The
 *    oracle walks the block table, rebuilds contiguous K/V in fp64 and computes
 *    softmax(scale * q.K^T) . V for each query head, with query head h reading
 *    KV head h / (Hq / Hkv).
 *
 *  - The 1-byte cache element ("PagedAttention Memory Management", apxml,
 *    section "Calculating Physical Block Sizes": P_bytes is 1 for FP8).  The
 *    format is OCP 8-bit floating point E4M3 ("FN"): 1 sign bit, 4 exponent
 *    bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN,
 *    largest finite 448, smallest subnormal 2^-9.  Encoding rounds to nearest,
 *    ties to even, and saturates finite overflow and infinities to +-448.
 *
 *  - Block copies (orc_copy_blocks: copy-on-write) and moves to and from a
 *    staging buffer (orc_move_blocks: swap-out / swap-in); see each function.
 *
 *  - Chunked-prefill attention (orc_paged_attention_prefill).  "What problem
 *    does PagedAttention solve for the KV cache in vLLM?" (katajob), section
 *    "Sharing, the second dividend": blocks that already hold a prompt
 *    prefix's K/V are reused and that part of prefill is skipped, so the
 *    remaining prompt tokens attend over the cached prefix through the block
 *    table; foundry, section "Effect": the boundary between reused and freshly
 *    prefilled blocks only changes how the reduction is tiled.  Each new query
 *    token sits at the end of its sequence's context (the chunk's own K/V are
 *    written first) and attends, causally, to every position up to its own:
 *    the same softmax(scale * q.K^T) . V as decode, over a shorter prefix.
 *
 * Everything is plain loops in double precision; no blocking, fusion or
 * reordering.  OpenMP only splits independent (sequence, KV head) pairs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_E4M3 = 2 };

enum {
  ORC_OK = 0,
  ORC_ERR_ARG = 1,      /* bad dtype combination or size */
  ORC_ERR_RANGE = 2,    /* slot or block id outside the pool */
  ORC_ERR_NOMEM = 3
};

/* ---------------------------------------------------------------- scalars */

static float f32_from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* bfloat16 is the upper half of an IEEE binary32. */
static double bf16_to_f64(uint16_t b) { return (double)f32_from_bits((uint32_t)b << 16); }

/* E4M3 (OCP "FN") code -> value, straight from the field definition. */
double orc_e4m3_decode(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, 1 - 7); /* subnormal: 0.m * 2^(1-bias) */
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7); /* normal: 1.m * 2^(e-bias) */
  return sign ? -mag : mag;
}

/* Value -> E4M3 code: round to nearest, ties to even, saturate to +-448.
 * A NaN input gives the code 0x7F whatever its sign bit. */
uint8_t orc_e4m3_encode(float y) {
  uint8_t sign;
  double a, q;
  int e2, E;
  if (isnan(y)) return 0x7F;
  sign = signbit(y) ? 0x80 : 0x00;
  a = fabs((double)y);
  if (a >= 448.0) return (uint8_t)(sign | 0x7E);
  if (a < ldexp(1.0, -6)) {
    /* below the smallest normal the grid is the multiples of 2^-9 */
    q = nearbyint(a * 512.0); /* 0..8; 8 is the smallest normal, code 0x08 */
    return (uint8_t)(sign | (uint8_t)q);
  }
  (void)frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
  E = e2 - 1;          /* a = 1.xxx * 2^E, E in [-6, 8] */
  q = nearbyint(ldexp(a, -E) * 8.0); /* 8..16 eighths of the leading power */
  if (q == 16.0) {
    q = 8.0;
    E += 1;
  }
  if (E > 8) return (uint8_t)(sign | 0x7E);
  return (uint8_t)(sign | (uint8_t)(((E + 7) << 3) | ((int)q - 8)));
}

void orc_e4m3_decode_n(const uint8_t* codes, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(codes[i]);
}

void orc_e4m3_encode_n(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(y[i]);
}

/* One stored element as fp64.  For the 1-byte cache the per-tensor scale is
 * applied here; the fp64 product is exact (the code's value has at most 4
 * significant bits, the f32 scale 24). */
static double load_elem(const void* base, int64_t idx, int dtype, double scale) {
  switch (dtype) {
    case ORC_F32: return (double)((const float*)base)[idx];
    case ORC_BF16: return bf16_to_f64(((const uint16_t*)base)[idx]);
    default: return orc_e4m3_decode(((const uint8_t*)base)[idx]) * scale;
  }
}

static float load_f32(const void* base, int64_t idx, int dtype) {
  if (dtype == ORC_F32) return ((const float*)base)[idx];
  return f32_from_bits((uint32_t)((const uint16_t*)base)[idx] << 16);
}

static size_t dtype_bytes(int dtype) { return dtype == ORC_F32 ? 4 : dtype == ORC_BF16 ? 2 : 1; }

/* ------------------------------------------------------------- KV write */

/*
 * k, v:          [T][H][D] in in_dtype (f32 or bf16)
 * slot_mapping:  [T]; slot < 0 skips the token (padding)
 * kc, vc:        [NB][H][bs][D] in cache_dtype
 * Same dtype: the element's bits are copied.  1-byte cache: the f32 value is
 * multiplied in f32 by inv_scale = 1.0f / scale and encoded as E4M3.
 */
int orc_paged_kv_write(const void* k, const void* v, int in_dtype, const int32_t* slot_mapping,
                       int64_t T, int32_t H, int32_t D, void* kc, void* vc, int cache_dtype,
                       int64_t NB, int32_t bs, float k_scale, float v_scale) {
  float inv_k = 1.0f, inv_v = 1.0f;
  int64_t t;
  if (H <= 0 || D <= 0 || bs <= 0 || NB < 0 || T < 0) return ORC_ERR_ARG;
  if (in_dtype != ORC_F32 && in_dtype != ORC_BF16) return ORC_ERR_ARG;
  if (cache_dtype != in_dtype && cache_dtype != ORC_FP8_E4M3) return ORC_ERR_ARG;
  if (cache_dtype == ORC_FP8_E4M3) {
    inv_k = 1.0f / k_scale;
    inv_v = 1.0f / v_scale;
  }
  for (t = 0; t < T; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot >= NB * (int64_t)bs) return ORC_ERR_RANGE;
  }
  /* tokens name distinct slots (caller contract), so they are independent */
#pragma omp parallel for schedule(static)
  for (t = 0; t < T; ++t) {
    int64_t slot = slot_mapping[t], blk, off;
    int32_t h, d;
    if (slot < 0) continue;
    blk = slot / bs;
    off = slot % bs;
    for (h = 0; h < H; ++h) {
      for (d = 0; d < D; ++d) {
        int64_t src = ((int64_t)t * H + h) * D + d;
        int64_t dst = ((blk * H + h) * bs + off) * D + d;
        if (cache_dtype == in_dtype) {
          size_t eb = dtype_bytes(in_dtype);
          memcpy((char*)kc + dst * eb, (const char*)k + src * eb, eb);
          memcpy((char*)vc + dst * eb, (const char*)v + src * eb, eb);
        } else {
          float xk = load_f32(k, src, in_dtype);
          float xv = load_f32(v, src, in_dtype);
          float yk = xk * inv_k; /* one f32 multiply, round to nearest even */
          float yv = xv * inv_v;
          ((uint8_t*)kc)[dst] = orc_e4m3_encode(yk);
          ((uint8_t*)vc)[dst] = orc_e4m3_encode(yv);
        }
      }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------- decode attention */

/*
 * q:             [S][Hq][D] in q_dtype (f32 or bf16)
 * kc, vc:        [NB][Hkv][bs][D] in cache_dtype (f32, bf16 or E4M3 codes)
 * block_tables:  [S][max_blocks]; entry j is the physical block of logical block j
 * context_lens:  [S]; tokens 0 .. len-1 of sequence s are attended
 * row_mask:      [S][Hq] (nonzero = compute) or NULL for every row
 * out:           [S][Hq][D] fp64; rows not computed are left untouched
 *
 * For a computed row (s, h), with n = context_lens[s] and hk = h / (Hq / Hkv):
 *   n == 0  ->  out = 0
 *   else    ->  K[t], V[t] = cache rows of token t (t < n) found through the
 *               table; z_t = scale * sum_d q[d] K[t][d];
 *               out = sum_t exp(z_t - max z) V[t] / sum_t exp(z_t - max z).
 */
int orc_paged_attention_decode(const void* q, int q_dtype, const void* kc, const void* vc,
                               int cache_dtype, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv,
                               int32_t D, int64_t NB, int32_t bs, int32_t max_blocks, float scale,
                               float k_scale, float v_scale, const uint8_t* row_mask, double* out) {
  int32_t G;
  int64_t pair;
  int status = ORC_OK;
  if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || max_blocks < 0) return ORC_ERR_ARG;
  if (Hq % Hkv != 0) return ORC_ERR_ARG;
  if (q_dtype != ORC_F32 && q_dtype != ORC_BF16) return ORC_ERR_ARG;
  if (cache_dtype != ORC_F32 && cache_dtype != ORC_BF16 && cache_dtype != ORC_FP8_E4M3)
    return ORC_ERR_ARG;
  G = Hq / Hkv;

  /* every table entry that will be read must name a block of the pool */
  for (int32_t s = 0; s < S; ++s) {
    int64_t n = context_lens[s];
    if (n < 0 || (n + bs - 1) / bs > max_blocks) return ORC_ERR_RANGE;
    for (int64_t j = 0; j < (n + bs - 1) / bs; ++j) {
      int32_t pb = block_tables[(int64_t)s * max_blocks + j];
      if (pb < 0 || pb >= NB) return ORC_ERR_RANGE;
    }
  }

#pragma omp parallel for schedule(dynamic, 1)
  for (pair = 0; pair < (int64_t)S * Hkv; ++pair) {
    int32_t s = (int32_t)(pair / Hkv), hk = (int32_t)(pair % Hkv);
    int64_t n = context_lens[s], t;
    int32_t g, d;
    int wanted = 0;
    double *Kc = NULL, *Vc = NULL, *z = NULL;
    for (g = 0; g < G; ++g)
      if (!row_mask || row_mask[(int64_t)s * Hq + hk * G + g]) wanted = 1;
    if (!wanted) continue;
    if (n > 0) {
      Kc = (double*)malloc(sizeof(double) * (size_t)(n * D));
      Vc = (double*)malloc(sizeof(double) * (size_t)(n * D));
      z = (double*)malloc(sizeof(double) * (size_t)n);
      if (!Kc || !Vc || !z) {
        free(Kc);
        free(Vc);
        free(z);
#pragma omp atomic write
        status = ORC_ERR_NOMEM;
        continue;
      }
      /* rebuild this KV head's contiguous K and V through the block table */
      for (t = 0; t < n; ++t) {
        int64_t pb = block_tables[(int64_t)s * max_blocks + t / bs];
        int64_t off = t % bs;
        for (d = 0; d < D; ++d) {
          int64_t idx = ((pb * Hkv + hk) * bs + off) * D + d;
          Kc[t * D + d] = load_elem(kc, idx, cache_dtype, (double)k_scale);
          Vc[t * D + d] = load_elem(vc, idx, cache_dtype, (double)v_scale);
        }
      }
    }
    for (g = 0; g < G; ++g) {
      int32_t h = hk * G + g;
      double* o = out + ((int64_t)s * Hq + h) * D;
      double zmax = -INFINITY, wsum = 0.0;
      if (row_mask && !row_mask[(int64_t)s * Hq + h]) continue;
      for (d = 0; d < D; ++d) o[d] = 0.0;
      if (n == 0) continue;
      for (t = 0; t < n; ++t) {
        double dot = 0.0;
        for (d = 0; d < D; ++d) dot += load_elem(q, ((int64_t)s * Hq + h) * D + d, q_dtype, 1.0) * Kc[t * D + d];
        z[t] = (double)scale * dot;
        if (z[t] > zmax) zmax = z[t];
      }
      for (t = 0; t < n; ++t) {
        double w = exp(z[t] - zmax);
        wsum += w;
        for (d = 0; d < D; ++d) o[d] += w * Vc[t * D + d];
      }
      for (d = 0; d < D; ++d) o[d] /= wsum;
    }
    free(Kc);
    free(Vc);
    free(z);
  }
  return status;
}

/* ------------------------------------------------------ block copy (CoW) */

/*
 * Copy-on-write support: before a branch writes into a physical block that
 * other sequences still list, the block's contents are copied to a fresh block
 * ("PagedAttention Memory Management", section "Complex Topologies and Memory
 * Sharing"; "What problem does PagedAttention solve...", section "Sharing, the
 * second dividend").  For every pair (src, dst) with both ids >= 0, block dst of
 * the K pool and of the V pool becomes a byte copy of block src; pairs with a
 * negative id are skipped.  block_bytes is the size of one block of one pool.
 */
int orc_copy_blocks(void* kc, void* vc, int64_t num_blocks, int64_t block_bytes,
                    const int32_t* pairs, int64_t num_pairs) {
  int64_t i;
  if (num_blocks < 0 || block_bytes < 0 || num_pairs < 0) return ORC_ERR_ARG;
  for (i = 0; i < num_pairs; ++i) {
    int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || dst < 0) continue;
    if (src >= num_blocks || dst >= num_blocks) return ORC_ERR_RANGE;
  }
  for (i = 0; i < num_pairs; ++i) {
    int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || dst < 0 || src == dst) continue;
    memcpy((char*)kc + (int64_t)dst * block_bytes, (const char*)kc + (int64_t)src * block_bytes,
           (size_t)block_bytes);
    memcpy((char*)vc + (int64_t)dst * block_bytes, (const char*)vc + (int64_t)src * block_bytes,
           (size_t)block_bytes);
  }
  return ORC_OK;
}

/*
 * Swap-out / swap-in ("What problem does PagedAttention solve...", section
 * "Operational consequences": a preempted sequence's state is swapped out and
 * later written back into free blocks).  Staging slot i <-> pool block ids[i];
 * a negative id skips slot i.  gather: stage[i] = pool[ids[i]];
 * scatter: pool[ids[i]] = stage[i], in increasing i.
 */
int orc_move_blocks(void* pool, int64_t num_blocks, int64_t block_bytes, void* stage,
                    const int32_t* ids, int64_t n, int gather) {
  int64_t i;
  if (num_blocks < 0 || block_bytes < 0 || n < 0) return ORC_ERR_ARG;
  for (i = 0; i < n; ++i)
    if (ids[i] >= num_blocks) return ORC_ERR_RANGE;
  for (i = 0; i < n; ++i) {
    char* blk;
    char* slot = (char*)stage + i * block_bytes;
    if (ids[i] < 0) continue;
    blk = (char*)pool + (int64_t)ids[i] * block_bytes;
    if (gather)
      memcpy(slot, blk, (size_t)block_bytes);
    else
      memcpy(blk, slot, (size_t)block_bytes);
  }
  return ORC_OK;
}

int orc_abi_version(void) { return 1; }

/* ---------------------------------------------------------- chunked prefill */

/*
 * q:                [T][Hq][D], q_dtype (f32 or bf16); rows of sequence s are
 *                   query_start[s] .. query_start[s+1]-1
 * query_start:      [S+1], non-decreasing, query_start[0] = 0
 * context_lens:     [S]; the n_s = query_start[s+1] - query_start[s] queries
 *                   of sequence s are its positions context_lens[s] - n_s ..
 *                   context_lens[s] - 1 (n_s <= context_lens[s])
 * the rest:         as orc_paged_attention_decode
 * out:              [T][Hq][D] fp64; query i of sequence s, head h, at position
 *                   p = context_lens[s] - n_s + i:
 *                   out = sum_{t <= p} softmax_t(scale q.K_t) V_t
 */
int orc_paged_attention_prefill(const void* q, int q_dtype, const void* kc, const void* vc,
                                int cache_dtype, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* query_start,
                                int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int64_t NB,
                                int32_t bs, int32_t max_blocks, float scale, float k_scale,
                                float v_scale, double* out) {
  int32_t G;
  int64_t pair;
  int status = ORC_OK;
  if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || max_blocks < 0) return ORC_ERR_ARG;
  if (Hq % Hkv != 0) return ORC_ERR_ARG;
  if (q_dtype != ORC_F32 && q_dtype != ORC_BF16) return ORC_ERR_ARG;
  if (cache_dtype != ORC_F32 && cache_dtype != ORC_BF16 && cache_dtype != ORC_FP8_E4M3)
    return ORC_ERR_ARG;
  if (query_start[0] != 0) return ORC_ERR_ARG;
  G = Hq / Hkv;

  for (int32_t s = 0; s < S; ++s) {
    int64_t n = context_lens[s];
    int64_t nq = (int64_t)query_start[s + 1] - query_start[s];
    if (nq < 0 || nq > n) return ORC_ERR_RANGE;
    if (n < 0 || (n + bs - 1) / bs > max_blocks) return ORC_ERR_RANGE;
    for (int64_t j = 0; j < (n + bs - 1) / bs; ++j) {
      int32_t pb = block_tables[(int64_t)s * max_blocks + j];
      if (pb < 0 || pb >= NB) return ORC_ERR_RANGE;
    }
  }

#pragma omp parallel for schedule(dynamic, 1)
  for (pair = 0; pair < (int64_t)S * Hkv; ++pair) {
    int32_t s = (int32_t)(pair / Hkv), hk = (int32_t)(pair % Hkv);
    int64_t n = context_lens[s], t, i;
    int64_t q0 = query_start[s], nq = (int64_t)query_start[s + 1] - query_start[s];
    int32_t g, d;
    double *Kc, *Vc, *z;
    if (nq == 0) continue;
    Kc = (double*)malloc(sizeof(double) * (size_t)(n * D));
    Vc = (double*)malloc(sizeof(double) * (size_t)(n * D));
    z = (double*)malloc(sizeof(double) * (size_t)n);
    if (!Kc || !Vc || !z) {
      free(Kc);
      free(Vc);
      free(z);
#pragma omp atomic write
      status = ORC_ERR_NOMEM;
      continue;
    }
    /* this KV head's contiguous K and V, through the block table */
    for (t = 0; t < n; ++t) {
      int64_t pb = block_tables[(int64_t)s * max_blocks + t / bs];
      int64_t off = t % bs;
      for (d = 0; d < D; ++d) {
        int64_t idx = ((pb * Hkv + hk) * bs + off) * D + d;
        Kc[t * D + d] = load_elem(kc, idx, cache_dtype, (double)k_scale);
        Vc[t * D + d] = load_elem(vc, idx, cache_dtype, (double)v_scale);
      }
    }
    for (i = 0; i < nq; ++i) {
      int64_t row = q0 + i;
      int64_t pos = n - nq + i; /* keys 0 .. pos are visible */
      for (g = 0; g < G; ++g) {
        int32_t h = hk * G + g;
        double* o = out + (row * Hq + h) * D;
        double zmax = -INFINITY, wsum = 0.0;
        for (d = 0; d < D; ++d) o[d] = 0.0;
        for (t = 0; t <= pos; ++t) {
          double dot = 0.0;
          for (d = 0; d < D; ++d) dot += load_elem(q, (row * Hq + h) * D + d, q_dtype, 1.0) * Kc[t * D + d];
          z[t] = (double)scale * dot;
          if (z[t] > zmax) zmax = z[t];
        }
        for (t = 0; t <= pos; ++t) {
          double w = exp(z[t] - zmax);
          wsum += w;
          for (d = 0; d < D; ++d) o[d] += w * Vc[t * D + d];
        }
        for (d = 0; d < D; ++d) o[d] /= wsum;
      }
    }
    free(Kc);
    free(Vc);
    free(z);
  }
  return status;
}
