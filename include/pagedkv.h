/*
 * pagedkv.h -- C ABI of libpagedkv.so: the paged KV cache hot path on AMD
 * Instinct MI355X (gfx950).
 *
 * Device operations (the first two are the hot path; the others build on the
 * same kernels and pool layout):
 *
 *   paged_kv_write          the slot-mapped KV-cache write.  Each new token's
 *                           key and value rows land in one slot (physical
 *                           block, offset) of a shared pool of fixed-size
 *                           blocks.  Source: "PagedAttention, clearly
 *                           explained" (a block holds the K/V of a fixed number
 *                           of consecutive tokens; a sequence only holds blocks
 *                           it has written) and "What problem does
 *                           PagedAttention solve for the KV cache in vLLM?",
 *                           section "The paging idea" (blocks are allocated as
 *                           the sequence grows).
 *
 *   paged_attention_decode  attention for one new query token per sequence,
 *                           with keys and values gathered through the
 *                           sequence's block table.  Source: the same thread (at
 *                           each decode step the kernel reads the block table
 *                           and gathers K/V from whichever physical blocks they
 *                           landed in) and "pipe-paged-block-allocation-kv-cache",
 *                           sections "In and out" (the table is handed to the
 *                           attention kernel, which gathers through that
 *                           indirection; output is identical given the same
 *                           reduction order) and "Concept" (attention is a
 *                           weighted sum over logically ordered positions).
 *
 *   paged_attention_decode_append   the two above in one launch for one new
 *                           token per sequence.
 *   paged_attention_decode_shared_prefix   decode for sequences that share a
 *                           prefix: the shared part computed once (cascade).
 *   paged_attention_decode_shared_prefix_append   the same with each
 *                           sequence's new token written in the tails' launch.
 *   paged_attention_prefill chunked prefill: many new query tokens per
 *                           sequence, causal, the cached prefix read through
 *                           the block table.
 *   paged_kv_copy_blocks    copy-on-write copies of whole blocks.
 *   paged_kv_gather_blocks / paged_kv_scatter_blocks   swap-out / swap-in of
 *                           whole blocks to and from a staging buffer.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are passed as pkv_tensor descriptors.  The library never
 *    allocates, frees or retains caller memory; every buffer is owned by the
 *    caller and must stay alive until the work queued on the stream is done.
 *  - Device entry points are asynchronous on `hip_stream` (a hipStream_t; NULL
 *    means the default stream).  They do not synchronize and do not allocate.
 *  - Validation looks only at descriptors, never at device memory.  On failure
 *    nothing is launched, a status other than PKV_OK is returned and
 *    pkv_last_error() describes it.  Kernels never trap: block ids, context
 *    lengths and slots are the caller's contract (see pkv_validate_* to check
 *    host copies).
 *  - Layouts (all row-major and dense, strides in elements):
 *      k, v            [T, Hkv, D]         new tokens
 *      slot_mapping    [T] int32           slot = block * block_size + offset; < 0 skips
 *      key_cache,
 *      value_cache     [NB, Hkv, bs, D]    one layer's pool (a block id names the
 *                                          same block in every layer's pool)
 *      q, out          [S, Hq, D]          query head h reads KV head h / (Hq / Hkv)
 *      block_tables    [S, max_blocks] int32  entry j = physical block of tokens
 *                                          j*bs .. j*bs+bs-1
 *      context_lens    [S] int32           tokens attended by sequence s (the new
 *                                          token included: write first, then decode)
 *  - Element types: f32 cache with f32 q/out/k/v; bf16 cache with bf16
 *    q/out/k/v; E4M3 cache (OCP 8-bit float, 1 sign / 4 exponent (bias 7) /
 *    3 mantissa bits, no infinities, max 448) with bf16 q/out, f32 or bf16
 *    k/v for the write, and a per-tensor scale carried in the cache
 *    descriptor: stored value = code value * scale.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 10
#define PKV_MAX_DIMS 4

typedef enum {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  PKV_FP8_E4M3 = 2,
  PKV_I32 = 3
} pkv_dtype;

typedef struct {
  void* data;                    /* device pointer (host pointer for pkv_validate_*) */
  int32_t dtype;                 /* pkv_dtype */
  int32_t ndim;                  /* number of used entries in shape/stride, <= 4 */
  int64_t shape[PKV_MAX_DIMS];
  int64_t stride[PKV_MAX_DIMS];  /* in elements; the kernels require dense row-major (a
                                    tensor with no elements may have any strides) */
  float scale;                   /* E4M3 tensors: dequantisation scale (> 0, finite);
                                    ignored for other element types */
} pkv_tensor;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required descriptor or data pointer is NULL */
  PKV_ERR_DTYPE = 2,       /* unsupported or mismatched element types */
  PKV_ERR_SHAPE = 3,       /* ranks or sizes disagree */
  PKV_ERR_LAYOUT = 4,      /* not dense row-major, or an output aliases an input */
  PKV_ERR_UNSUPPORTED = 5, /* head_dim, block_size, group size or partition size outside
                              what the kernels are built for */
  PKV_ERR_WORKSPACE = 6,   /* split-K workspace missing or too small */
  PKV_ERR_HIP = 7,         /* the HIP runtime reported an error at launch */
  PKV_ERR_RANGE = 8        /* pkv_validate_*: an id, length or slot is out of range */
} pkv_status;

typedef enum {
  /* one workgroup per (sequence, KV head) walks the whole context */
  PKV_DECODE_SINGLE_PASS = 0,
  /* split-K: the context of each (sequence, KV head) is cut into partitions
     of partition_size tokens; each partition's partial softmax state goes to
     the workspace and a merge kernel combines a sequence's partitions in
     partition order (sequences that fit in one partition are finalised in
     place).  With one wavefront per partition (the default up to 512 tokens)
     persistent wavefronts, 4 per compute unit, stream equal runs of the
     (sequence, KV head, partition) list back to back; otherwise one
     workgroup per partition.  Either way a partition's state is computed from
     the same tiles in the same order, so the results are the same. */
  PKV_DECODE_PARTITIONED = 1,
  /* balanced split: the 16-token tiles of all (sequence, KV head) pairs are
     flattened and num_workers wavefronts each take an equal contiguous run,
     so all of them stream the same number of bytes whatever the spread of
     context lengths; a pair covered by several runs is merged from the
     workspace in run order */
  PKV_DECODE_BALANCED = 2,
  /* the library picks from the sizes it can see (no context lengths): many
     (sequence, KV head) pairs (at least 16 per compute unit) -> single pass
     with 4 wavefronts per workgroup; otherwise balanced, with 8 workers per
     compute unit from 8 pairs per compute unit up, else 4 */
  PKV_DECODE_AUTO = 3
} pkv_decode_mode;

typedef struct {
  int32_t mode;             /* pkv_decode_mode */
  int32_t partition_size;   /* PARTITIONED: tokens per partition, a positive multiple of 16 */
  int32_t waves_per_group;  /* SINGLE_PASS / PARTITIONED: wavefronts per workgroup walking
                               disjoint tiles: 0 = library default (1 for partitions of at
                               most 512 tokens, else 4), else 1, 2, 4 or 8 */
  int32_t num_workers;      /* BALANCED, and PARTITIONED with one wavefront per partition:
                               wavefronts sharing the work; 0 = library default (4 per
                               compute unit of the current device) */
  void* workspace;          /* device memory, >= paged_attention_decode_workspace_bytes();
                               not needed for SINGLE_PASS */
  size_t workspace_bytes;
  int32_t flags;            /* PKV_DECODE_* flags below, or 0 */
  const int32_t* seq_order; /* SINGLE_PASS / PARTITIONED with more than one wavefront per
                               workgroup (also AUTO when it picks the single pass): NULL,
                               or device int32 [num_seqs], a permutation of
                               0..num_seqs-1 giving the order in which the sequences'
                               workgroups start.  Longest context first (pkv_decode_order)
                               keeps a long sequence from starting last and running alone
                               when the lengths vary.  Only the schedule changes: results
                               are bit-identical for every permutation.  An entry outside
                               [0, num_seqs) makes its workgroups exit, and a repeated
                               entry leaves another sequence's rows unwritten
                               (pkv_validate_seq_order checks a host copy).  BALANCED,
                               one-wavefront PARTITIONED and the shared-prefix calls
                               ignore it. */
} pkv_decode_opts;

/* opts->flags: launch only the streaming kernel and leave its partial states
 * in the workspace; the caller then calls paged_attention_decode_merge with
 * the same arguments on the same stream before reading `out` or reusing the
 * workspace.  Lets a caller time or schedule the two kernels apart.  Modes
 * without a merge (single pass, one partition) finish in the first call. */
#define PKV_DECODE_DEFER_MERGE 1

/* opts->flags: the batch's K/V blocks are each read once by this call (no
 * physical block appears in two sequences' tables, e.g. every refcount is 1),
 * so the pool reads carry the non-temporal hint: they stream past L2 and the
 * MALL instead of filling them.  Results are bit-identical with or without the
 * flag; only speed changes.  Measured on MI355X: faster on unshared batches,
 * much slower when many sequences share blocks (their reuse is then lost), so
 * it is off unless the caller knows the blocks are unshared. */
#define PKV_DECODE_STREAM_KV 2

/* Version of this header the library was built from (PKV_ABI_VERSION). */
int32_t pkv_abi_version(void);

/* Message for the last non-OK status returned on the calling thread ("" if
 * none).  The pointer stays valid until the next call on the same thread. */
const char* pkv_last_error(void);

/*
 * Slot-mapped KV-cache write.
 *   k, v          [T, Hkv, D], f32 or bf16 (same type for both)
 *   slot_mapping  [T] int32; token t goes to block slot / bs, offset slot % bs;
 *                 a negative slot skips the token
 *   key_cache,
 *   value_cache   [NB, Hkv, bs, D]
 * Same element type in and out: the bits are copied.  E4M3 cache: each value
 * is multiplied in f32 by inv = 1.0f / cache.scale (inv formed once in f32)
 * and rounded to the nearest E4M3 value, ties to even; magnitudes past 448
 * and infinities become +-448; NaN becomes code 0x7F.
 * Slots must be distinct and < NB * bs (caller contract; duplicates race,
 * out-of-range slots write outside the pool).  Cache bytes of slots not named
 * are never touched.
 * Errors: PKV_ERR_NULL, PKV_ERR_DTYPE, PKV_ERR_SHAPE, PKV_ERR_LAYOUT,
 * PKV_ERR_UNSUPPORTED (D not a multiple of 8), PKV_ERR_HIP.
 */
pkv_status paged_kv_write(const pkv_tensor* k, const pkv_tensor* v,
                          const pkv_tensor* slot_mapping, pkv_tensor* key_cache,
                          pkv_tensor* value_cache, void* hip_stream);

/*
 * Decode attention over the paged cache.
 *   out           [S, Hq, D], same element type as q (f32 or bf16)
 *   q             [S, Hq, D]
 *   key_cache,
 *   value_cache   [NB, Hkv, bs, D]; bs == block_size
 *   block_tables  [S, max_blocks] int32; entries j < ceil(len/bs) must be in [0, NB)
 *   context_lens  [S] int32; 0 <= len <= max_blocks * bs
 *   scale         multiplies q.k before the softmax (e.g. 1/sqrt(D))
 *   opts          NULL = single pass with the default wave count
 * For each sequence s and query head h (KV head hk = h / (Hq / Hkv)):
 *   out[s,h,:] = sum_t softmax_t(scale * q[s,h,:].K[t,:]) V[t,:] over t < len,
 *   K/V rows read through the table; len == 0 gives zeros.  Slots past len and
 *   blocks not listed may hold any bits, NaN included: they never reach out.
 * Supported: Hq % Hkv == 0 with Hq / Hkv <= 16, D in {64, 128}, block_size a
 * multiple of 16 up to 256.
 * Results are deterministic and do not depend on which physical blocks hold
 * the tokens.
 * Errors: PKV_ERR_NULL, PKV_ERR_DTYPE, PKV_ERR_SHAPE, PKV_ERR_LAYOUT,
 * PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP.
 */
pkv_status paged_attention_decode(pkv_tensor* out, const pkv_tensor* q,
                                  const pkv_tensor* key_cache, const pkv_tensor* value_cache,
                                  const pkv_tensor* block_tables,
                                  const pkv_tensor* context_lens, float scale,
                                  int32_t block_size, const pkv_decode_opts* opts,
                                  void* hip_stream);

/*
 * paged_attention_decode for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, result and errors as paged_attention_decode, but the split
 * workspace is the library's own scratch: one fixed device array of
 * pkv_noalloc_scratch_bytes() (32 MiB) that each GPU holds from the library's
 * load until the process ends.  The call allocates nothing and frees nothing.
 *   opts->workspace / workspace_bytes   ignored (the scratch takes their place)
 *   opts->flags                         PKV_DECODE_DEFER_MERGE is refused
 * A call whose mode needs more split workspace than the scratch holds fails
 * with PKV_ERR_WORKSPACE before anything is launched (e.g. 512-token partitions
 * of 8 x 131072-token sequences need ~30 MB; the balanced split of a
 * 64-sequence batch ~5 MB).  Nothing in the scratch has to start at zero.
 * All calls on one GPU share its scratch: calls that overlap on one GPU (on
 * different streams, not ordered by events) race and give wrong results.
 */
pkv_status paged_attention_decode_noalloc(pkv_tensor* out, const pkv_tensor* q,
                                          const pkv_tensor* key_cache,
                                          const pkv_tensor* value_cache,
                                          const pkv_tensor* block_tables,
                                          const pkv_tensor* context_lens, float scale,
                                          int32_t block_size, const pkv_decode_opts* opts,
                                          void* hip_stream);

/* Bytes of scratch behind paged_attention_decode_noalloc (per GPU). */
size_t pkv_noalloc_scratch_bytes(void);

/*
 * Second half of a call made with PKV_DECODE_DEFER_MERGE: merges the partial
 * states the streaming kernel left in the workspace into `out`.  Arguments and
 * errors as for paged_attention_decode (all of them as in the first call);
 * launches nothing when the mode has no merge.
 */
pkv_status paged_attention_decode_merge(pkv_tensor* out, const pkv_tensor* q,
                                        const pkv_tensor* key_cache,
                                        const pkv_tensor* value_cache,
                                        const pkv_tensor* block_tables,
                                        const pkv_tensor* context_lens, float scale,
                                        int32_t block_size, const pkv_decode_opts* opts,
                                        void* hip_stream);

/*
 * Decode attention for a batch whose sequences all begin with the same
 * prefix_len tokens, held once in shared physical blocks (a system prompt or a
 * forked prompt: "PagedAttention Memory Management", section "Complex
 * Topologies and Memory Sharing"; "What problem does PagedAttention solve...",
 * section "Sharing, the second dividend").  The shared part is computed once
 * for all sequences (their query heads against the prefix keys on the matrix
 * cores, the prefix K/V read once), each sequence's own tail streams through
 * the balanced split, and the partial softmax states are merged in a fixed
 * order (prefix pieces, then tail pieces).
 *   prefix_len    a positive multiple of block_size; every table's first
 *                 prefix_len / block_size entries name the same blocks and
 *                 every context_len >= prefix_len (pkv_validate_shared_prefix)
 *   the rest      as paged_attention_decode; opts->mode must be AUTO or
 *                 BALANCED (or opts NULL), num_workers is honoured,
 *                 PKV_DECODE_DEFER_MERGE is refused, and the workspace must hold
 *                 paged_attention_decode_shared_prefix_workspace_bytes()
 * Result: attention over each whole context, equal within rounding to
 * paged_attention_decode on the same inputs; deterministic.
 * Errors: as paged_attention_decode.
 */
pkv_status paged_attention_decode_shared_prefix(pkv_tensor* out, const pkv_tensor* q,
                                                const pkv_tensor* key_cache,
                                                const pkv_tensor* value_cache,
                                                const pkv_tensor* block_tables,
                                                const pkv_tensor* context_lens, int32_t prefix_len,
                                                float scale, int32_t block_size,
                                                const pkv_decode_opts* opts, void* hip_stream);

/*
 * One decode step in one call: the KV write of each sequence's new token (the
 * token the step attends last) followed by decode attention, with the write
 * folded into the decode launch.  Same sources as the two operations: the new
 * token is written first, then attended with the rest of its context.
 *   k, v          [S, Hkv, D], q's element type: sequence s's new K/V rows
 *                 (bf16 for an E4M3 cache, quantized as paged_kv_write does)
 *   slot_mapping  [S] int32: slot of sequence s's new token; negative = no write
 *   the rest      as for paged_attention_decode
 * Result: the same cache bytes and, bit for bit, the same `out` as
 * paged_kv_write(k, v, slot_mapping, ...) followed by paged_attention_decode
 * with the same options, provided each non-negative slot is position
 * len - 1 of its own sequence (table entry (len-1) / bs, offset (len-1) % bs)
 * and its block is read by no other sequence in the call
 * (pkv_validate_append_slots checks host copies).  Then the row is read from
 * k / v by the kernel that attends it and stored to its slot from registers.
 * A slot that is not position len - 1 is still written, and the attention
 * reads that position from the pool; if any sequence of the call reads the
 * written slot, its result is undefined (the read races the write).
 * Errors: as paged_attention_decode, and PKV_ERR_NULL / PKV_ERR_DTYPE /
 * PKV_ERR_SHAPE / PKV_ERR_LAYOUT for k, v and slot_mapping.
 */
pkv_status paged_attention_decode_append(pkv_tensor* out, const pkv_tensor* q,
                                         const pkv_tensor* k, const pkv_tensor* v,
                                         const pkv_tensor* slot_mapping, pkv_tensor* key_cache,
                                         pkv_tensor* value_cache,
                                         const pkv_tensor* block_tables,
                                         const pkv_tensor* context_lens, float scale,
                                         int32_t block_size, const pkv_decode_opts* opts,
                                         void* hip_stream);

/*
 * One decode step for sequences that share a prefix, in one call: each
 * sequence's new token is written by the launch that attends its tail
 * (paged_attention_decode_append's folding), and the shared part is computed
 * once (paged_attention_decode_shared_prefix).  Same sources as the two.  The
 * new token is private to its sequence: a block shared by several sequences
 * is copied before it is written (paged_kv_copy_blocks), so the token lies in
 * the tail.
 *   k, v, slot_mapping  as paged_attention_decode_append
 *   prefix_len, the rest  as paged_attention_decode_shared_prefix, and every
 *                 context_len > prefix_len (a sequence whose new token would
 *                 fall inside the prefix gets an undefined result)
 * Result: the same cache bytes and, bit for bit, the same `out` as
 * paged_kv_write(k, v, slot_mapping, ...) followed by
 * paged_attention_decode_shared_prefix with the same options, under the slot
 * conditions of paged_attention_decode_append (pkv_validate_append_slots).
 * Errors: as paged_attention_decode_shared_prefix, and those of
 * paged_attention_decode_append for k, v and slot_mapping.
 */
pkv_status paged_attention_decode_shared_prefix_append(
    pkv_tensor* out, const pkv_tensor* q, const pkv_tensor* k, const pkv_tensor* v,
    const pkv_tensor* slot_mapping, pkv_tensor* key_cache, pkv_tensor* value_cache,
    const pkv_tensor* block_tables, const pkv_tensor* context_lens, int32_t prefix_len, float scale,
    int32_t block_size, const pkv_decode_opts* opts, void* hip_stream);

typedef struct {
  int32_t rows_per_wave;  /* (query token, query head) rows per wavefront: 0 = library
                             default (32; 16 for f32), 16, 32, or 64 (head_dim 64, not f32) */
} pkv_prefill_opts;

/*
 * Chunked-prefill attention over the paged cache: several new query tokens
 * per sequence, each attending causally to the sequence's cached prefix (read
 * through the block table) and to the chunk's earlier tokens.  Source: "What
 * problem does PagedAttention solve for the KV cache in vLLM?", section
 * "Sharing, the second dividend" (reused prefix blocks skip that part of
 * prefill; the rest of the prompt attends over them through the table), and
 * "pipe-paged-block-allocation-kv-cache", section "Effect".
 *   out              [T, Hq, D], q's element type
 *   q                [T, Hq, D]; rows query_start_loc[s] .. query_start_loc[s+1]-1
 *                    are sequence s's chunk of n_s tokens
 *   query_start_loc  [S + 1] int32, non-decreasing, [0] = 0, [S] = T
 *   context_lens     [S] int32; the chunk is the last n_s <= len positions: its
 *                    K/V must already be in the pool (paged_kv_write first)
 *   max_query_len    >= every n_s; sizes the launch (a longer chunk is still
 *                    computed correctly, with fewer workgroups than it could use)
 *   key_cache, value_cache, block_tables, scale, block_size: as for
 *                    paged_attention_decode
 *   opts             NULL = defaults
 * For sequence s, query i at position p = len - n_s + i and query head h:
 *   out[row,h,:] = sum_{t <= p} softmax_t(scale * q[row,h,:].K[t,:]) V[t,:].
 * Slots past len and blocks not listed may hold any bits; they never reach out.
 * Results are deterministic and do not depend on which physical blocks hold
 * the tokens.  No workspace is needed.
 * Errors: PKV_ERR_NULL, PKV_ERR_DTYPE, PKV_ERR_SHAPE, PKV_ERR_LAYOUT,
 * PKV_ERR_UNSUPPORTED, PKV_ERR_HIP.
 */
pkv_status paged_attention_prefill(pkv_tensor* out, const pkv_tensor* q,
                                   const pkv_tensor* key_cache, const pkv_tensor* value_cache,
                                   const pkv_tensor* block_tables, const pkv_tensor* context_lens,
                                   const pkv_tensor* query_start_loc, int32_t max_query_len,
                                   float scale, int32_t block_size, const pkv_prefill_opts* opts,
                                   void* hip_stream);

/*
 * Copy-on-write block copies.  A physical block listed by several block tables
 * is copied to a fresh block before one branch writes into it ("PagedAttention
 * Memory Management", section "Complex Topologies and Memory Sharing"; "What
 * problem does PagedAttention solve...", section "Sharing, the second
 * dividend").
 *   key_cache,
 *   value_cache   [NB, Hkv, bs, D], same shape and element type
 *   block_pairs   [P, 2] int32 rows (src, dst): block dst of both pools becomes a
 *                 byte copy of block src; a row with a negative id, or src == dst,
 *                 is skipped
 * Caller contract (checked on host copies by pkv_validate_block_pairs): ids
 * < NB, destinations distinct, and no destination is also a source, so the
 * result does not depend on the order of the copies.
 * Errors: PKV_ERR_NULL, PKV_ERR_DTYPE, PKV_ERR_SHAPE, PKV_ERR_LAYOUT, PKV_ERR_HIP.
 */
pkv_status paged_kv_copy_blocks(pkv_tensor* key_cache, pkv_tensor* value_cache,
                                const pkv_tensor* block_pairs, void* hip_stream);

/*
 * Swap-out and swap-in of whole blocks (preemption under memory pressure:
 * "What problem does PagedAttention solve for the KV cache in vLLM?", section
 * "Operational consequences": a preempted sequence's blocks are freed and its
 * state swapped out, to be written back into free blocks later).
 *   key_cache, value_cache  [NB, Hkv, bs, D]
 *   block_ids               [n] int32; a negative id skips its staging slot
 *   out_k/out_v, in_k/in_v  [n, Hkv, bs, D], the pools' element type: staging
 *                           slot i holds block block_ids[i]; device memory (a
 *                           host copy is then one contiguous copy-engine
 *                           transfer per buffer, made by the caller)
 * gather: out[i] = pool[block_ids[i]];  scatter: pool[block_ids[i]] = in[i].
 * Caller contract (pkv_validate_block_ids on host copies): ids < NB, and for a
 * scatter no id repeated.  The staging buffers must not overlap the pools.
 * Errors: PKV_ERR_NULL, PKV_ERR_DTYPE, PKV_ERR_SHAPE, PKV_ERR_LAYOUT (also: a
 * pool or staging pointer that is not device memory), PKV_ERR_HIP.
 */
pkv_status paged_kv_gather_blocks(const pkv_tensor* key_cache, const pkv_tensor* value_cache,
                                  const pkv_tensor* block_ids, pkv_tensor* out_k,
                                  pkv_tensor* out_v, void* hip_stream);
pkv_status paged_kv_scatter_blocks(const pkv_tensor* in_k, const pkv_tensor* in_v,
                                   const pkv_tensor* block_ids, pkv_tensor* key_cache,
                                   pkv_tensor* value_cache, void* hip_stream);

/* Measurement support, not a step of the method: the device's attainable
 * streaming-read rate, against which the decode kernels' byte rates are
 * reported next to the datasheet peak.  Reads `bytes` of device memory at
 * `buf` once (16-byte non-temporal loads, pkv_read_probe_blocks() workgroups
 * of 256 threads) and writes to sink[b] the XOR of the 32-bit words that
 * workgroup b read, so the XOR of all sink words is the XOR of the buffer's
 * words.  buf and sink: device memory (PKV_ERR_LAYOUT otherwise), buf 16-byte
 * aligned and bytes a multiple of 16 (PKV_ERR_SHAPE); sink holds at least
 * pkv_read_probe_blocks() words.  bytes 0: nothing is launched.  Asynchronous
 * on hip_stream. */
int32_t pkv_read_probe_blocks(void);
pkv_status pkv_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* hip_stream);

/* Measurement support, not a step of the method: the gather ceiling of the
 * decode's tile stream on a bf16, head-dim-128 pool (rows of 256 bytes).
 * tile_rows (device int32 [num_tiles]) names the first of 16 consecutive pool
 * rows of each tile (row = (block * num_kv_heads + head) * block_size +
 * offset); K comes from key_cache, V from value_cache, at the same rows.
 * `workers` wavefronts (4 per workgroup) each read an equal contiguous run of
 * the list, the balanced split without its arithmetic:
 *   mode 0: the decode's own operand loads, straight into registers;
 *   mode 1: each tile staged through LDS first (global-to-LDS copies, 1 KB
 *           contiguous per instruction, two tiles in flight per wavefront),
 *           then the same operands read from LDS.
 * sink[b] gets the XOR of what workgroup b read; sink holds (workers + 3) / 4
 * words.  A row outside [0, num_rows - 16] reads row 0 instead.  Device
 * pointers (PKV_ERR_LAYOUT), 16-byte aligned pools (PKV_ERR_SHAPE), workers in
 * [1, 2^20] and mode 0 or 1 (PKV_ERR_UNSUPPORTED).  Asynchronous on hip_stream. */
pkv_status pkv_tile_gather_probe(const void* key_cache, const void* value_cache,
                                 const int32_t* tile_rows, int64_t num_tiles, int64_t num_rows,
                                 int32_t workers, int32_t mode, uint32_t* sink, void* hip_stream);

/* Workspace bytes paged_attention_decode needs with these sizes and options
 * (0 when none is needed: no sequences, single pass, or one partition per
 * sequence).
 * Returns 0 as well for invalid arguments. */
size_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t max_blocks_per_seq, int32_t block_size,
                                              const pkv_decode_opts* opts);

/* Workspace bytes of paged_attention_decode_shared_prefix (0 for invalid
 * arguments). */
size_t paged_attention_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                            int32_t num_kv_heads, int32_t head_dim,
                                                            int32_t max_blocks_per_seq,
                                                            int32_t block_size, int32_t prefix_len,
                                                            const pkv_decode_opts* opts);

/*
 * Longest-context-first order of a batch, on HOST arrays, for
 * pkv_decode_opts.seq_order: order[i] is the sequence with the i-th longest
 * context, ties in index order.  A list schedule that starts the longest jobs
 * first ends close to the average load; with the sequences in their given
 * order a long one can start last and run alone.  Returns PKV_OK,
 * PKV_ERR_NULL or PKV_ERR_SHAPE (num_seqs < 0).
 */
pkv_status pkv_decode_order(const int32_t* context_lens, int32_t num_seqs, int32_t* order);

/*
 * Opt-in host-side checks of the caller contract, on HOST copies.
 * pkv_validate_slots: every slot < num_blocks * block_size and no slot
 *   repeated among the non-negative ones.
 * pkv_validate_decode_inputs: every context length in [0, max_blocks * bs]
 *   and every table entry j < ceil(len / bs) in [0, num_blocks).
 * Return PKV_OK, PKV_ERR_NULL, PKV_ERR_SHAPE (bad sizes) or PKV_ERR_RANGE.
 */
pkv_status pkv_validate_slots(const int32_t* slots, int64_t num_tokens, int64_t num_blocks,
                              int32_t block_size);
pkv_status pkv_validate_decode_inputs(const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, int32_t block_size);
/* pkv_validate_append_slots: the decode inputs as above, and every slot >= 0
 * is position len - 1 of its sequence (so len > 0) in a block that no other
 * sequence reads. */
pkv_status pkv_validate_append_slots(const int32_t* slots, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t max_blocks_per_seq, int64_t num_blocks,
                                     int32_t block_size);
/* pkv_validate_prefill_inputs: the decode inputs as above, query_start_loc
 * starts at 0, never decreases and ends at num_query_rows, and every chunk is
 * at most its context length and at most max_query_len. */
pkv_status pkv_validate_prefill_inputs(const int32_t* query_start_loc, const int32_t* block_tables,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t max_blocks_per_seq, int64_t num_blocks,
                                       int32_t block_size, int64_t num_query_rows,
                                       int32_t max_query_len);
/* pkv_validate_shared_prefix: the decode inputs as above, every context
 * length >= prefix_len and every table lists the same prefix blocks. */
pkv_status pkv_validate_shared_prefix(const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, int32_t block_size, int32_t prefix_len);
/* pkv_validate_seq_order: a permutation of 0..num_seqs-1. */
pkv_status pkv_validate_seq_order(const int32_t* seq_order, int32_t num_seqs);
/* pkv_validate_block_ids: every id >= 0 is < num_blocks and none repeats. */
pkv_status pkv_validate_block_ids(const int32_t* block_ids, int64_t num_ids, int64_t num_blocks);
/* pkv_validate_block_pairs: rows with both ids >= 0 name blocks < num_blocks,
 * their destinations are distinct and none is also a source. */
pkv_status pkv_validate_block_pairs(const int32_t* block_pairs, int64_t num_pairs,
                                    int64_t num_blocks);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
