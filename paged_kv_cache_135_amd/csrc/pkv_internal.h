// Internal declarations shared by the HIP translation units of libpagedkv.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

// One KV-cache write launch: T tokens x Hkv heads x D elements for K and V.
struct WriteArgs {
  const void* k;
  const void* v;
  const int32_t* slots;
  void* kc;
  void* vc;
  int64_t num_tokens;
  int32_t num_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t in_dtype;     // PKV_F32 or PKV_BF16
  int32_t cache_dtype;  // in_dtype or PKV_FP8_E4M3
  float inv_k;          // 1.0f / k scale (E4M3 cache only)
  float inv_v;
};

enum DecodeMode : int32_t { kSinglePass = 0, kPartitioned = 1, kBalanced = 2 };

// Which kernels of a decode call to launch: the streaming kernel and its merge
// (or reduce) kernel, only the first, or only the second.
enum DecodePhase : int32_t { kBothPhases = 0, kSplitPhase = 1, kMergePhase = 2 };

// One decode call (partition or balanced kernel + optional reduce).
struct DecodeArgs {
  const void* q;
  void* out;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* seq_order;  // single pass / partitioned: sequence of grid row z, or null
  // split workspace.  Partitioned: [S][Hq][NP][D] and [S][Hq][NP][2].
  // Balanced: slot = worker + segment, [slots][G][D] and [slots][G][2], plus
  // per segment (sequence, KV head) the first and last worker of its partials.
  float* ws_acc;        // unnormalised partial outputs
  float* ws_ml;         // partial running max (log2 units) and sum
  int32_t* ws_meta;     // balanced only: [S * Hkv][2]
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;        // Hq / Hkv
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks;
  int32_t part_tiles;   // 16-token tiles per partition (single pass: covers max_blocks)
  int32_t num_parts;    // partitions per (sequence, KV head) = grid.x
  int32_t waves;        // wavefronts per workgroup
  int32_t mode;         // DecodeMode
  int32_t num_workers;  // balanced: wavefronts sharing the flattened tiles
  int32_t cache_dtype;
  float qk_scale;       // scale * log2(e) (* k scale for E4M3)
  float v_scale;        // 1, or the V scale for E4M3
  int32_t phase;        // DecodePhase
  // Shared prefix (balanced mode only): the first len_offset tokens of every
  // sequence are a prefix handled by the prefix kernel; the balanced kernel
  // walks only the tails (tables already advanced by len_offset / bs columns)
  // and, with cascade set, leaves every pair as pieces for the merge, which
  // also takes the prefix pieces: num_prefix_splits slots per pair from slot
  // prefix_slot0 + pair * num_prefix_splits.
  int32_t len_offset;
  int32_t cascade;
  int32_t stream_kv;    // pool tile reads carry the non-temporal hint
  int32_t num_prefix_splits;
  int64_t prefix_slot0;
  // Append (write folded into the decode): sequence s's new token, rows
  // [S][Hkv][D] of q's element type, goes to slots[s]; when that slot is
  // position len-1 of the sequence, the attention takes the row from kn/vn.
  int32_t append;
  const void* kn;
  const void* vn;
  const int32_t* slots;
  float inv_k;          // 1.0f / k scale (E4M3 cache only)
  float inv_v;
};

// Whole-block moves between pools and staging buffers: for each p < num_pairs,
// block src_ids[p * id_stride] of src becomes block dst_ids[p * id_stride] of
// dst, for the K and the V buffers.  A null id array means the identity (p).
// Negative ids skip the pair; with skip_same, src == dst skips it too (an
// in-place copy-on-write pair naming one block twice).
struct CopyArgs {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int32_t* src_ids;
  const int32_t* dst_ids;
  int32_t id_stride;
  int32_t skip_same;
  int64_t num_pairs;
  int64_t block_bytes;   // one block of one buffer
};

// One chunked-prefill call: the queries of sequence s are rows
// qstart[s] .. qstart[s+1]-1 of q, at the last positions of its context.
struct PrefillArgs {
  const void* q;        // [T][Hq][D]
  void* out;            // [T][Hq][D]
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* qstart;  // [S + 1]
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t head_dim;
  int32_t block_size;
  int32_t max_blocks;
  int32_t max_query_len;  // sizes the grid only; longer chunks are covered by a stride loop
  int32_t rows_per_wave;  // 16, 32 or 64 (query, head) rows per wavefront
  int32_t cache_dtype;
  int32_t workgroups;     // at most this many workgroups (one per compute unit)
  float qk_scale;         // scale * log2(e) (* k scale for E4M3)
  float v_scale;
};

// The shared-prefix part of a cascade decode: every sequence's queries
// against the prefix keys (one physical block list), split over keys.
struct PrefixArgs {
  const void* q;          // [S][Hq][D]
  const void* kc;
  const void* vc;
  const int32_t* blocks;  // the prefix's physical blocks, prefix_len / block_size of them
  float* ws_acc;          // partial states in the balanced merge's slot layout
  float* ws_ml;
  int64_t slot0;          // slot of (pair 0, split 0); pair p, split k -> slot0 + p * splits + k
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t head_dim;
  int32_t block_size;
  int32_t prefix_len;
  int32_t splits;         // key ranges per (pair): tiles k * T / splits .. (k + 1) * T / splits
  int32_t cache_dtype;
  float qk_scale;
};

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream);
hipError_t launch_shared_prefix(const PrefixArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_copy_blocks(const CopyArgs& a, hipStream_t stream);
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks,
                             hipStream_t stream);
hipError_t launch_gather_probe(const void* kc, const void* vc, const int32_t* rows, int64_t num_tiles,
                               int64_t num_rows, int32_t workers, int32_t mode, uint32_t* sink,
                               hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// The allocation-free decode's scratch: a fixed device array of kScratchBytes;
// its device address on the current GPU (looked up once per device).
constexpr size_t kScratchBytes = size_t(32) << 20;
hipError_t scratch_for_current_device(void** ptr);

}  // namespace pkv
