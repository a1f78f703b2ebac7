// extern "C" entry points of libpagedkv.so: descriptor validation, launch
// parameters and error reporting.  Declarations and contracts: include/pagedkv.h.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

int64_t elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    case PKV_I32: return 4;
    default: return 0;
  }
}

int64_t numel(const pkv_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

// rank, non-negative sizes, dense row-major strides, data present when non-empty
pkv_status check_tensor(const pkv_tensor* t, const char* name, int ndim) {
  if (!t) return fail(PKV_ERR_NULL, "%s: descriptor is NULL", name);
  if (t->ndim != ndim) return fail(PKV_ERR_SHAPE, "%s: expected %d dims, got %d", name, ndim, t->ndim);
  if (elem_bytes(t->dtype) == 0) return fail(PKV_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return fail(PKV_ERR_SHAPE, "%s: negative size in dim %d", name, i);
  // a tensor with no elements has no layout (frameworks report any strides
  // for one, zero included)
  if (numel(t) == 0) return PKV_OK;
  int64_t expect = 1;
  for (int i = ndim - 1; i >= 0; --i) {
    if (t->shape[i] > 1 && t->stride[i] != expect)
      return fail(PKV_ERR_LAYOUT, "%s: not dense row-major (dim %d stride %lld, expected %lld)",
                  name, i, (long long)t->stride[i], (long long)expect);
    expect *= t->shape[i];
  }
  if (!t->data) return fail(PKV_ERR_NULL, "%s: data pointer is NULL", name);
  return PKV_OK;
}

pkv_status check_align(const pkv_tensor* t, const char* name, uintptr_t align) {
  if (numel(t) > 0 && (reinterpret_cast<uintptr_t>(t->data) % align) != 0)
    return fail(PKV_ERR_LAYOUT, "%s: data must be %u-byte aligned", name, (unsigned)align);
  return PKV_OK;
}

bool overlap(const pkv_tensor* a, const pkv_tensor* b) {
  const int64_t na = numel(a) * elem_bytes(a->dtype), nb = numel(b) * elem_bytes(b->dtype);
  if (na == 0 || nb == 0) return false;
  const char* pa = static_cast<const char*>(a->data);
  const char* pb = static_cast<const char*>(b->data);
  return pa < pb + nb && pb < pa + na;
}

pkv_status check_scale(const pkv_tensor* t, const char* name) {
  if (t->dtype == PKV_FP8_E4M3 && !(std::isfinite(t->scale) && t->scale > 0.f))
    return fail(PKV_ERR_SHAPE, "%s: E4M3 scale must be finite and > 0 (got %g)", name,
                (double)t->scale);
  return PKV_OK;
}

#define PKV_TRY(expr)                \
  do {                               \
    pkv_status st_ = (expr);         \
    if (st_ != PKV_OK) return st_;   \
  } while (0)

int64_t num_partitions(int64_t max_blocks, int64_t block_size, int64_t partition_size) {
  if (partition_size <= 0) return 1;
  const int64_t tokens = max_blocks * block_size;
  const int64_t np = (tokens + partition_size - 1) / partition_size;
  return np < 1 ? 1 : np;
}

// Compute units of the current device (cached per device; 256 if unknown).
// Host threads may race to fill an entry; they store the same value.
int32_t device_cus() {
  static std::atomic<int32_t> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int32_t cus = cache[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus = n;
    cache[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// Default balanced worker count: 4 wavefronts per compute unit.
int32_t default_workers() { return 4 * device_cus(); }

// Launch plan derived from the options and sizes.
struct Plan {
  int32_t mode = PKV_DECODE_SINGLE_PASS;
  int64_t partitions = 1;   // PARTITIONED
  int64_t part_tiles = 1;
  int32_t waves = 4;
  int32_t workers = 0;      // BALANCED
  int32_t prefix_splits = 0;  // shared-prefix decode: key splits of the prefix per pair
  int64_t slots(int64_t S, int64_t Hkv) const {
    return workers + S * Hkv + S * Hkv * prefix_splits;
  }
  size_t workspace_floats(int64_t S, int64_t Hq, int64_t Hkv, int64_t D) const {
    if (mode == PKV_DECODE_PARTITIONED && partitions > 1) return (size_t)(S * Hq * partitions * (D + 2));
    if (mode == PKV_DECODE_BALANCED) return (size_t)(slots(S, Hkv) * (Hq / Hkv) * (D + 2));
    return 0;
  }
  size_t meta_bytes(int64_t S, int64_t Hkv) const {
    return mode == PKV_DECODE_BALANCED ? (size_t)(S * Hkv * 2 * 4) : 0;
  }
};

// Key splits of a shared prefix: about one (128-row workgroup, KV head, split)
// unit per compute unit, at least four tiles per split; more splits cost more
// in the merge than they save (256-sequence batch, whole call: 1 split
// 113.9 us, 2: 105.0, 3: 104.5, 4: 103.4, 6: 111.5).
int32_t prefix_splits(int64_t S, int64_t G, int64_t Hkv, int64_t prefix_len) {
  const int64_t tiles = prefix_len / 16;
  const int64_t row_groups = (S * G + 127) / 128;
  const int64_t want = (device_cus() + row_groups * Hkv - 1) / (row_groups * Hkv);
  const int64_t cap = tiles / 4 > 1 ? tiles / 4 : 1;
  return (int32_t)(want < 1 ? 1 : want > cap ? cap : want);
}

pkv_status plan(const pkv_decode_opts* opts, int64_t S, int64_t Hq, int64_t Hkv, int64_t maxb,
                int64_t bs, Plan* p, int64_t prefix_len = 0) {
  int32_t mode = opts ? opts->mode : PKV_DECODE_SINGLE_PASS;
  int32_t waves = opts ? opts->waves_per_group : 0;
  int32_t auto_workers = 0;
  if (prefix_len > 0) {
    // the tails run the balanced split (cascade pieces need its merge)
    if (mode != PKV_DECODE_AUTO && mode != PKV_DECODE_BALANCED && opts)
      return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode runs the balanced split: mode must "
                                       "be AUTO or BALANCED");
    // 4 workers per CU: the 256-sequence batch's tails take 106 us at 4,
    // 110 at 8 (118 at 3, 134 at 5: counts that leave CUs unevenly loaded lose)
    auto_workers = 4 * device_cus();
    mode = PKV_DECODE_BALANCED;
    p->prefix_splits = prefix_splits(S, Hq / Hkv, Hkv, prefix_len);
  } else if (mode == PKV_DECODE_AUTO) {
    // measured on MI355X: many short (sequence, KV head) pairs stream best one
    // workgroup each, with 4 wavefronts (512-2,048 sequences of 32 / 8 heads,
    // bf16 and E4M3: 1-10% faster than 8); few or long ones need the balanced split
    const int64_t pairs = S * Hkv, cus = device_cus();
    if (pairs >= 16 * cus) {
      mode = PKV_DECODE_SINGLE_PASS;
      if (waves == 0) waves = 4;
    } else {
      mode = PKV_DECODE_BALANCED;
      auto_workers = (int32_t)((pairs >= 8 * cus ? 8 : 4) * cus);
    }
  }
  p->mode = mode;
  // split-K partitions of up to 32 tiles stream best one wavefront each (8 x
  // 131,072 tokens by 512: 385 us with 1, 394 with 2, 400 with 4, 436 with 8)
  if (waves == 0 && mode == PKV_DECODE_PARTITIONED && opts && opts->partition_size > 0 &&
      opts->partition_size <= 512)
    waves = 1;
  p->waves = waves == 0 ? 4 : waves;
  if (p->waves != 1 && p->waves != 2 && p->waves != 4 && p->waves != 8)
    return fail(PKV_ERR_UNSUPPORTED, "waves_per_group %d: must be 0, 1, 2, 4 or 8", waves);
  const int64_t max_tiles = (maxb * bs + 15) / 16;
  switch (mode) {
    case PKV_DECODE_SINGLE_PASS:
      p->partitions = 1;
      p->part_tiles = max_tiles > 0 ? max_tiles : 1;
      return PKV_OK;
    case PKV_DECODE_PARTITIONED: {
      const int32_t part = opts->partition_size;
      if (part <= 0 || part % 16 != 0)
        return fail(PKV_ERR_UNSUPPORTED, "partition_size %d: must be a positive multiple of 16", part);
      p->partitions = num_partitions(maxb, bs, part);
      if (p->partitions > 65535 * 16384LL)
        return fail(PKV_ERR_UNSUPPORTED, "too many partitions");
      p->part_tiles = p->partitions > 1 ? part / 16 : (max_tiles > 0 ? max_tiles : 1);
      // one-wavefront partitions run on persistent wavefronts, by default 4
      // per CU, each streaming a run of them (8 x 131,072 tokens by 512:
      // 335 us per launch, against 385 us with a workgroup per partition)
      if (p->waves == 1) {
        const int32_t wk = opts->num_workers;
        if (wk < 0 || wk > (1 << 24))
          return fail(PKV_ERR_UNSUPPORTED, "num_workers %d: must be in [0, 2^24]", wk);
        p->workers = wk != 0 ? wk : default_workers();
      }
      return PKV_OK;
    }
    case PKV_DECODE_BALANCED: {
      const int32_t wk = opts ? opts->num_workers : 0;
      if (wk < 0 || wk > (1 << 24))
        return fail(PKV_ERR_UNSUPPORTED, "num_workers %d: must be in [0, 2^24]", wk);
      p->workers = wk != 0 ? wk : auto_workers != 0 ? auto_workers : default_workers();
      if (S * Hkv > INT32_MAX / 2) return fail(PKV_ERR_UNSUPPORTED, "too many (sequence, KV head) pairs");
      if (p->slots(S, Hkv) > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "too many partial slots");
      return PKV_OK;
    }
    default:
      return fail(PKV_ERR_UNSUPPORTED, "unknown decode mode %d", mode);
  }
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_last_error(void) { return g_last_error.c_str(); }

pkv_status paged_kv_write(const pkv_tensor* k, const pkv_tensor* v, const pkv_tensor* slot_mapping,
                          pkv_tensor* key_cache, pkv_tensor* value_cache, void* hip_stream) {
  PKV_TRY(check_tensor(k, "k", 3));
  PKV_TRY(check_tensor(v, "v", 3));
  PKV_TRY(check_tensor(slot_mapping, "slot_mapping", 1));
  PKV_TRY(check_tensor(key_cache, "key_cache", 4));
  PKV_TRY(check_tensor(value_cache, "value_cache", 4));
  if (k->dtype != PKV_F32 && k->dtype != PKV_BF16)
    return fail(PKV_ERR_DTYPE, "k: must be f32 or bf16");
  if (v->dtype != k->dtype) return fail(PKV_ERR_DTYPE, "v: dtype differs from k");
  if (slot_mapping->dtype != PKV_I32) return fail(PKV_ERR_DTYPE, "slot_mapping: must be int32");
  if (value_cache->dtype != key_cache->dtype)
    return fail(PKV_ERR_DTYPE, "value_cache: dtype differs from key_cache");
  if (key_cache->dtype != k->dtype && key_cache->dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_DTYPE, "key_cache: must match k's dtype or be E4M3");
  for (int i = 0; i < 3; ++i)
    if (v->shape[i] != k->shape[i]) return fail(PKV_ERR_SHAPE, "v: shape differs from k");
  for (int i = 0; i < 4; ++i)
    if (value_cache->shape[i] != key_cache->shape[i])
      return fail(PKV_ERR_SHAPE, "value_cache: shape differs from key_cache");
  const int64_t T = k->shape[0], H = k->shape[1], D = k->shape[2];
  const int64_t NB = key_cache->shape[0], bs = key_cache->shape[2];
  if (slot_mapping->shape[0] != T) return fail(PKV_ERR_SHAPE, "slot_mapping: expected [%lld]", (long long)T);
  if (key_cache->shape[1] != H || key_cache->shape[3] != D)
    return fail(PKV_ERR_SHAPE, "key_cache: heads/head_dim differ from k");
  if (D <= 0 || D % 8 != 0 || D > 1024)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %lld: must be a positive multiple of 8, <= 1024", (long long)D);
  if (bs <= 0 || H <= 0 || H > 1024)
    return fail(PKV_ERR_SHAPE, "block_size and num_kv_heads must be positive (heads <= 1024)");
  if (NB * bs > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "pool has more than 2^31-1 slots");
  PKV_TRY(check_scale(key_cache, "key_cache"));
  PKV_TRY(check_scale(value_cache, "value_cache"));
  PKV_TRY(check_align(k, "k", 16));
  PKV_TRY(check_align(v, "v", 16));
  PKV_TRY(check_align(key_cache, "key_cache", 16));
  PKV_TRY(check_align(value_cache, "value_cache", 16));
  if (overlap(key_cache, value_cache)) return fail(PKV_ERR_LAYOUT, "key_cache and value_cache overlap");
  const pkv_tensor* inputs[] = {k, v, slot_mapping};
  for (const pkv_tensor* in : inputs)
    if (overlap(in, key_cache) || overlap(in, value_cache))
      return fail(PKV_ERR_LAYOUT, "an input overlaps a cache");
  if (T == 0) return ok();

  pkv::WriteArgs a{};
  a.k = k->data;
  a.v = v->data;
  a.slots = static_cast<const int32_t*>(slot_mapping->data);
  a.kc = key_cache->data;
  a.vc = value_cache->data;
  a.num_tokens = T;
  a.num_heads = (int32_t)H;
  a.head_dim = (int32_t)D;
  a.block_size = (int32_t)bs;
  a.in_dtype = k->dtype;
  a.cache_dtype = key_cache->dtype;
  a.inv_k = key_cache->dtype == PKV_FP8_E4M3 ? 1.0f / key_cache->scale : 1.0f;
  a.inv_v = value_cache->dtype == PKV_FP8_E4M3 ? 1.0f / value_cache->scale : 1.0f;
  const hipError_t e = pkv::launch_kv_write(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "paged_kv_write launch: %s", hipGetErrorString(e));
  return ok();
}

size_t paged_attention_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                            int32_t num_kv_heads, int32_t head_dim,
                                                            int32_t max_blocks_per_seq,
                                                            int32_t block_size, int32_t prefix_len,
                                                            const pkv_decode_opts* opts) {
  if (num_seqs < 0 || num_q_heads < 0 || num_kv_heads <= 0 || head_dim < 0 ||
      max_blocks_per_seq < 0 || block_size <= 0 || num_q_heads % num_kv_heads != 0 ||
      prefix_len <= 0 || prefix_len % block_size != 0)
    return 0;
  Plan p;
  if (plan(opts, num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq, block_size, &p,
           prefix_len) != PKV_OK)
    return 0;
  return p.workspace_floats(num_seqs, num_q_heads, num_kv_heads, head_dim) * 4u + p.meta_bytes(num_seqs, num_kv_heads);
}

pkv_status paged_attention_prefill(pkv_tensor* out, const pkv_tensor* q,
                                   const pkv_tensor* key_cache, const pkv_tensor* value_cache,
                                   const pkv_tensor* block_tables, const pkv_tensor* context_lens,
                                   const pkv_tensor* query_start_loc, int32_t max_query_len,
                                   float scale, int32_t block_size, const pkv_prefill_opts* opts,
                                   void* hip_stream) {
  PKV_TRY(check_tensor(out, "out", 3));
  PKV_TRY(check_tensor(q, "q", 3));
  PKV_TRY(check_tensor(key_cache, "key_cache", 4));
  PKV_TRY(check_tensor(value_cache, "value_cache", 4));
  PKV_TRY(check_tensor(block_tables, "block_tables", 2));
  PKV_TRY(check_tensor(context_lens, "context_lens", 1));
  PKV_TRY(check_tensor(query_start_loc, "query_start_loc", 1));
  if (q->dtype != PKV_F32 && q->dtype != PKV_BF16) return fail(PKV_ERR_DTYPE, "q: must be f32 or bf16");
  if (out->dtype != q->dtype) return fail(PKV_ERR_DTYPE, "out: dtype differs from q");
  if (value_cache->dtype != key_cache->dtype)
    return fail(PKV_ERR_DTYPE, "value_cache: dtype differs from key_cache");
  const int32_t ct = key_cache->dtype;
  if (!((ct == PKV_F32 && q->dtype == PKV_F32) || (ct == PKV_BF16 && q->dtype == PKV_BF16) ||
        (ct == PKV_FP8_E4M3 && q->dtype == PKV_BF16)))
    return fail(PKV_ERR_DTYPE, "cache/q dtypes: supported are f32/f32, bf16/bf16, e4m3/bf16");
  if (block_tables->dtype != PKV_I32 || context_lens->dtype != PKV_I32 ||
      query_start_loc->dtype != PKV_I32)
    return fail(PKV_ERR_DTYPE, "block_tables, context_lens and query_start_loc must be int32");
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i]) return fail(PKV_ERR_SHAPE, "out: shape differs from q");
  for (int i = 0; i < 4; ++i)
    if (value_cache->shape[i] != key_cache->shape[i])
      return fail(PKV_ERR_SHAPE, "value_cache: shape differs from key_cache");
  const int64_t T = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  const int64_t S = context_lens->shape[0];
  const int64_t Hkv = key_cache->shape[1], bs = key_cache->shape[2];
  const int64_t maxb = block_tables->shape[1];
  if (key_cache->shape[3] != D) return fail(PKV_ERR_SHAPE, "key_cache: head_dim differs from q");
  if (block_tables->shape[0] != S || query_start_loc->shape[0] != S + 1)
    return fail(PKV_ERR_SHAPE, "block_tables must be [S, max_blocks] and query_start_loc [S + 1]");
  if (bs != block_size) return fail(PKV_ERR_SHAPE, "block_size %d != key_cache.shape[2] %lld",
                                    block_size, (long long)bs);
  if (bs < 16 || bs > 256 || bs % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %lld: must be a multiple of 16 in [16, 256]", (long long)bs);
  if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %lld: must be 64 or 128", (long long)D);
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0)
    return fail(PKV_ERR_SHAPE, "num_q_heads %lld must be a positive multiple of num_kv_heads %lld",
                (long long)Hq, (long long)Hkv);
  if (S > 65535 || Hkv > 65535) return fail(PKV_ERR_UNSUPPORTED, "more than 65535 sequences or KV heads");
  if (S > 0 && maxb <= 0) return fail(PKV_ERR_SHAPE, "block_tables: needs at least one column");
  if (maxb * bs > INT32_MAX / 2) return fail(PKV_ERR_UNSUPPORTED, "max_blocks * block_size too large");
  if (T > INT32_MAX / 2 || T * (Hq / Hkv) > INT32_MAX / 2)
    return fail(PKV_ERR_UNSUPPORTED, "too many query rows");
  if (max_query_len < 0 || max_query_len > T)
    return fail(PKV_ERR_SHAPE, "max_query_len %d outside [0, %lld]", max_query_len, (long long)T);
  // default: 32 rows per wavefront; f32 fragments are twice as large, so 16
  const int32_t rpw = opts && opts->rows_per_wave ? opts->rows_per_wave : ct == PKV_F32 ? 16 : 32;
  if (rpw != 16 && rpw != 32 && (rpw != 64 || ct == PKV_F32 || D != 64))
    return fail(PKV_ERR_UNSUPPORTED,
                "rows_per_wave %d: must be 0, 16, 32, or 64 with head_dim 64 (not f32)", rpw);
  PKV_TRY(check_scale(key_cache, "key_cache"));
  PKV_TRY(check_scale(value_cache, "value_cache"));
  PKV_TRY(check_align(out, "out", 16));
  PKV_TRY(check_align(q, "q", 16));
  PKV_TRY(check_align(key_cache, "key_cache", 16));
  PKV_TRY(check_align(value_cache, "value_cache", 16));
  const pkv_tensor* inputs[] = {q, key_cache, value_cache, block_tables, context_lens, query_start_loc};
  for (const pkv_tensor* t : inputs)
    if (overlap(out, t)) return fail(PKV_ERR_LAYOUT, "out overlaps an input");
  if (S == 0 || T == 0) return ok();

  pkv::PrefillArgs a{};
  a.q = q->data;
  a.out = out->data;
  a.kc = key_cache->data;
  a.vc = value_cache->data;
  a.tables = static_cast<const int32_t*>(block_tables->data);
  a.lens = static_cast<const int32_t*>(context_lens->data);
  a.qstart = static_cast<const int32_t*>(query_start_loc->data);
  a.num_seqs = (int32_t)S;
  a.num_q_heads = (int32_t)Hq;
  a.num_kv_heads = (int32_t)Hkv;
  a.group = (int32_t)(Hq / Hkv);
  a.head_dim = (int32_t)D;
  a.block_size = (int32_t)bs;
  a.max_blocks = (int32_t)maxb;
  a.max_query_len = max_query_len;
  a.rows_per_wave = rpw;
  a.cache_dtype = ct;
  a.workgroups = device_cus();
  const double log2e = 1.4426950408889634;
  const double kscale = ct == PKV_FP8_E4M3 ? (double)key_cache->scale : 1.0;
  a.qk_scale = (float)((double)scale * log2e * kscale);
  a.v_scale = ct == PKV_FP8_E4M3 ? value_cache->scale : 1.0f;
  const hipError_t e = pkv::launch_prefill(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "paged_attention_prefill launch: %s", hipGetErrorString(e));
  return ok();
}

pkv_status paged_kv_copy_blocks(pkv_tensor* key_cache, pkv_tensor* value_cache,
                                const pkv_tensor* block_pairs, void* hip_stream) {
  PKV_TRY(check_tensor(key_cache, "key_cache", 4));
  PKV_TRY(check_tensor(value_cache, "value_cache", 4));
  PKV_TRY(check_tensor(block_pairs, "block_pairs", 2));
  if (value_cache->dtype != key_cache->dtype)
    return fail(PKV_ERR_DTYPE, "value_cache: dtype differs from key_cache");
  if (key_cache->dtype != PKV_F32 && key_cache->dtype != PKV_BF16 && key_cache->dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_DTYPE, "key_cache: must be f32, bf16 or E4M3");
  if (block_pairs->dtype != PKV_I32) return fail(PKV_ERR_DTYPE, "block_pairs: must be int32");
  for (int i = 0; i < 4; ++i)
    if (value_cache->shape[i] != key_cache->shape[i])
      return fail(PKV_ERR_SHAPE, "value_cache: shape differs from key_cache");
  if (block_pairs->shape[1] != 2) return fail(PKV_ERR_SHAPE, "block_pairs: expected [P, 2]");
  const int64_t P = block_pairs->shape[0];
  const int64_t block_bytes = key_cache->shape[1] * key_cache->shape[2] * key_cache->shape[3] *
                              elem_bytes(key_cache->dtype);
  if (block_bytes % 16 != 0)
    return fail(PKV_ERR_LAYOUT, "one block must be a multiple of 16 bytes (got %lld)", (long long)block_bytes);
  if (P > INT32_MAX / 2) return fail(PKV_ERR_SHAPE, "too many pairs");
  PKV_TRY(check_align(key_cache, "key_cache", 16));
  PKV_TRY(check_align(value_cache, "value_cache", 16));
  PKV_TRY(check_align(block_pairs, "block_pairs", 4));
  if (overlap(key_cache, value_cache)) return fail(PKV_ERR_LAYOUT, "key_cache and value_cache overlap");
  if (overlap(block_pairs, key_cache) || overlap(block_pairs, value_cache))
    return fail(PKV_ERR_LAYOUT, "block_pairs overlaps a cache");
  if (P == 0) return ok();
  pkv::CopyArgs a{};
  a.src_k = key_cache->data;
  a.src_v = value_cache->data;
  a.dst_k = key_cache->data;
  a.dst_v = value_cache->data;
  a.src_ids = static_cast<const int32_t*>(block_pairs->data);
  a.dst_ids = a.src_ids + 1;
  a.id_stride = 2;
  a.skip_same = 1;
  a.num_pairs = P;
  a.block_bytes = block_bytes;
  const hipError_t e = pkv::launch_copy_blocks(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "paged_kv_copy_blocks launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"

namespace {

// Device memory of the current process (not host memory, pinned or not):
// the kernels dereference every pointer they are given.
bool device_memory(const void* p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // an unknown pointer: clear the query's error
    return false;
  }
  return at.type == hipMemoryTypeDevice;
}

// Shared checks of a gather (pools -> staging) or scatter (staging -> pools).
pkv_status block_move(const char* fn, const pkv_tensor* pool_k, const pkv_tensor* pool_v,
                      const pkv_tensor* stage_k, const pkv_tensor* stage_v,
                      const pkv_tensor* block_ids, bool gather, void* hip_stream) {
  PKV_TRY(check_tensor(pool_k, "key_cache", 4));
  PKV_TRY(check_tensor(pool_v, "value_cache", 4));
  PKV_TRY(check_tensor(stage_k, gather ? "out_k" : "in_k", 4));
  PKV_TRY(check_tensor(stage_v, gather ? "out_v" : "in_v", 4));
  PKV_TRY(check_tensor(block_ids, "block_ids", 1));
  if (block_ids->dtype != PKV_I32) return fail(PKV_ERR_DTYPE, "block_ids: must be int32");
  const pkv_tensor* all[] = {pool_v, stage_k, stage_v};
  for (const pkv_tensor* t : all)
    if (t->dtype != pool_k->dtype) return fail(PKV_ERR_DTYPE, "pools and staging buffers differ in dtype");
  if (pool_k->dtype != PKV_F32 && pool_k->dtype != PKV_BF16 && pool_k->dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_DTYPE, "key_cache: must be f32, bf16 or E4M3");
  const int64_t n = block_ids->shape[0];
  for (int i = 0; i < 4; ++i) {
    if (pool_v->shape[i] != pool_k->shape[i]) return fail(PKV_ERR_SHAPE, "value_cache: shape differs from key_cache");
    if (i > 0 && (stage_k->shape[i] != pool_k->shape[i] || stage_v->shape[i] != pool_k->shape[i]))
      return fail(PKV_ERR_SHAPE, "staging buffers must be [n, Hkv, bs, D] like the pools");
  }
  if (stage_k->shape[0] != n || stage_v->shape[0] != n)
    return fail(PKV_ERR_SHAPE, "staging buffers must hold one block per id (%lld)", (long long)n);
  const int64_t bb = pool_k->shape[1] * pool_k->shape[2] * pool_k->shape[3] * elem_bytes(pool_k->dtype);
  if (bb % 16 != 0) return fail(PKV_ERR_LAYOUT, "one block must be a multiple of 16 bytes");
  if (n > INT32_MAX / 2) return fail(PKV_ERR_SHAPE, "too many blocks");
  const pkv_tensor* bufs[] = {pool_k, pool_v, stage_k, stage_v};
  for (const pkv_tensor* t : bufs) PKV_TRY(check_align(t, "buffer", 16));
  PKV_TRY(check_align(block_ids, "block_ids", 4));
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlap(bufs[i], bufs[j])) return fail(PKV_ERR_LAYOUT, "pools and staging buffers overlap");
  for (const pkv_tensor* t : bufs)
    if (overlap(block_ids, t)) return fail(PKV_ERR_LAYOUT, "block_ids overlaps a buffer");
  if (n == 0) return ok();
  for (const pkv_tensor* t : bufs)
    if (!device_memory(t->data))
      return fail(PKV_ERR_LAYOUT, "%s: pools and staging buffers must be device memory", fn);
  pkv::CopyArgs a{};
  a.src_k = gather ? pool_k->data : stage_k->data;
  a.src_v = gather ? pool_v->data : stage_v->data;
  a.dst_k = gather ? stage_k->data : pool_k->data;
  a.dst_v = gather ? stage_v->data : pool_v->data;
  a.src_ids = gather ? static_cast<const int32_t*>(block_ids->data) : nullptr;
  a.dst_ids = gather ? nullptr : static_cast<const int32_t*>(block_ids->data);
  a.id_stride = 1;
  a.skip_same = 0;
  a.num_pairs = n;
  a.block_bytes = bb;
  const hipError_t e = pkv::launch_copy_blocks(a, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

pkv_status paged_kv_gather_blocks(const pkv_tensor* key_cache, const pkv_tensor* value_cache,
                                  const pkv_tensor* block_ids, pkv_tensor* out_k,
                                  pkv_tensor* out_v, void* hip_stream) {
  return block_move("paged_kv_gather_blocks", key_cache, value_cache, out_k, out_v, block_ids,
                    true, hip_stream);
}

pkv_status paged_kv_scatter_blocks(const pkv_tensor* in_k, const pkv_tensor* in_v,
                                   const pkv_tensor* block_ids, pkv_tensor* key_cache,
                                   pkv_tensor* value_cache, void* hip_stream) {
  return block_move("paged_kv_scatter_blocks", key_cache, value_cache, in_k, in_v, block_ids,
                    false, hip_stream);
}

int32_t pkv_read_probe_blocks(void) { return 4 * device_cus(); }

pkv_status pkv_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* hip_stream) {
  if (bytes == 0) return ok();  // nothing to read, nothing launched
  if (!buf || !sink) return fail(PKV_ERR_NULL, "pkv_read_probe: null buffer");
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(PKV_ERR_SHAPE, "pkv_read_probe: buf must be 16-byte aligned and bytes a multiple of 16");
  if (!device_memory(buf) || !device_memory(sink))
    return fail(PKV_ERR_LAYOUT, "pkv_read_probe: buf and sink must be device memory");
  const hipError_t e = pkv::launch_read_probe(buf, (int64_t)bytes, sink, pkv_read_probe_blocks(),
                                              static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_read_probe: %s", hipGetErrorString(e));
  return ok();
}

pkv_status pkv_tile_gather_probe(const void* key_cache, const void* value_cache,
                                 const int32_t* tile_rows, int64_t num_tiles, int64_t num_rows,
                                 int32_t workers, int32_t mode, uint32_t* sink, void* hip_stream) {
  if (num_tiles <= 0) return ok();  // nothing to read, nothing launched
  if (!key_cache || !value_cache || !tile_rows || !sink)
    return fail(PKV_ERR_NULL, "pkv_tile_gather_probe: null pointer");
  if (workers < 1 || workers > (1 << 20) || (mode != 0 && mode != 1))
    return fail(PKV_ERR_UNSUPPORTED, "pkv_tile_gather_probe: workers %d, mode %d", workers, mode);
  if (reinterpret_cast<uintptr_t>(key_cache) % 16 != 0 || reinterpret_cast<uintptr_t>(value_cache) % 16 != 0 ||
      num_rows < 16)
    return fail(PKV_ERR_SHAPE, "pkv_tile_gather_probe: pools must be 16-byte aligned with >= 16 rows");
  if (!device_memory(key_cache) || !device_memory(value_cache) || !device_memory(tile_rows) ||
      !device_memory(sink))
    return fail(PKV_ERR_LAYOUT, "pkv_tile_gather_probe: pointers must be device memory");
  const hipError_t e = pkv::launch_gather_probe(key_cache, value_cache, tile_rows, num_tiles, num_rows,
                                                workers, mode, sink, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_tile_gather_probe: %s", hipGetErrorString(e));
  return ok();
}

size_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              int32_t max_blocks_per_seq, int32_t block_size,
                                              const pkv_decode_opts* opts) {
  if (num_seqs <= 0 || num_q_heads < 0 || num_kv_heads <= 0 || head_dim < 0 ||
      max_blocks_per_seq < 0 || block_size < 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  Plan p;
  if (plan(opts, num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq, block_size, &p) != PKV_OK)
    return 0;
  return p.workspace_floats(num_seqs, num_q_heads, num_kv_heads, head_dim) * 4u + p.meta_bytes(num_seqs, num_kv_heads);
}

}  // extern "C"

namespace {

// The new tokens of an append call: one per sequence.
struct AppendIn {
  const pkv_tensor* k;
  const pkv_tensor* v;
  const pkv_tensor* slots;
};

pkv_status decode_impl(const char* fn, pkv_tensor* out, const pkv_tensor* q,
                       const pkv_tensor* key_cache, const pkv_tensor* value_cache,
                       const pkv_tensor* block_tables, const pkv_tensor* context_lens, float scale,
                       int32_t block_size, const pkv_decode_opts* opts, const AppendIn* app,
                       int32_t phase, void* hip_stream, int32_t prefix_len = 0) {
  PKV_TRY(check_tensor(out, "out", 3));
  PKV_TRY(check_tensor(q, "q", 3));
  PKV_TRY(check_tensor(key_cache, "key_cache", 4));
  PKV_TRY(check_tensor(value_cache, "value_cache", 4));
  PKV_TRY(check_tensor(block_tables, "block_tables", 2));
  PKV_TRY(check_tensor(context_lens, "context_lens", 1));
  if (q->dtype != PKV_F32 && q->dtype != PKV_BF16) return fail(PKV_ERR_DTYPE, "q: must be f32 or bf16");
  if (out->dtype != q->dtype) return fail(PKV_ERR_DTYPE, "out: dtype differs from q");
  if (value_cache->dtype != key_cache->dtype)
    return fail(PKV_ERR_DTYPE, "value_cache: dtype differs from key_cache");
  const int32_t ct = key_cache->dtype;
  if (!((ct == PKV_F32 && q->dtype == PKV_F32) || (ct == PKV_BF16 && q->dtype == PKV_BF16) ||
        (ct == PKV_FP8_E4M3 && q->dtype == PKV_BF16)))
    return fail(PKV_ERR_DTYPE, "cache/q dtypes: supported are f32/f32, bf16/bf16, e4m3/bf16");
  if (block_tables->dtype != PKV_I32 || context_lens->dtype != PKV_I32)
    return fail(PKV_ERR_DTYPE, "block_tables and context_lens must be int32");
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != q->shape[i]) return fail(PKV_ERR_SHAPE, "out: shape differs from q");
  for (int i = 0; i < 4; ++i)
    if (value_cache->shape[i] != key_cache->shape[i])
      return fail(PKV_ERR_SHAPE, "value_cache: shape differs from key_cache");
  const int64_t S = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  const int64_t Hkv = key_cache->shape[1], bs = key_cache->shape[2];
  const int64_t maxb = block_tables->shape[1];
  if (key_cache->shape[3] != D) return fail(PKV_ERR_SHAPE, "key_cache: head_dim differs from q");
  if (block_tables->shape[0] != S || context_lens->shape[0] != S)
    return fail(PKV_ERR_SHAPE, "block_tables/context_lens: leading dim must be num_seqs");
  if (bs != block_size) return fail(PKV_ERR_SHAPE, "block_size %d != key_cache.shape[2] %lld",
                                    block_size, (long long)bs);
  if (bs < 16 || bs > 256 || bs % 16 != 0)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %lld: must be a multiple of 16 in [16, 256]", (long long)bs);
  if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %lld: must be 64 or 128", (long long)D);
  if (Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0)
    return fail(PKV_ERR_SHAPE, "num_q_heads %lld must be a positive multiple of num_kv_heads %lld",
                (long long)Hq, (long long)Hkv);
  if (Hq / Hkv > 16) return fail(PKV_ERR_UNSUPPORTED, "group size %lld > 16", (long long)(Hq / Hkv));
  if (S > 65535 || Hkv > 65535) return fail(PKV_ERR_UNSUPPORTED, "more than 65535 sequences or KV heads");
  if (S > 0 && maxb <= 0) return fail(PKV_ERR_SHAPE, "block_tables: needs at least one column");
  if (maxb * bs > INT32_MAX / 2) return fail(PKV_ERR_UNSUPPORTED, "max_blocks * block_size too large");
  PKV_TRY(check_scale(key_cache, "key_cache"));
  PKV_TRY(check_scale(value_cache, "value_cache"));
  PKV_TRY(check_align(out, "out", 16));
  PKV_TRY(check_align(q, "q", 16));
  PKV_TRY(check_align(key_cache, "key_cache", 16));
  PKV_TRY(check_align(value_cache, "value_cache", 16));
  PKV_TRY(check_align(block_tables, "block_tables", 4));
  PKV_TRY(check_align(context_lens, "context_lens", 4));
  const pkv_tensor* inputs[] = {q, key_cache, value_cache, block_tables, context_lens};
  for (const pkv_tensor* t : inputs)
    if (overlap(out, t)) return fail(PKV_ERR_LAYOUT, "out overlaps an input");
  if (app) {
    PKV_TRY(check_tensor(app->k, "k", 3));
    PKV_TRY(check_tensor(app->v, "v", 3));
    PKV_TRY(check_tensor(app->slots, "slot_mapping", 1));
    if (app->k->dtype != q->dtype || app->v->dtype != q->dtype)
      return fail(PKV_ERR_DTYPE, "k, v: must have q's dtype");
    if (app->slots->dtype != PKV_I32) return fail(PKV_ERR_DTYPE, "slot_mapping: must be int32");
    for (const pkv_tensor* t : {app->k, app->v})
      if (t->shape[0] != S || t->shape[1] != Hkv || t->shape[2] != D)
        return fail(PKV_ERR_SHAPE, "k, v: expected [num_seqs, num_kv_heads, head_dim] = [%lld, %lld, %lld]",
                    (long long)S, (long long)Hkv, (long long)D);
    if (app->slots->shape[0] != S) return fail(PKV_ERR_SHAPE, "slot_mapping: expected [num_seqs]");
    if (key_cache->shape[0] * bs > INT32_MAX)
      return fail(PKV_ERR_UNSUPPORTED, "pool has more than 2^31-1 slots");
    PKV_TRY(check_align(app->k, "k", 16));
    PKV_TRY(check_align(app->v, "v", 16));
    PKV_TRY(check_align(app->slots, "slot_mapping", 4));
    const pkv_tensor* news[] = {app->k, app->v, app->slots};
    for (const pkv_tensor* t : news)
      if (overlap(t, key_cache) || overlap(t, value_cache) || overlap(t, out))
        return fail(PKV_ERR_LAYOUT, "k, v or slot_mapping overlaps a cache or out");
    if (overlap(key_cache, value_cache)) return fail(PKV_ERR_LAYOUT, "key_cache and value_cache overlap");
  }

  if (prefix_len < 0 || prefix_len % bs != 0 || prefix_len > maxb * bs)
    return fail(PKV_ERR_SHAPE, "prefix_len %d: must be a multiple of block_size in [0, %lld]",
                prefix_len, (long long)(maxb * bs));

  if (opts && (opts->flags & ~(PKV_DECODE_DEFER_MERGE | PKV_DECODE_STREAM_KV)) != 0)
    return fail(PKV_ERR_UNSUPPORTED, "opts->flags 0x%x: unknown PKV_DECODE_* bits", (unsigned)opts->flags);
  if (opts && reinterpret_cast<uintptr_t>(opts->seq_order) % 4 != 0)
    return fail(PKV_ERR_LAYOUT, "opts->seq_order must be 4-byte aligned");
  Plan p;
  PKV_TRY(plan(opts, S, Hq, Hkv, maxb, bs, &p, prefix_len));
  if (S == 0) return ok();  // nothing to compute, so no workspace either
  pkv::DecodeArgs a{};
  const size_t need = p.workspace_floats(S, Hq, Hkv, D) * 4u + p.meta_bytes(S, Hkv);
  if (need > 0) {
    if (!opts || !opts->workspace || opts->workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "this decode mode needs a workspace of %zu bytes (got %zu)", need,
                  opts && opts->workspace ? opts->workspace_bytes : (size_t)0);
    if (reinterpret_cast<uintptr_t>(opts->workspace) % 16 != 0)
      return fail(PKV_ERR_WORKSPACE, "workspace must be 16-byte aligned");
    a.ws_acc = static_cast<float*>(opts->workspace);
    if (p.mode == PKV_DECODE_BALANCED) {
      const size_t slots = (size_t)p.slots(S, Hkv);
      a.ws_ml = a.ws_acc + slots * (Hq / Hkv) * D;
      a.ws_meta = reinterpret_cast<int32_t*>(a.ws_ml + slots * (Hq / Hkv) * 2);
    } else {
      a.ws_ml = a.ws_acc + (size_t)S * Hq * p.partitions * D;
    }
  }

  a.q = q->data;
  a.out = out->data;
  a.kc = key_cache->data;
  a.vc = value_cache->data;
  a.tables = static_cast<const int32_t*>(block_tables->data);
  a.lens = static_cast<const int32_t*>(context_lens->data);
  // the start order only concerns the grid of the single pass / partitioned kernel
  if (opts && opts->seq_order && prefix_len == 0 && p.mode != PKV_DECODE_BALANCED)
    a.seq_order = opts->seq_order;
  a.num_seqs = (int32_t)S;
  a.num_q_heads = (int32_t)Hq;
  a.num_kv_heads = (int32_t)Hkv;
  a.group = (int32_t)(Hq / Hkv);
  a.head_dim = (int32_t)D;
  a.block_size = (int32_t)bs;
  a.max_blocks = (int32_t)maxb;
  a.part_tiles = (int32_t)p.part_tiles;
  a.num_parts = (int32_t)p.partitions;
  a.waves = p.waves;
  a.mode = p.mode == PKV_DECODE_BALANCED ? pkv::kBalanced
           : p.mode == PKV_DECODE_PARTITIONED ? pkv::kPartitioned : pkv::kSinglePass;
  a.num_workers = p.workers;
  a.cache_dtype = ct;
  const double log2e = 1.4426950408889634;
  const double kscale = ct == PKV_FP8_E4M3 ? (double)key_cache->scale : 1.0;
  a.qk_scale = (float)((double)scale * log2e * kscale);
  a.v_scale = ct == PKV_FP8_E4M3 ? value_cache->scale : 1.0f;
  a.phase = phase;
  a.stream_kv = opts && (opts->flags & PKV_DECODE_STREAM_KV) ? 1 : 0;
  if (app) {
    a.append = 1;
    a.kn = app->k->data;
    a.vn = app->v->data;
    a.slots = static_cast<const int32_t*>(app->slots->data);
    a.inv_k = ct == PKV_FP8_E4M3 ? 1.0f / key_cache->scale : 1.0f;
    a.inv_v = ct == PKV_FP8_E4M3 ? 1.0f / value_cache->scale : 1.0f;
  }
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  if (prefix_len > 0) {
    // cascade: prefix pieces from the prefix kernel, tail pieces from the
    // balanced split over the tables past the prefix, merged together
    a.len_offset = prefix_len;
    a.cascade = 1;
    a.num_prefix_splits = p.prefix_splits;
    a.prefix_slot0 = (int64_t)p.workers + S * Hkv;
    a.tables += prefix_len / bs;
    if (phase != pkv::kMergePhase) {
      pkv::PrefixArgs pa{};
      pa.q = q->data;
      pa.kc = key_cache->data;
      pa.vc = value_cache->data;
      pa.blocks = static_cast<const int32_t*>(block_tables->data);  // row 0: the shared blocks
      pa.ws_acc = a.ws_acc;
      pa.ws_ml = a.ws_ml;
      pa.slot0 = a.prefix_slot0;
      pa.num_seqs = (int32_t)S;
      pa.num_q_heads = (int32_t)Hq;
      pa.num_kv_heads = (int32_t)Hkv;
      pa.group = (int32_t)(Hq / Hkv);
      pa.head_dim = (int32_t)D;
      pa.block_size = (int32_t)bs;
      pa.prefix_len = prefix_len;
      pa.splits = p.prefix_splits;
      pa.cache_dtype = ct;
      pa.qk_scale = a.qk_scale;
      const hipError_t e = pkv::launch_shared_prefix(pa, stream);
      if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
    }
  }
  const hipError_t e = pkv::launch_decode(a, stream);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(e));
  return ok();
}

int32_t phase_of(const pkv_decode_opts* opts) {
  return opts && (opts->flags & PKV_DECODE_DEFER_MERGE) ? pkv::kSplitPhase : pkv::kBothPhases;
}

}  // namespace

extern "C" {

pkv_status paged_attention_decode(pkv_tensor* out, const pkv_tensor* q, const pkv_tensor* key_cache,
                                  const pkv_tensor* value_cache, const pkv_tensor* block_tables,
                                  const pkv_tensor* context_lens, float scale, int32_t block_size,
                                  const pkv_decode_opts* opts, void* hip_stream) {
  return decode_impl("paged_attention_decode", out, q, key_cache, value_cache, block_tables,
                     context_lens, scale, block_size, opts, nullptr, phase_of(opts), hip_stream);
}

pkv_status paged_attention_decode_noalloc(pkv_tensor* out, const pkv_tensor* q,
                                          const pkv_tensor* key_cache,
                                          const pkv_tensor* value_cache,
                                          const pkv_tensor* block_tables,
                                          const pkv_tensor* context_lens, float scale,
                                          int32_t block_size, const pkv_decode_opts* opts,
                                          void* hip_stream) {
  // the split workspace is sized from the descriptors alone, before any device call
  PKV_TRY(check_tensor(q, "q", 3));
  PKV_TRY(check_tensor(key_cache, "key_cache", 4));
  PKV_TRY(check_tensor(block_tables, "block_tables", 2));
  if (opts && (opts->flags & PKV_DECODE_DEFER_MERGE))
    return fail(PKV_ERR_UNSUPPORTED, "paged_attention_decode_noalloc: PKV_DECODE_DEFER_MERGE is "
                                     "not supported (the scratch is not the caller's)");
  pkv_decode_opts o{};
  if (opts) o = *opts;
  o.workspace = nullptr;
  o.workspace_bytes = 0;
  const int64_t S = q->shape[0], Hq = q->shape[1], D = q->shape[2], Hkv = key_cache->shape[1];
  const int64_t maxb = block_tables->shape[1];
  size_t need = 0;
  if (S > 0 && Hkv > 0 && Hq % Hkv == 0 && S <= INT32_MAX && Hq <= INT32_MAX && D <= INT32_MAX &&
      maxb <= INT32_MAX)
    need = paged_attention_decode_workspace_bytes((int32_t)S, (int32_t)Hq, (int32_t)Hkv, (int32_t)D,
                                                  (int32_t)maxb, block_size, opts ? &o : nullptr);
  if (need > pkv::kScratchBytes)
    return fail(PKV_ERR_WORKSPACE, "paged_attention_decode_noalloc: this call needs %zu bytes of "
                                   "split workspace, more than the %zu bytes of scratch",
                need, pkv::kScratchBytes);
  if (need > 0) {
    void* p = nullptr;
    const hipError_t e = pkv::scratch_for_current_device(&p);
    if (e != hipSuccess)
      return fail(PKV_ERR_HIP, "paged_attention_decode_noalloc: scratch address: %s",
                  hipGetErrorString(e));
    o.workspace = p;
    o.workspace_bytes = pkv::kScratchBytes;
  }
  return decode_impl("paged_attention_decode_noalloc", out, q, key_cache, value_cache, block_tables,
                     context_lens, scale, block_size, opts ? &o : nullptr, nullptr,
                     pkv::kBothPhases, hip_stream);
}

size_t pkv_noalloc_scratch_bytes(void) { return pkv::kScratchBytes; }

pkv_status paged_attention_decode_merge(pkv_tensor* out, const pkv_tensor* q,
                                        const pkv_tensor* key_cache, const pkv_tensor* value_cache,
                                        const pkv_tensor* block_tables,
                                        const pkv_tensor* context_lens, float scale,
                                        int32_t block_size, const pkv_decode_opts* opts,
                                        void* hip_stream) {
  return decode_impl("paged_attention_decode_merge", out, q, key_cache, value_cache, block_tables,
                     context_lens, scale, block_size, opts, nullptr, pkv::kMergePhase, hip_stream);
}

pkv_status paged_attention_decode_shared_prefix(pkv_tensor* out, const pkv_tensor* q,
                                                const pkv_tensor* key_cache,
                                                const pkv_tensor* value_cache,
                                                const pkv_tensor* block_tables,
                                                const pkv_tensor* context_lens, int32_t prefix_len,
                                                float scale, int32_t block_size,
                                                const pkv_decode_opts* opts, void* hip_stream) {
  if (prefix_len <= 0) return fail(PKV_ERR_SHAPE, "prefix_len must be positive");
  if (opts && (opts->flags & PKV_DECODE_DEFER_MERGE))
    return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode launches its kernels together: "
                                     "PKV_DECODE_DEFER_MERGE is not supported");
  return decode_impl("paged_attention_decode_shared_prefix", out, q, key_cache, value_cache,
                     block_tables, context_lens, scale, block_size, opts, nullptr, phase_of(opts),
                     hip_stream, prefix_len);
}

pkv_status paged_attention_decode_append(pkv_tensor* out, const pkv_tensor* q, const pkv_tensor* k,
                                         const pkv_tensor* v, const pkv_tensor* slot_mapping,
                                         pkv_tensor* key_cache, pkv_tensor* value_cache,
                                         const pkv_tensor* block_tables,
                                         const pkv_tensor* context_lens, float scale,
                                         int32_t block_size, const pkv_decode_opts* opts,
                                         void* hip_stream) {
  if (!k || !v || !slot_mapping) return fail(PKV_ERR_NULL, "k, v and slot_mapping must not be NULL");
  const AppendIn app{k, v, slot_mapping};
  return decode_impl("paged_attention_decode_append", out, q, key_cache, value_cache, block_tables,
                     context_lens, scale, block_size, opts, &app, phase_of(opts), hip_stream);
}

pkv_status paged_attention_decode_shared_prefix_append(
    pkv_tensor* out, const pkv_tensor* q, const pkv_tensor* k, const pkv_tensor* v,
    const pkv_tensor* slot_mapping, pkv_tensor* key_cache, pkv_tensor* value_cache,
    const pkv_tensor* block_tables, const pkv_tensor* context_lens, int32_t prefix_len, float scale,
    int32_t block_size, const pkv_decode_opts* opts, void* hip_stream) {
  if (!k || !v || !slot_mapping) return fail(PKV_ERR_NULL, "k, v and slot_mapping must not be NULL");
  if (prefix_len <= 0) return fail(PKV_ERR_SHAPE, "prefix_len must be positive");
  if (opts && (opts->flags & PKV_DECODE_DEFER_MERGE))
    return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode launches its kernels together: "
                                     "PKV_DECODE_DEFER_MERGE is not supported");
  const AppendIn app{k, v, slot_mapping};
  return decode_impl("paged_attention_decode_shared_prefix_append", out, q, key_cache, value_cache,
                     block_tables, context_lens, scale, block_size, opts, &app, phase_of(opts),
                     hip_stream, prefix_len);
}

pkv_status pkv_validate_slots(const int32_t* slots, int64_t num_tokens, int64_t num_blocks,
                              int32_t block_size) {
  if (num_tokens < 0 || num_blocks < 0 || block_size <= 0)
    return fail(PKV_ERR_SHAPE, "negative sizes or non-positive block_size");
  if (num_tokens > 0 && !slots) return fail(PKV_ERR_NULL, "slots is NULL");
  const int64_t cap = num_blocks * block_size;
  std::vector<int32_t> live;
  live.reserve((size_t)num_tokens);
  for (int64_t t = 0; t < num_tokens; ++t) {
    if (slots[t] < 0) continue;
    if (slots[t] >= cap)
      return fail(PKV_ERR_RANGE, "slot %d of token %lld is outside the pool (%lld slots)", slots[t],
                  (long long)t, (long long)cap);
    live.push_back(slots[t]);
  }
  std::sort(live.begin(), live.end());
  for (size_t i = 1; i < live.size(); ++i)
    if (live[i] == live[i - 1]) return fail(PKV_ERR_RANGE, "slot %d is repeated", live[i]);
  return ok();
}

pkv_status pkv_validate_decode_inputs(const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t max_blocks_per_seq,
                                      int64_t num_blocks, int32_t block_size) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || num_blocks < 0 || block_size <= 0)
    return fail(PKV_ERR_SHAPE, "negative sizes or non-positive block_size");
  if (num_seqs > 0 && (!block_tables || !context_lens)) return fail(PKV_ERR_NULL, "NULL input");
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t n = context_lens[s];
    if (n < 0 || n > (int64_t)max_blocks_per_seq * block_size)
      return fail(PKV_ERR_RANGE, "context_lens[%d] = %lld outside [0, %lld]", s, (long long)n,
                  (long long)max_blocks_per_seq * block_size);
    const int64_t nb = (n + block_size - 1) / block_size;
    for (int64_t j = 0; j < nb; ++j) {
      const int32_t b = block_tables[(int64_t)s * max_blocks_per_seq + j];
      if (b < 0 || b >= num_blocks)
        return fail(PKV_ERR_RANGE, "block_tables[%d][%lld] = %d outside [0, %lld)", s, (long long)j,
                    b, (long long)num_blocks);
    }
  }
  return ok();
}

pkv_status pkv_decode_order(const int32_t* context_lens, int32_t num_seqs, int32_t* order) {
  if (num_seqs < 0) return fail(PKV_ERR_SHAPE, "num_seqs %d < 0", num_seqs);
  if (num_seqs > 0 && (!context_lens || !order)) return fail(PKV_ERR_NULL, "NULL input");
  for (int32_t s = 0; s < num_seqs; ++s) order[s] = s;
  std::stable_sort(order, order + num_seqs,
                   [&](int32_t x, int32_t y) { return context_lens[x] > context_lens[y]; });
  return ok();
}

pkv_status pkv_validate_seq_order(const int32_t* seq_order, int32_t num_seqs) {
  if (num_seqs < 0) return fail(PKV_ERR_SHAPE, "num_seqs %d < 0", num_seqs);
  if (num_seqs > 0 && !seq_order) return fail(PKV_ERR_NULL, "seq_order is NULL");
  std::vector<char> seen((size_t)num_seqs, 0);
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t s = seq_order[i];
    if (s < 0 || s >= num_seqs)
      return fail(PKV_ERR_RANGE, "seq_order[%d] = %d outside [0, %d)", i, s, num_seqs);
    if (seen[(size_t)s]) return fail(PKV_ERR_RANGE, "seq_order[%d] = %d repeats", i, s);
    seen[(size_t)s] = 1;
  }
  return ok();
}

pkv_status pkv_validate_append_slots(const int32_t* slots, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t max_blocks_per_seq, int64_t num_blocks,
                                     int32_t block_size) {
  PKV_TRY(pkv_validate_decode_inputs(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                     num_blocks, block_size));
  if (num_seqs > 0 && !slots) return fail(PKV_ERR_NULL, "slots is NULL");
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (slots[s] < 0) continue;
    const int64_t n = context_lens[s];
    if (n == 0) return fail(PKV_ERR_RANGE, "sequence %d has no tokens but slot %d", s, slots[s]);
    const int64_t pos = n - 1;
    const int64_t want = (int64_t)block_tables[(int64_t)s * max_blocks_per_seq + pos / block_size] *
                             block_size + pos % block_size;
    if (slots[s] != want)
      return fail(PKV_ERR_RANGE, "slot %d of sequence %d is not position %lld (slot %lld)", slots[s],
                  s, (long long)pos, (long long)want);
  }
  // a block written by one sequence must not be read by another in the same
  // call (a block still shared has to be copied before the write)
  std::unordered_map<int32_t, int32_t> writer;
  for (int32_t s = 0; s < num_seqs; ++s)
    if (slots[s] >= 0) writer.emplace(slots[s] / block_size, s);
  for (int32_t s = 0; s < num_seqs && !writer.empty(); ++s) {
    const int64_t nb = ((int64_t)context_lens[s] + block_size - 1) / block_size;
    for (int64_t j = 0; j < nb; ++j) {
      const auto it = writer.find(block_tables[(int64_t)s * max_blocks_per_seq + j]);
      if (it != writer.end() && it->second != s)
        return fail(PKV_ERR_RANGE, "block %d is written by sequence %d and read by sequence %d",
                    it->first, it->second, s);
    }
  }
  return ok();
}

pkv_status pkv_validate_prefill_inputs(const int32_t* query_start_loc, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t max_blocks_per_seq, int64_t num_blocks,
                                      int32_t block_size, int64_t num_query_rows,
                                      int32_t max_query_len) {
  PKV_TRY(pkv_validate_decode_inputs(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                     num_blocks, block_size));
  if (!query_start_loc) return fail(PKV_ERR_NULL, "query_start_loc is NULL");
  if (query_start_loc[0] != 0) return fail(PKV_ERR_RANGE, "query_start_loc[0] = %d, not 0", query_start_loc[0]);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t n = (int64_t)query_start_loc[s + 1] - query_start_loc[s];
    if (n < 0) return fail(PKV_ERR_RANGE, "query_start_loc decreases at sequence %d", s);
    if (n > context_lens[s])
      return fail(PKV_ERR_RANGE, "sequence %d has %lld queries but %d tokens", s, (long long)n,
                  context_lens[s]);
    if (n > max_query_len)
      return fail(PKV_ERR_RANGE, "sequence %d has %lld queries > max_query_len %d", s,
                  (long long)n, max_query_len);
  }
  if (query_start_loc[num_seqs] != num_query_rows)
    return fail(PKV_ERR_RANGE, "query_start_loc[S] = %d, q has %lld rows", query_start_loc[num_seqs],
                (long long)num_query_rows);
  return ok();
}

pkv_status pkv_validate_shared_prefix(const int32_t* block_tables, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t max_blocks_per_seq,
                                     int64_t num_blocks, int32_t block_size, int32_t prefix_len) {
  PKV_TRY(pkv_validate_decode_inputs(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                     num_blocks, block_size));
  if (prefix_len <= 0 || prefix_len % block_size != 0 ||
      (int64_t)prefix_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_ERR_SHAPE, "prefix_len %d: must be a positive multiple of block_size", prefix_len);
  const int32_t nb = prefix_len / block_size;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (context_lens[s] < prefix_len)
      return fail(PKV_ERR_RANGE, "sequence %d has %d tokens, fewer than the prefix's %d", s,
                  context_lens[s], prefix_len);
    for (int32_t j = 0; j < nb; ++j)
      if (block_tables[(int64_t)s * max_blocks_per_seq + j] != block_tables[j])
        return fail(PKV_ERR_RANGE, "sequence %d does not list the shared block %d at entry %d", s,
                    block_tables[j], j);
  }
  return ok();
}

pkv_status pkv_validate_block_ids(const int32_t* block_ids, int64_t num_ids, int64_t num_blocks) {
  if (num_ids < 0 || num_blocks < 0) return fail(PKV_ERR_SHAPE, "negative sizes");
  if (num_ids > 0 && !block_ids) return fail(PKV_ERR_NULL, "block_ids is NULL");
  std::vector<int32_t> ids;
  for (int64_t i = 0; i < num_ids; ++i) {
    if (block_ids[i] < 0) continue;
    if (block_ids[i] >= num_blocks)
      return fail(PKV_ERR_RANGE, "block id %d outside the pool of %lld blocks", block_ids[i],
                  (long long)num_blocks);
    ids.push_back(block_ids[i]);
  }
  std::sort(ids.begin(), ids.end());
  for (size_t i = 1; i < ids.size(); ++i)
    if (ids[i] == ids[i - 1]) return fail(PKV_ERR_RANGE, "block id %d repeated", ids[i]);
  return ok();
}

pkv_status pkv_validate_block_pairs(const int32_t* block_pairs, int64_t num_pairs,
                                    int64_t num_blocks) {
  if (num_pairs < 0 || num_blocks < 0) return fail(PKV_ERR_SHAPE, "negative sizes");
  if (num_pairs > 0 && !block_pairs) return fail(PKV_ERR_NULL, "block_pairs is NULL");
  std::vector<int32_t> srcs, dsts;
  for (int64_t i = 0; i < num_pairs; ++i) {
    const int32_t s = block_pairs[2 * i], d = block_pairs[2 * i + 1];
    if (s < 0 || d < 0 || s == d) continue;
    if (s >= num_blocks || d >= num_blocks)
      return fail(PKV_ERR_RANGE, "pair %lld (%d, %d) outside the pool of %lld blocks", (long long)i,
                  s, d, (long long)num_blocks);
    srcs.push_back(s);
    dsts.push_back(d);
  }
  std::sort(dsts.begin(), dsts.end());
  for (size_t i = 1; i < dsts.size(); ++i)
    if (dsts[i] == dsts[i - 1]) return fail(PKV_ERR_RANGE, "destination block %d repeated", dsts[i]);
  for (int32_t s : srcs)
    if (std::binary_search(dsts.begin(), dsts.end(), s))
      return fail(PKV_ERR_RANGE, "block %d is both a source and a destination", s);
  return ok();
}

}  // extern "C"
