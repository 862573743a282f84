// C ABI of librla_attn.so: host-side validation, launch planning and error
// reporting.  Every check runs before anything is enqueued, so a rejected call
// has no effect on the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "kernels.hpp"
#include "rla_attn.h"

static_assert(RLA_DECODE_STATIC_SCRATCH_BYTES == rla::kStaticDecodeScratchBytes,
              "header and library disagree on the static decode scratch size");

namespace {

thread_local char g_err[512] = "";

rla_status fail(rla_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

rla_status ok() {
  g_err[0] = '\0';
  return RLA_OK;
}

rla_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(RLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Shared parameter checks.  attention_call: the full attention contract
// (head shard, block size, scale, causal flag, fixed fold order); otherwise
// only what a merge uses (Hq, head_dim, dtypes, fold order).  group = Hq / Hkv
// on success of an attention check.
rla_status check_params(const rla_attn_params* p, bool attention_call, int* group) {
  if (p == nullptr) return fail(RLA_ERR_NULL_POINTER, "params is NULL");
  if (p->num_q_heads <= 0) return fail(RLA_ERR_BAD_SHAPE, "num_q_heads=%d must be positive", p->num_q_heads);
  if (p->head_dim != rla::kHeadDimPublic)
    return fail(RLA_ERR_UNSUPPORTED, "head_dim=%d unsupported (only 128)", p->head_dim);
  if (p->acc_dtype != RLA_DT_FP32) return fail(RLA_ERR_UNSUPPORTED, "acc_dtype must be FP32");
  if (p->out_dtype != RLA_DT_BF16 && p->out_dtype != RLA_DT_FP32)
    return fail(RLA_ERR_UNSUPPORTED, "out_dtype=%d unsupported", p->out_dtype);
  if (p->merge_order != RLA_ORDER_GLOBAL_BLOCK_INDEX && p->merge_order != RLA_ORDER_ARRIVAL)
    return fail(RLA_ERR_UNSUPPORTED, "merge_order=%d unknown", p->merge_order);
  if (!attention_call) return RLA_OK;
  if (p->merge_order != RLA_ORDER_GLOBAL_BLOCK_INDEX)
    return fail(RLA_ERR_UNSUPPORTED, "attention calls fold in global_block_index order only");
  if (p->num_kv_heads <= 0) return fail(RLA_ERR_BAD_SHAPE, "num_kv_heads=%d must be positive", p->num_kv_heads);
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(RLA_ERR_BAD_SHAPE, "Hq=%d is not a multiple of Hkv=%d", p->num_q_heads, p->num_kv_heads);
  const int g = p->num_q_heads / p->num_kv_heads;
  static_assert(rla::kDecodeStageHeads >= 8, "decode tail units stage the items of groups of up to 8 q heads");
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(RLA_ERR_UNSUPPORTED, "GQA group Hq/Hkv=%d not in {1,2,4,8}", g);
  if (p->kv_block_size != 64 && p->kv_block_size != 128)
    return fail(RLA_ERR_UNSUPPORTED, "kv_block_size=%d unsupported (64 or 128)", p->kv_block_size);
  if (!(std::isfinite(p->softmax_scale)) || p->softmax_scale <= 0.0f)
    return fail(RLA_ERR_BAD_SHAPE, "softmax_scale must be finite and positive");
  if (p->causal != 0 && p->causal != 1) return fail(RLA_ERR_BAD_SHAPE, "causal must be 0 or 1");
  if (group) *group = g;
  return RLA_OK;
}

// The kernels address one head's K/V rows and one head's Q rows with 32-bit
// byte offsets (buffer resources).
bool fits_32bit_offsets(int64_t rows, int heads) {
  return rows <= 0 || (rows - 1) * heads * rla::kHeadDimPublic * 2 + rla::kHeadDimPublic * 2 <= 0x7fffffff;
}

// c = softmax_scale * log2(e), rounded once to fp32; every kernel receives it.
float score_scale(const rla_attn_params* p) {
  return static_cast<float>(static_cast<double>(p->softmax_scale) * 1.4426950408889634073599);
}

// Shared body of prefill and chunked prefill.
rla_status prefill_common(const rla_attn_params* p, const void* q, const void* k, const void* v,
                          int32_t batch, int32_t q_rows, int64_t pos0, int64_t kv_len, int32_t s_kv,
                          const rla_shard* shard, void* out, float* lse, void* stream) {
  int g = 0;
  rla_status st = check_params(p, true, &g);
  if (st != RLA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr) return fail(RLA_ERR_NULL_POINTER, "q, k or v is NULL");
  const int Hq = p->num_q_heads, Hkv = p->num_kv_heads, D = rla::kHeadDimPublic;

  if (!fits_32bit_offsets(kv_len, p->num_kv_heads) || !fits_32bit_offsets(q_rows, Hq))
    return fail(RLA_ERR_UNSUPPORTED, "sequence too long: one head's rows must span < 2 GiB (q_rows=%d, kv_len=%lld)",
                q_rows, (long long)kv_len);

  rla::PrefillArgs a;
  std::memset(&a, 0, sizeof a);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.q_bstride = static_cast<int64_t>(q_rows) * Hq * D;
  a.kv_bstride = static_cast<int64_t>(s_kv) * Hkv * D;
  a.kv_len = kv_len;
  a.B = batch;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = g;  // the launcher picks the tile shape (heads_per_wg, pos_groups, hsubs, n_ptiles)
  a.causal = p->causal;
  a.c = score_scale(p);

  bool emit = false;
  int64_t q_begin = 0, q_count = q_rows;
  if (shard != nullptr) {
    emit = true;
    if (shard->kv_blocks == nullptr || shard->partials == nullptr)
      return fail(RLA_ERR_NULL_POINTER, "shard->kv_blocks or shard->partials is NULL");
    const rla_partials* pt = shard->partials;
    if (pt->out == nullptr || pt->lse == nullptr) return fail(RLA_ERR_NULL_POINTER, "partials out/lse is NULL");
    if (shard->n_kv_blocks < 1 || shard->n_kv_blocks > RLA_MAX_PARTS)
      return fail(RLA_ERR_BAD_SHAPE, "n_kv_blocks=%d outside [1, %d]", shard->n_kv_blocks, RLA_MAX_PARTS);
    q_begin = shard->q_begin;
    q_count = shard->q_count;
    if (q_begin < 0 || q_count < 1 || q_begin + q_count > q_rows)
      return fail(RLA_ERR_BAD_SHAPE, "query slab [%lld, %lld) outside [0, %d)", (long long)q_begin,
                  (long long)(q_begin + q_count), q_rows);
    const int64_t n_blocks = (kv_len + p->kv_block_size - 1) / p->kv_block_size;
    std::vector<int64_t> ids(shard->kv_blocks, shard->kv_blocks + shard->n_kv_blocks);
    for (int64_t id : ids)
      if (id < 0 || id >= n_blocks || id > 0xffff)
        return fail(RLA_ERR_BAD_SHAPE, "kv block id %lld outside [0, %lld)", (long long)id, (long long)n_blocks);
    std::sort(ids.begin(), ids.end());
    if (std::adjacent_find(ids.begin(), ids.end()) != ids.end())
      return fail(RLA_ERR_DUPLICATE_BLOCK, "shard owns a kv block twice");
    if (pt->n_parts < shard->n_kv_blocks)
      return fail(RLA_ERR_BAD_SHAPE, "partials hold %d parts, shard owns %d blocks", pt->n_parts,
                  shard->n_kv_blocks);
    if (pt->rows != static_cast<int64_t>(batch) * q_count)
      return fail(RLA_ERR_BAD_SHAPE, "partials rows=%lld, expected batch*q_count=%lld", (long long)pt->rows,
                  (long long)batch * q_count);
    a.n_emit = shard->n_kv_blocks;
    for (int i = 0; i < shard->n_kv_blocks; ++i) a.emit_blocks[i] = static_cast<uint16_t>(shard->kv_blocks[i]);
    a.part_out = pt->out;
    a.part_lse = pt->lse;
  } else {
    if (out == nullptr || lse == nullptr) return fail(RLA_ERR_NULL_POINTER, "out or lse is NULL");
    a.out = out;
    a.lse = lse;
  }
  a.q = static_cast<const uint16_t*>(q) + q_begin * Hq * D;
  a.Sq = static_cast<int32_t>(q_count);
  a.pos0 = pos0 + q_begin;
  hipError_t e = rla::launch_prefill(a, p->kv_block_size, p->out_dtype == RLA_DT_FP32, emit,
                                     static_cast<hipStream_t>(stream));
  return hip_status(e, "prefill launch");
}

// The two decode launches (block items, ordered fold) after validation.
// context_lens == nullptr: every sequence has uniform_len keys; page_table ==
// nullptr: page i of sequence s is s*max_pages_per_seq + i.
rla_status run_decode(const rla_attn_params* p, int g, const void* q, const void* k_pool, const void* v_pool,
                      int64_t num_pages, int32_t page_size, const int32_t* page_table, int32_t max_pages_per_seq,
                      const int32_t* context_lens, int32_t uniform_len, const int32_t* host_context_lens,
                      int32_t batch, int32_t max_context_len, int64_t cap, void* workspace, void* out, float* lse,
                      hipStream_t s) {
  const int64_t max_blocks = std::max<int64_t>(1, (static_cast<int64_t>(max_context_len) + p->kv_block_size - 1) /
                                                      p->kv_block_size);
  const int64_t items = static_cast<int64_t>(batch) * max_blocks * p->num_q_heads;
  const int64_t out_bytes = (items * rla::kHeadDimPublic * 4 + 255) / 256 * 256;
  float* items_out = static_cast<float*>(workspace);
  float* items_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + out_bytes);

  rla::DecodeArgs d;
  std::memset(&d, 0, sizeof d);
  d.q = static_cast<const uint16_t*>(q);
  d.k_pool = static_cast<const uint16_t*>(k_pool);
  d.v_pool = static_cast<const uint16_t*>(v_pool);
  d.page_table = page_table;
  d.ctx_lens = context_lens;
  d.uniform_len = uniform_len;
  d.items_out = items_out;
  d.items_lse = items_lse;
  d.num_pages = num_pages;
  d.P = page_size;
  d.log2_P = 0;
  while ((1 << d.log2_P) < page_size) ++d.log2_P;  // page_size divides 64 or 128: a power of two
  d.max_pages = max_pages_per_seq;
  d.Bd = batch;
  d.Hq = p->num_q_heads;
  d.Hkv = p->num_kv_heads;
  d.G = g;
  d.max_blocks = static_cast<int32_t>(max_blocks);
  d.len_cap = static_cast<int32_t>(cap);
  d.c = score_scale(p);
  d.unit_blocks = rla::kDecodeUnitBlocks;
  // Head units fold up to 64 blocks each.  That saves those blocks' item
  // writes, but one workgroup walks them in turn, so heads are that long only
  // when the head units alone fill the GPU's decode workgroup slots (256 CUs,
  // two each); with fewer (sequence, kv head) pairs they shrink in proportion,
  // down to one tail unit's length, keeping a small batch spread over many
  // workgroups.  Their page ids must also fit the workgroup's staging area.
  constexpr int64_t kSlots = 512;
  const int64_t pairs = static_cast<int64_t>(batch) * p->num_kv_heads;
  int64_t head = pairs >= kSlots ? 64 : 64 * pairs / kSlots / rla::kDecodeUnitBlocks * rla::kDecodeUnitBlocks;
  head = std::max<int64_t>(head, rla::kDecodeUnitBlocks);
  head = std::min<int64_t>(head, static_cast<int64_t>(rla::kDecodeIdsCap) * page_size / p->kv_block_size);
  d.head_blocks = static_cast<int32_t>(head);
  d.out = out;
  d.lse = lse;
  auto tails_of = [&](int64_t len) {
    const int64_t nb = (len + p->kv_block_size - 1) / p->kv_block_size;
    return nb > d.head_blocks ? (nb - d.head_blocks + rla::kDecodeUnitBlocks - 1) / rla::kDecodeUnitBlocks : 0;
  };
  if (context_lens == nullptr) {
    // every sequence has uniform_len keys: one head and the same tails each
    d.len_mode = rla::kLensUniform;
    d.n_units = static_cast<int64_t>(batch) * (1 + tails_of(std::max<int64_t>(0, std::min<int64_t>(uniform_len, cap))));
  } else if (host_context_lens != nullptr && batch <= rla::kDecodeTableSeqs) {
    // the (validated) host lengths and the tail prefix sums travel with the
    // launches: exactly the units they need, no device length read
    d.len_mode = rla::kLensTable;
    int64_t tails = 0;
    for (int i = 0; i < batch; ++i) {
      d.lens[i] = host_context_lens[i];
      d.unit_start[i] = static_cast<int32_t>(tails);
      tails += tails_of(host_context_lens[i]);
    }
    d.unit_start[batch] = static_cast<int32_t>(tails);
    for (int i = 0; i < batch; ++i) d.head_order[i] = static_cast<int16_t>(i);
    std::stable_sort(d.head_order, d.head_order + batch,
                     [&](int16_t x, int16_t y) { return host_context_lens[x] > host_context_lens[y]; });
    d.n_units = batch + tails;
  } else {
    // device lengths: every unit up to max_context_len, idle ones exit
    d.len_mode = rla::kLensDevice;
    d.n_units = static_cast<int64_t>(batch) * (1 + tails_of(max_context_len));
  }
  const bool f32 = p->out_dtype == RLA_DT_FP32;
  hipError_t e = rla::launch_decode_items(d, p->kv_block_size, f32, s);
  if (e != hipSuccess) return hip_status(e, "decode launch");

  rla::FoldArgs f;
  std::memset(&f, 0, sizeof f);
  f.part_out = items_out;
  f.part_lse = items_lse;
  f.ctx_lens = context_lens;
  f.uniform_len = uniform_len;
  f.len_mode = d.len_mode;
  f.head_blocks = d.head_blocks;
  if (d.len_mode == rla::kLensTable) std::memcpy(f.lens, d.lens, sizeof(int32_t) * batch);
  f.out = out;
  f.lse = lse;
  f.rows = batch;
  f.Hq = p->num_q_heads;
  f.n_parts = static_cast<int32_t>(max_blocks);
  f.block = p->kv_block_size;
  f.len_cap = static_cast<int32_t>(cap);
  e = rla::launch_fold(f, true, f32, s);
  return hip_status(e, "decode fold launch");
}

// A chunk of one query is a decode step over the cache: the contiguous cache
// [B][s_max][Hkv][128] is a paged pool with one key per page (page id
// b*s_max + j), so the decode kernels run it, spreading the KV blocks over
// many workgroups and folding the block items in order.  Their per-(row,
// block) arithmetic is that of the prefill kernels, so the bits are the same.
// The route is taken when the page ids fit int32 (no shard); its block items
// go to the caller's workspace.
bool single_query_route(int32_t batch, int32_t chunk_len, int32_t s_max, const rla_shard* shard) {
  return chunk_len == 1 && shard == nullptr && static_cast<int64_t>(batch) * s_max <= 0x7fffffff;
}

// Validation shared by the two decode entry points (everything but the
// workspace).  On success *group and *cap hold Hq/Hkv and the length cap.
rla_status validate_decode(const rla_attn_params* p, const void* q, const void* k_pool, const void* v_pool,
                           int64_t num_pages, int32_t page_size, const int32_t* page_table,
                           int32_t max_pages_per_seq, const int32_t* context_lens, const int32_t* host_context_lens,
                           int32_t batch, int32_t max_context_len, void* out, float* lse, int* group, int64_t* cap) {
  rla_status st = check_params(p, true, group);
  if (st != RLA_OK) return st;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || page_table == nullptr ||
      context_lens == nullptr || out == nullptr || lse == nullptr)
    return fail(RLA_ERR_NULL_POINTER, "a required pointer is NULL");
  if (batch < 1 || max_context_len < 0 || max_context_len > (1 << 30) || num_pages < 1 || page_size < 1 ||
      max_pages_per_seq < 1)
    return fail(RLA_ERR_BAD_SHAPE, "need batch>=1, 0<=max_context_len<=2^30, num_pages>=1, page_size>=1, "
                "max_pages_per_seq>=1");
  if (p->kv_block_size % page_size != 0)
    return fail(RLA_ERR_UNSUPPORTED, "page_size=%d must divide kv_block_size=%d", page_size, p->kv_block_size);
  if (num_pages > 0x7fffffff) return fail(RLA_ERR_BAD_SHAPE, "num_pages exceeds int32 page ids");
  *cap = std::min<int64_t>(max_context_len, static_cast<int64_t>(max_pages_per_seq) * page_size);
  if (host_context_lens != nullptr) {
    for (int i = 0; i < batch; ++i)
      if (host_context_lens[i] < 0 || host_context_lens[i] > *cap)
        return fail(RLA_ERR_BAD_SHAPE, "context_lens[%d]=%d outside [0, %lld]", i, host_context_lens[i],
                    (long long)*cap);
  }
  return RLA_OK;
}

}  // namespace

extern "C" {


const char* rla_last_error(void) { return g_err; }

const char* rla_core_id(void) { return "rla.attention.core.v1"; }

rla_status rla_attn_prefill(const rla_attn_params* p, const void* q, const void* k, const void* v,
                            int32_t batch, int32_t seq_len, const rla_shard* shard, void* out, float* lse,
                            void* hip_stream) {
  if (batch < 1 || seq_len < 1)
    return fail(RLA_ERR_BAD_SHAPE, "batch=%d and seq_len=%d must be >= 1", batch, seq_len);
  return prefill_common(p, q, k, v, batch, seq_len, 0, seq_len, seq_len, shard, out, lse, hip_stream);
}

size_t rla_chunked_workspace_bytes(const rla_attn_params* p, int32_t batch, int32_t chunk_len, int32_t cache_len,
                                   int32_t s_max) {
  if (batch < 1 || cache_len < 0 || s_max < 1 || !single_query_route(batch, chunk_len, s_max, nullptr)) return 0;
  return rla_decode_workspace_bytes(p, batch, cache_len + 1);
}

rla_status rla_attn_prefill_chunked(const rla_attn_params* p, const void* q_chunk, const void* k_cache,
                                    const void* v_cache, int32_t batch, int32_t chunk_len, int32_t cache_len,
                                    int32_t s_max, const rla_shard* shard, void* workspace,
                                    size_t workspace_bytes, void* out, float* lse, void* hip_stream) {
  if (batch < 1 || chunk_len < 1 || cache_len < 0 || s_max < 1 ||
      static_cast<int64_t>(cache_len) + chunk_len > s_max)
    return fail(RLA_ERR_BAD_SHAPE, "need batch>=1, chunk_len>=1, cache_len>=0, cache_len+chunk_len<=s_max "
                "(got %d, %d, %d, %d)", batch, chunk_len, cache_len, s_max);
  if (single_query_route(batch, chunk_len, s_max, shard)) {
    int g = 0;
    const rla_status st0 = check_params(p, true, &g);
    if (st0 != RLA_OK) return st0;
    if (q_chunk == nullptr || k_cache == nullptr || v_cache == nullptr || out == nullptr || lse == nullptr ||
        workspace == nullptr)
      return fail(RLA_ERR_NULL_POINTER, "a required pointer is NULL (a chunk of one query needs the workspace)");
    const int32_t len = cache_len + 1;
    const size_t need = rla_decode_workspace_bytes(p, batch, len);
    if (workspace_bytes < need)
      return fail(RLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    return run_decode(p, g, q_chunk, k_cache, v_cache, static_cast<int64_t>(batch) * s_max, 1, nullptr, s_max,
                      nullptr, len, nullptr, batch, len, len, workspace, out, lse, static_cast<hipStream_t>(hip_stream));
  }
  return prefill_common(p, q_chunk, k_cache, v_cache, batch, chunk_len, cache_len,
                        static_cast<int64_t>(cache_len) + chunk_len, s_max, shard, out, lse, hip_stream);
}

rla_status rla_attn_prefill_paged(const rla_attn_params* p, const void* q_chunk, const void* k_pool,
                                  const void* v_pool, int64_t num_pages, int32_t page_size,
                                  const int32_t* page_table, int32_t max_pages_per_seq, int32_t batch,
                                  int32_t chunk_len, int32_t cache_len, void* out, float* lse,
                                  void* hip_stream) {
  int g = 0;
  rla_status st = check_params(p, true, &g);
  if (st != RLA_OK) return st;
  if (q_chunk == nullptr || k_pool == nullptr || v_pool == nullptr || page_table == nullptr || out == nullptr ||
      lse == nullptr)
    return fail(RLA_ERR_NULL_POINTER, "a required pointer is NULL");
  if (batch < 1 || chunk_len < 1 || cache_len < 0 || num_pages < 1 || max_pages_per_seq < 1)
    return fail(RLA_ERR_BAD_SHAPE, "need batch>=1, chunk_len>=1, cache_len>=0, num_pages>=1, max_pages_per_seq>=1");
  if (num_pages > 0x7fffffff) return fail(RLA_ERR_BAD_SHAPE, "num_pages exceeds int32 page ids");
  if (page_size < 4 || page_size > p->kv_block_size || (page_size & (page_size - 1)) != 0)
    return fail(RLA_ERR_UNSUPPORTED, "page_size=%d must be a power of two in [4, kv_block_size=%d]", page_size,
                p->kv_block_size);
  const int64_t kv_len = static_cast<int64_t>(cache_len) + chunk_len;
  if (static_cast<int64_t>(max_pages_per_seq) * page_size < kv_len)
    return fail(RLA_ERR_BAD_SHAPE, "max_pages_per_seq*page_size=%lld does not cover cache_len+chunk_len=%lld",
                (long long)max_pages_per_seq * page_size, (long long)kv_len);
  // key positions and block starts (plus one block) stay inside int32 in the kernels
  if (kv_len > (1 << 30)) return fail(RLA_ERR_BAD_SHAPE, "cache_len+chunk_len=%lld exceeds 2^30", (long long)kv_len);
  const int Hq = p->num_q_heads, D = rla::kHeadDimPublic;
  if (!fits_32bit_offsets(chunk_len, Hq))
    return fail(RLA_ERR_UNSUPPORTED, "chunk too long: one head's query rows must span < 2 GiB");

  rla::PrefillArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = static_cast<const uint16_t*>(q_chunk);
  a.k = static_cast<const uint16_t*>(k_pool);
  a.v = static_cast<const uint16_t*>(v_pool);
  a.q_bstride = static_cast<int64_t>(chunk_len) * Hq * D;
  a.kv_bstride = 0;  // keys come through the page table
  a.pos0 = cache_len;
  a.kv_len = kv_len;
  a.B = batch;
  a.Sq = chunk_len;
  a.Hq = Hq;
  a.Hkv = p->num_kv_heads;
  a.G = g;
  a.causal = p->causal;
  a.c = score_scale(p);
  a.out = out;
  a.lse = lse;
  a.page_table = page_table;
  a.num_pages = num_pages;
  a.max_pages = max_pages_per_seq;
  a.log2_P = 0;
  while ((1 << a.log2_P) < page_size) ++a.log2_P;
  hipError_t e = rla::launch_prefill_paged(a, p->kv_block_size, p->out_dtype == RLA_DT_FP32,
                                           static_cast<hipStream_t>(hip_stream));
  return hip_status(e, "paged prefill launch");
}

size_t rla_decode_workspace_bytes(const rla_attn_params* p, int32_t batch, int32_t max_context_len) {
  int g = 0;
  if (check_params(p, true, &g) != RLA_OK || batch < 1 || max_context_len < 0) return 0;
  const int64_t max_blocks = std::max<int64_t>(1, (static_cast<int64_t>(max_context_len) + p->kv_block_size - 1) /
                                                      p->kv_block_size);
  const int64_t items = static_cast<int64_t>(batch) * max_blocks * p->num_q_heads;
  const int64_t out_bytes = (items * rla::kHeadDimPublic * 4 + 255) / 256 * 256;
  return static_cast<size_t>(out_bytes + items * 4);
}

rla_status rla_attn_decode_paged(const rla_attn_params* p, const void* q, const void* k_pool, const void* v_pool,
                                 int64_t num_pages, int32_t page_size, const int32_t* page_table,
                                 int32_t max_pages_per_seq, const int32_t* context_lens,
                                 const int32_t* host_context_lens, int32_t batch, int32_t max_context_len,
                                 void* workspace, size_t workspace_bytes, void* out, float* lse,
                                 void* hip_stream) {
  int g = 0;
  int64_t cap = 0;
  rla_status st = validate_decode(p, q, k_pool, v_pool, num_pages, page_size, page_table, max_pages_per_seq,
                                  context_lens, host_context_lens, batch, max_context_len, out, lse, &g, &cap);
  if (st != RLA_OK) return st;
  if (workspace == nullptr) return fail(RLA_ERR_NULL_POINTER, "workspace is NULL");
  const size_t need = rla_decode_workspace_bytes(p, batch, max_context_len);
  if (workspace_bytes < need)
    return fail(RLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  return run_decode(p, g, q, k_pool, v_pool, num_pages, page_size, page_table, max_pages_per_seq, context_lens, 0,
                    host_context_lens, batch, max_context_len, cap, workspace, out, lse,
                    static_cast<hipStream_t>(hip_stream));
}

rla_status rla_attn_decode_paged_static(const rla_attn_params* p, const void* q, const void* k_pool,
                                        const void* v_pool, int64_t num_pages, int32_t page_size,
                                        const int32_t* page_table, int32_t max_pages_per_seq,
                                        const int32_t* context_lens, const int32_t* host_context_lens,
                                        int32_t batch, int32_t max_context_len, void* out, float* lse,
                                        void* hip_stream) {
  int g = 0;
  int64_t cap = 0;
  rla_status st = validate_decode(p, q, k_pool, v_pool, num_pages, page_size, page_table, max_pages_per_seq,
                                  context_lens, host_context_lens, batch, max_context_len, out, lse, &g, &cap);
  if (st != RLA_OK) return st;
  const size_t need = rla_decode_workspace_bytes(p, batch, max_context_len);
  if (need > RLA_DECODE_STATIC_SCRATCH_BYTES)
    return fail(RLA_ERR_WORKSPACE_TOO_SMALL, "decode needs %zu bytes of block items, above the %zu-byte static "
                "scratch of rla_attn_decode_paged_static", need, (size_t)RLA_DECODE_STATIC_SCRATCH_BYTES);
  hipError_t e = hipSuccess;
  void* scratch = rla::static_decode_scratch(&e);
  if (scratch == nullptr) return hip_status(e, "static decode scratch");
  return run_decode(p, g, q, k_pool, v_pool, num_pages, page_size, page_table, max_pages_per_seq, context_lens, 0,
                    host_context_lens, batch, max_context_len, cap, scratch, out, lse,
                    static_cast<hipStream_t>(hip_stream));
}

rla_status rla_attn_backward(const rla_attn_params* p, const void* q, const void* k, const void* v,
                             const void* out, const float* lse, const void* dout, int32_t batch,
                             int32_t q_rows, int32_t cache_len, int32_t s_max, int32_t accumulate,
                             rla_dtype grad_dtype, void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
  int g = 0;
  rla_status st = check_params(p, true, &g);
  if (st != RLA_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || lse == nullptr || dout == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr || workspace == nullptr)
    return fail(RLA_ERR_NULL_POINTER, "a required pointer is NULL");
  if (batch < 1 || q_rows < 1 || cache_len < 0 || s_max < 1 || static_cast<int64_t>(cache_len) + q_rows > s_max)
    return fail(RLA_ERR_BAD_SHAPE, "need batch>=1, q_rows>=1, cache_len>=0, cache_len+q_rows<=s_max "
                "(got %d, %d, %d, %d)", batch, q_rows, cache_len, s_max);
  if (accumulate != 0 && accumulate != 1) return fail(RLA_ERR_BAD_SHAPE, "accumulate must be 0 or 1");
  if (grad_dtype != RLA_DT_BF16 && grad_dtype != RLA_DT_FP32)
    return fail(RLA_ERR_UNSUPPORTED, "grad_dtype=%d unsupported", grad_dtype);
  if (accumulate && grad_dtype != RLA_DT_FP32)
    return fail(RLA_ERR_UNSUPPORTED, "accumulate needs fp32 gradients (the running sums are fp32)");
  const int Hq = p->num_q_heads, Hkv = p->num_kv_heads, D = rla::kHeadDimPublic;
  const int64_t kv_len = static_cast<int64_t>(cache_len) + q_rows;
  // Sq_pad = q_rows rounded up to the 64-row tile; its rows must fit the
  // 32-bit row offsets too.
  const int64_t sq_pad = (static_cast<int64_t>(q_rows) + 63) / 64 * 64;
  if (!fits_32bit_offsets(kv_len, Hkv) || !fits_32bit_offsets(sq_pad, Hq) || sq_pad > 0x7fffffff)
    return fail(RLA_ERR_UNSUPPORTED, "sequence too long: one head's rows must span < 2 GiB (q_rows=%d, kv_len=%lld)",
                q_rows, (long long)kv_len);
  const size_t need = rla_backward_workspace_bytes(p, batch, q_rows);
  if (workspace_bytes < need)
    return fail(RLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);

  rla::BackwardArgs a;
  std::memset(&a, 0, sizeof a);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = out;
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.q_bstride = static_cast<int64_t>(q_rows) * Hq * D;
  a.kv_bstride = static_cast<int64_t>(s_max) * Hkv * D;
  a.pos0 = cache_len;
  a.kv_len = kv_len;
  a.B = batch;
  a.Sq = q_rows;
  a.Sq_pad = static_cast<int32_t>(sq_pad);
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = g;
  a.hpw = g < 4 ? g : 4;
  a.hsubs = g / a.hpw;
  a.n_qtiles = static_cast<int32_t>(sq_pad / 64);
  a.n_kblocks = static_cast<int32_t>((kv_len + 127) / 128);
  a.causal = p->causal;
  a.accumulate = accumulate;
  a.grad_bf16 = grad_dtype == RLA_DT_BF16;
  a.c = score_scale(p);
  a.scale = p->softmax_scale;

  a.ws = static_cast<float*>(workspace);
  return hip_status(rla::launch_backward(a, p->out_dtype == RLA_DT_FP32, static_cast<hipStream_t>(hip_stream)),
                    "backward launch");
}

size_t rla_backward_workspace_bytes(const rla_attn_params* p, int32_t batch, int32_t q_rows) {
  if (check_params(p, true, nullptr) != RLA_OK || batch < 1 || q_rows < 1) return 0;
  const size_t sq_pad = (static_cast<size_t>(q_rows) + 63) / 64 * 64;
  return static_cast<size_t>(batch) * p->num_q_heads * 2 * sq_pad * sizeof(float);
}

size_t rla_lm_head_workspace_bytes(int32_t T, int32_t V) {
  if (T < 1 || V < 1) return 0;
  return rla::lm_head_scratch_floats(T, V) * sizeof(float);
}

rla_status rla_lm_head_logprobs(const void* x, rla_dtype x_dtype, const float* w, const int32_t* tokens, int32_t T,
                                int32_t H, int32_t V, float* logp, float* logz, void* workspace,
                                size_t workspace_bytes, void* hip_stream) {
  if (x == nullptr || w == nullptr || tokens == nullptr || logp == nullptr || workspace == nullptr)
    return fail(RLA_ERR_NULL_POINTER, "a required pointer is NULL");
  if (x_dtype != RLA_DT_BF16 && x_dtype != RLA_DT_FP32) return fail(RLA_ERR_UNSUPPORTED, "x_dtype=%d unsupported", x_dtype);
  if (T < 1 || H < 8 || H % 8 != 0 || V < 1)
    return fail(RLA_ERR_BAD_SHAPE, "need T>=1, H>=8 with H %% 8 == 0, V>=1 (got %d, %d, %d)", T, H, V);
  const size_t need = rla_lm_head_workspace_bytes(T, V);
  if (workspace_bytes < need)
    return fail(RLA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  rla::LmHeadArgs a;
  std::memset(&a, 0, sizeof a);
  a.x = x;
  a.w = w;
  a.tokens = tokens;
  a.logp = logp;
  a.logz = logz;
  a.T = T;
  a.H = H;
  a.V = V;
  a.part = static_cast<float*>(workspace);  // the launcher places zsel after the block partials
  return hip_status(rla::launch_lm_head(a, x_dtype == RLA_DT_FP32, static_cast<hipStream_t>(hip_stream)),
                    "lm_head launch");
}

rla_status rla_merge_states(const rla_attn_params* p, const rla_partials* parts, void* out, float* lse,
                            void* hip_stream) {
  rla_status st = check_params(p, false, nullptr);
  if (st != RLA_OK) return st;
  if (parts == nullptr || parts->out == nullptr || parts->lse == nullptr || parts->global_block_index == nullptr ||
      out == nullptr || lse == nullptr)
    return fail(RLA_ERR_NULL_POINTER, "a required pointer is NULL");
  if (parts->n_parts < 1 || parts->n_parts > RLA_MAX_PARTS)
    return fail(RLA_ERR_BAD_SHAPE, "n_parts=%d outside [1, %d]", parts->n_parts, RLA_MAX_PARTS);
  if (parts->rows < 1) return fail(RLA_ERR_BAD_SHAPE, "rows must be >= 1");
  const int n = parts->n_parts;
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  const int64_t* gbi = parts->global_block_index;
  std::stable_sort(order.begin(), order.end(), [gbi](int x, int y) { return gbi[x] < gbi[y]; });
  for (int i = 1; i < n; ++i)
    if (gbi[order[i]] == gbi[order[i - 1]])
      return fail(RLA_ERR_DUPLICATE_BLOCK, "global_block_index %lld appears twice", (long long)gbi[order[i]]);
  if (p->merge_order == RLA_ORDER_ARRIVAL)
    for (int i = 0; i < n; ++i) order[i] = i;

  rla::FoldArgs f;
  std::memset(&f, 0, sizeof f);
  f.part_out = parts->out;
  f.part_lse = parts->lse;
  f.out = out;
  f.lse = lse;
  f.rows = parts->rows;
  f.Hq = p->num_q_heads;
  f.n_parts = n;
  for (int i = 0; i < n; ++i) f.order[i] = static_cast<uint16_t>(order[i]);
  hipError_t e = rla::launch_fold(f, false, p->out_dtype == RLA_DT_FP32, static_cast<hipStream_t>(hip_stream));
  return hip_status(e, "merge launch");
}

}  // extern "C"
