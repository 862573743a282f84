/*
 * rla_attn.h — C ABI of the deterministic grouped-query attention library for
 * AMD MI355X (gfx950), librla_attn.so.
 *
 * What it computes.  Forward attention for grouped-query heads (q head h reads
 * kv head h / (Hq / Hkv)) on post-RoPE bf16 inputs, with FP32 accumulation,
 * per-KV-block partial states (out_i, lse_i) that are combined in ascending
 * global block index, and a downcast to bf16 only at the final write.  The
 * pages that specify it: "WS2 Attention PR5 Drift Benchmark" (sections
 * "Scope": Qwen3-8B target Hq=32, Hkv=8, D=128, TP head shards, CP=1/2, full
 * and chunked prefill, BF16 path vs FP32 reference; "Transformer Engine
 * Reuse": partial state = (out_i, lse_i, global_block_index_i), sorted by
 * global_block_index before the online-softmax correction; "Report Contract":
 * merge order always global_block_index, downcast at the final write) and
 * "[WS2][Attention] H100 validation and reproduction guide for #235 PR1-PR8"
 * (sections "Status": FP32 accumulation, fixed merge order, final-write
 * downcast, no split-KV; "Acceptance": Out and attention-domain LSE,
 * bitwise-equal results).
 *
 * Because every (query row, KV block) partial state is computed with the same
 * operations wherever it is computed, and the fold over blocks always runs in
 * ascending block index, the results are bit-identical across batch
 * composition, chunk size, page placement, context-parallel split and the
 * arrival order of partial states.
 *
 * Conventions (all entry points):
 *  - Tensors are device pointers, caller-owned, contiguous, token-major:
 *    q / out [batch][tokens][Hq][128], k / v [batch][tokens][Hkv][128],
 *    lse [batch][tokens][Hq] (fp32, natural log).  bf16 tensors are passed as
 *    raw 16-bit patterns.  Pointers marked [host] are host memory.
 *  - head_dim must be 128; kv_block_size 64 or 128; Hq % Hkv == 0 with
 *    Hq / Hkv in {1, 2, 4, 8}; acc_dtype must be RLA_DT_FP32.
 *  - Every argument is validated on the host before anything is launched; a
 *    rejected call writes nothing and returns an error code (no fallback).
 *    rla_last_error() then describes the failure (thread-local).
 *  - Work is enqueued on `hip_stream` (a hipStream_t, NULL = default stream)
 *    and is asynchronous; device faults surface at the caller's synchronize.
 *    A launch failure returns RLA_ERR_HIP.
 *  - No call allocates device memory: scratch space is caller-provided device
 *    memory whose size the matching rla_*_workspace_bytes query returns; a
 *    workspace smaller than that is rejected with RLA_ERR_WORKSPACE_TOO_SMALL
 *    before anything is enqueued.
 *  - Thread safety: stateless apart from the thread-local error string.
 *  - Empty rows (no visible key) give Out = 0 and LSE = -inf.
 */
#ifndef RLA_ATTN_H
#define RLA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RLA_OK = 0,
  RLA_ERR_NULL_POINTER = 1,
  RLA_ERR_BAD_SHAPE = 2,
  RLA_ERR_UNSUPPORTED = 3,
  RLA_ERR_DUPLICATE_BLOCK = 4,
  RLA_ERR_WORKSPACE_TOO_SMALL = 5,
  RLA_ERR_HIP = 6
} rla_status;

typedef enum { RLA_DT_BF16 = 0, RLA_DT_FP32 = 1 } rla_dtype;

/* Order in which partial states are folded.  GLOBAL_BLOCK_INDEX is the
 * contract ("WS2 Attention PR5 Drift Benchmark", "Report Contract").  ARRIVAL
 * folds in the order given and exists only as a diagnostic for
 * rla_merge_states (it shows the drift that sorting removes); the attention
 * entry points accept GLOBAL_BLOCK_INDEX only. */
typedef enum { RLA_ORDER_GLOBAL_BLOCK_INDEX = 0, RLA_ORDER_ARRIVAL = 1 } rla_merge_order;

/* Largest number of partial states one rla_merge_states call folds, and of
 * blocks one emit-mode prefill call owns. */
#define RLA_MAX_PARTS 512

typedef struct {
  int32_t num_q_heads;   /* local head shard: TP changes only these two counts  */
  int32_t num_kv_heads;
  int32_t head_dim;      /* must be 128                                          */
  int32_t kv_block_size; /* 64 or 128 keys: the merge unit; block i holds keys
                            [i*kv_block_size, (i+1)*kv_block_size) counted from
                            sequence position 0                                  */
  float softmax_scale;   /* applied in fp32 to the fp32 dot product              */
  int32_t causal;        /* prefill/chunked: 1 = key position <= query position;
                            decode: ignored (the query sees all cached keys)      */
  int32_t merge_order;   /* rla_merge_order                                      */
  int32_t acc_dtype;     /* must be RLA_DT_FP32                                  */
  int32_t out_dtype;     /* RLA_DT_BF16 (downcast at final write) or RLA_DT_FP32 */
} rla_attn_params;

/* Partial states: the pages' state_i = (out_i, lse_i, global_block_index_i)
 * for every row, one part per KV block ("Transformer Engine Reuse").
 * out_i is normalised by the block's own sum; lse_i is that block's natural
 * log-sum-exp; an empty block for a row is (0, -inf). */
typedef struct {
  float* out;                         /* [n_parts][rows][Hq][128] fp32, device */
  float* lse;                         /* [n_parts][rows][Hq] fp32, device      */
  const int64_t* global_block_index;  /* [host][n_parts], arrival order        */
  int32_t n_parts;                    /* 1 .. RLA_MAX_PARTS                     */
  int64_t rows;                       /* rows per part (batch * tokens)         */
} rla_partials;

/* Emulated context-parallel shard: a set of global KV blocks whose partial
 * states are written instead of folded, for the query rows
 * [q_begin, q_begin + q_count) of every sequence.  Part p of `partials`
 * receives block kv_blocks[p] for rows b*q_count + (t - q_begin).  The caller
 * sets partials->global_block_index (typically to kv_blocks) for the merge. */
typedef struct {
  const int64_t* kv_blocks;           /* [host][n_kv_blocks], distinct ids     */
  int32_t n_kv_blocks;                /* 1 .. RLA_MAX_PARTS                     */
  int64_t q_begin;                    /* query slab start (chunk-relative row)  */
  int64_t q_count;                    /* query slab length                      */
  rla_partials* partials;             /* out [n_kv_blocks][batch*q_count][Hq][128],
                                         lse [n_kv_blocks][batch*q_count][Hq]  */
} rla_shard;

/* Full (causal) prefill over `batch` sequences of `seq_len` tokens ("WS2
 * Attention PR5 Drift Benchmark", section "Scope": full prefill of the
 * Qwen3-8B attention shape on post-RoPE Q/K, CP=1 or CP=2; "Transformer
 * Engine Reuse": one partial state per KV block, merged in global block index
 * order).
 * q [batch][seq_len][Hq][128], k, v [batch][seq_len][Hkv][128] bf16, post-RoPE.
 * shard == NULL: fused path, writes out [batch][seq_len][Hq][128] (bf16 or fp32
 * per out_dtype) and lse [batch][seq_len][Hq].  shard != NULL: emit path, writes
 * the shard's partial states; out and lse are ignored (may be NULL). */
rla_status rla_attn_prefill(const rla_attn_params* p, const void* q, const void* k, const void* v,
                            int32_t batch, int32_t seq_len, const rla_shard* shard, void* out,
                            float* lse, void* hip_stream);

/* Chunked-prefill replay step ("Scope": chunked-prefill replay).  The chunk's
 * query i sits at absolute position cache_len + i and attends the cached keys
 * [0, cache_len + chunk_len) (causally); the chunk's own K/V must already be in
 * the caches at positions [cache_len, cache_len + chunk_len).
 * q_chunk [batch][chunk_len][Hq][128]; k_cache, v_cache [batch][s_max][Hkv][128];
 * out [batch][chunk_len][Hq][128], lse [batch][chunk_len][Hq].
 * Requires cache_len >= 0, chunk_len >= 1, cache_len + chunk_len <= s_max.
 * shard as in rla_attn_prefill (q_begin/q_count relative to the chunk).
 * A chunk of one query without a shard runs as a decode step (the cache read
 * as a pool of one-key pages: KV blocks spread over many workgroups, block
 * items folded in order); its block items go to `workspace`, which must hold
 * rla_chunked_workspace_bytes(p, batch, chunk_len, cache_len, s_max) bytes of
 * device memory (RLA_ERR_WORKSPACE_TOO_SMALL otherwise; contents on return
 * unspecified).  Every other call needs no workspace (it may be NULL, size 0).
 * The result bits do not depend on the route. */
rla_status rla_attn_prefill_chunked(const rla_attn_params* p, const void* q_chunk, const void* k_cache,
                                    const void* v_cache, int32_t batch, int32_t chunk_len,
                                    int32_t cache_len, int32_t s_max, const rla_shard* shard, void* workspace,
                                    size_t workspace_bytes, void* out, float* lse, void* hip_stream);

/* Workspace bytes rla_attn_prefill_chunked needs without a shard: the decode
 * workspace of `batch` sequences of cache_len + 1 keys for a chunk of one
 * query, else 0 (also 0 on invalid arguments). */
size_t rla_chunked_workspace_bytes(const rla_attn_params* p, int32_t batch, int32_t chunk_len, int32_t cache_len,
                                   int32_t s_max);

/* Paged chunked prefill ("Commands": paged prefill/decode with batch and
 * page-layout invariance): rla_attn_prefill_chunked with the keys gathered
 * through a page table instead of read from a contiguous cache.  Query i of
 * the chunk sits at position cache_len + i and attends keys [0, cache_len + i]
 * (causal; all cache_len + chunk_len keys when p->causal == 0); key j of
 * sequence b is slot j % page_size of page page_table[b][j / page_size].
 * q_chunk [batch][chunk_len][Hq][128] bf16; k_pool, v_pool
 * [num_pages][Hkv][page_size][128] bf16 already holding the chunk's keys;
 * page_table [batch][max_pages_per_seq] int32 (device).  page_size must be a
 * power of two with 4 <= page_size <= kv_block_size (one load instruction
 * covers 4 consecutive keys of one page), max_pages_per_seq * page_size
 * must cover cache_len + chunk_len, and cache_len + chunk_len <= 2^30.  A page id outside [0, num_pages) is
 * clamped into that range before use, so a bad table cannot fault, but its
 * result is unspecified.  The result is bit for bit that of
 * rla_attn_prefill_chunked over the same keys, whatever the page layout.
 * out [batch][chunk_len][Hq][128] (bf16 or fp32), lse [batch][chunk_len][Hq]. */
rla_status rla_attn_prefill_paged(const rla_attn_params* p, const void* q_chunk, const void* k_pool,
                                  const void* v_pool, int64_t num_pages, int32_t page_size,
                                  const int32_t* page_table, int32_t max_pages_per_seq, int32_t batch,
                                  int32_t chunk_len, int32_t cache_len, void* out, float* lse,
                                  void* hip_stream);

/* Paged-KV decode ("Commands": paged prefill/decode with batch and page-layout
 * invariance): one query token per sequence attending its cached keys
 * [0, context_lens[s]).  Key j of sequence s is slot j % page_size of page
 * page_table[s][j / page_size] in the pools.
 * q [batch][Hq][128]; k_pool, v_pool [num_pages][Hkv][page_size][128] bf16;
 * page_table [batch][max_pages_per_seq] int32 (device); context_lens [batch]
 * int32 (device).  host_context_lens [host][batch] may be NULL; when given it
 * must hold the same lengths as context_lens.  It is validated against
 * max_context_len and the table width before anything is enqueued, and for
 * batch <= 256 the kernels take every length from it (the lengths and the
 * per-sequence workgroup offsets travel with the launches, context_lens is not
 * read) and cover exactly the blocks it needs.  Without it, or above 256
 * sequences, the kernels read context_lens and the launch covers every block
 * up to max_context_len, idle workgroups exiting.  The results are the same
 * bits either way.  page_size must divide kv_block_size.  Lengths above
 * min(max_context_len, max_pages_per_seq*page_size) are clamped to it, and a
 * page id outside [0, num_pages) is clamped into that range before use, so a
 * bad table cannot fault, but its result is unspecified.
 * workspace: at least rla_decode_workspace_bytes(p, batch, max_context_len)
 * bytes of device memory (per-block partial states); contents on return are
 * unspecified.  out [batch][Hq][128], lse [batch][Hq]. */
rla_status rla_attn_decode_paged(const rla_attn_params* p, const void* q, const void* k_pool,
                                 const void* v_pool, int64_t num_pages, int32_t page_size,
                                 const int32_t* page_table, int32_t max_pages_per_seq,
                                 const int32_t* context_lens, const int32_t* host_context_lens,
                                 int32_t batch, int32_t max_context_len, void* workspace,
                                 size_t workspace_bytes, void* out, float* lse, void* hip_stream);

/* For callers that cannot allocate or provide device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * rla_attn_decode_paged without the workspace argument.  The block items go
 * to a fixed array inside the library, RLA_DECODE_STATIC_SCRATCH_BYTES of
 * device memory per GPU the library runs on, held until the process ends; a
 * call needing more (rla_decode_workspace_bytes above it) is rejected with
 * RLA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  The array is
 * shared by every call on one GPU: calls that overlap in time on one GPU
 * (different streams, different threads) race and give unspecified results;
 * calls ordered on one stream are safe.  It allocates nothing (the array's
 * device address is looked up once per device, on the first call there) and
 * gives the same bits as rla_attn_decode_paged. */
#define RLA_DECODE_STATIC_SCRATCH_BYTES ((size_t)132 << 20)
rla_status rla_attn_decode_paged_static(const rla_attn_params* p, const void* q, const void* k_pool,
                                        const void* v_pool, int64_t num_pages, int32_t page_size,
                                        const int32_t* page_table, int32_t max_pages_per_seq,
                                        const int32_t* context_lens, const int32_t* host_context_lens,
                                        int32_t batch, int32_t max_context_len, void* out, float* lse,
                                        void* hip_stream);

/* Merge of partial states ("Transformer Engine Reuse"; "Scope":
 * merge_order_probe).  With RLA_ORDER_GLOBAL_BLOCK_INDEX the parts are folded
 * in ascending global_block_index whatever their arrival order; a repeated
 * index returns RLA_ERR_DUPLICATE_BLOCK.  Uses merge_order, out_dtype and
 * num_q_heads of p.  out [rows][Hq][128] (bf16 or fp32), lse [rows][Hq]. */
rla_status rla_merge_states(const rla_attn_params* p, const rla_partials* parts, void* out, float* lse,
                            void* hip_stream);

/* Backward of (chunked) prefill: dQ, dK, dV of Out ("[WS2][Attention] H100
 * validation and reproduction guide", sections "PR stack": the prefill and
 * chunked-prefill backward leg; "Status" and "Acceptance": dQ, dK and dV
 * bitwise equal across decompositions).  The queries are those of
 * rla_attn_prefill_chunked: query i sits at position cache_len + i and attends
 * keys [0, cache_len + q_rows) (causally when p->causal); full prefill is
 * cache_len = 0, q_rows = s_max = seq_len.
 * Inputs (device, bf16 unless noted): q, dout [batch][q_rows][Hq][128];
 * k, v [batch][s_max][Hkv][128]; out [batch][q_rows][Hq][128], the forward
 * output in p->out_dtype (bf16 or fp32); lse [batch][q_rows][Hq] fp32, the
 * forward's natural-log LSE.  The gradient reaching LSE is taken as zero.
 * Outputs (device, grad_dtype: fp32, or bf16 = the round-to-nearest-even of
 * the fp32 result, the only rounding of the gradients): dq
 * [batch][q_rows][Hq][128]; dk, dv [batch][s_max][Hkv][128], written for keys
 * [0, cache_len + q_rows) only.
 * accumulate = 0: dk/dv are overwritten.  accumulate = 1 (fp32 only): this
 * call's contributions are added to the fp32 values already in dk/dv (which
 * the caller zero-fills before the first call): replaying the query rows as
 * consecutive chunks whose cache_len are multiples of 64 gives dq, dk and dv
 * bit for bit equal to one call over all rows.
 * Every element is one fixed-order FP32 MFMA accumulation (dK/dV: query tiles
 * of 64 rows in ascending order, q heads of the group in ascending order
 * inside a tile; dQ: keys in ascending order), so results do not depend on
 * the batch makeup or on scheduling.  P and dS are rounded to bf16 as MFMA
 * operands; dS includes softmax_scale.  kv_block_size is not used.
 * workspace: at least rla_backward_workspace_bytes(p, batch, q_rows) bytes of
 * device memory (per-row LSE and Delta, 8 bytes per query row and head, rows
 * padded to 64); contents on return unspecified. */
rla_status rla_attn_backward(const rla_attn_params* p, const void* q, const void* k, const void* v,
                             const void* out, const float* lse, const void* dout, int32_t batch,
                             int32_t q_rows, int32_t cache_len, int32_t s_max, int32_t accumulate,
                             rla_dtype grad_dtype, void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, void* hip_stream);

/* Workspace bytes rla_attn_backward needs (0 on invalid arguments). */
size_t rla_backward_workspace_bytes(const rla_attn_params* p, int32_t batch, int32_t q_rows);

/* Selected log-probability through an FP32 lm_head ("WS2 Attention PR5 Drift
 * Benchmark", section "Scope": both attention outputs of a drift comparison go
 * through the same deterministic synthetic FP32 lm_head and the active
 * tokens' selected log-probs are compared; "[WS2][Attention] H100 validation
 * and reproduction guide", section "Status": decode/prefill dlogp max abs 0.0).
 * For token t: z_tv = sum_h x[t][h] * w[v][h] (FP32 MFMA accumulation in a
 * fixed order over h), logz[t] = ln sum_v exp(z_tv) (per-32-row block max and
 * sum, folded in ascending block order), logp[t] = z_{t,tokens[t]} - logz[t].
 * x [T][H] device, bf16 bits (x_dtype RLA_DT_BF16) or fp32: typically an Out
 * tensor [T][Hq][128] read as H = Hq*128; w [V][H] fp32 device; tokens [T]
 * int32 device; logp [T] fp32 device; logz [T] fp32 device or NULL.  H must be
 * a positive multiple of 8.  A token id outside [0, V) gives logp = NaN.
 * A token's results do not depend on the other tokens of the call.
 * workspace: at least rla_lm_head_workspace_bytes(T, V) bytes of device memory
 * (per-block partial sums and the selected logits); contents on return
 * unspecified. */
rla_status rla_lm_head_logprobs(const void* x, rla_dtype x_dtype, const float* w, const int32_t* tokens,
                                int32_t T, int32_t H, int32_t V, float* logp, float* logz, void* workspace,
                                size_t workspace_bytes, void* hip_stream);

/* Workspace bytes rla_lm_head_logprobs needs: (ceil(V/32) * T * 2 + T) floats
 * (0 on invalid arguments). */
size_t rla_lm_head_workspace_bytes(int32_t T, int32_t V);

/* Workspace bytes rla_attn_decode_paged needs (0 on invalid arguments). */
size_t rla_decode_workspace_bytes(const rla_attn_params* p, int32_t batch, int32_t max_context_len);

/* Description of the last failure on the calling thread ("" after success). */
const char* rla_last_error(void);

/* Provenance string naming the arithmetic contract, e.g. "rla.attention.core.v1". */
const char* rla_core_id(void);

#ifdef __cplusplus
}
#endif

#endif /* RLA_ATTN_H */
