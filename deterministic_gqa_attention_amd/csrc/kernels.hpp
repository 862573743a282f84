// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Plain structs passed by value as kernel arguments; all pointers are device
// pointers.  Tensors are bf16 bit patterns (uint16_t) unless noted.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rla {

constexpr int kHeadDimPublic = 128;  // the only head dimension the kernels implement
constexpr int kMaxParts = 512;  // partial states per merge / owned blocks per emit launch
constexpr int kDecodeUnitBlocks = 4;  // KV blocks of one decode tail unit
constexpr int kDecodeIdsCap = 2048;   // page ids one decode workgroup stages (bounds its head unit)
constexpr int kDecodeStageHeads = 8;  // q heads per group a tail unit stages in LDS (the largest group accepted)

// Prefill and chunked prefill.  Query row t of batch b sits at absolute
// position pos0 + t; it attends keys [0, kv_len) (and key <= position when
// causal).  Layouts: q rows at q + b*q_bstride + (t*Hq + h)*D; keys at
// k + b*kv_bstride + (key*Hkv + hk)*D; outputs out/lse as [B][Sq][Hq](D).
struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* out;                 // bf16 or fp32 [B][Sq][Hq][D] (fused mode)
  float* lse;                // [B][Sq][Hq] (fused mode)
  float* part_out;           // emit mode: [n_emit][B*Sq][Hq][D]
  float* part_lse;           // emit mode: [n_emit][B*Sq][Hq]
  int64_t q_bstride;         // elements between batches of q
  int64_t kv_bstride;        // elements between batches of k / v
  int64_t pos0;
  int64_t kv_len;
  int32_t B, Sq, Hq, Hkv, G;
  int32_t heads_per_wg;      // q heads of one group handled by one workgroup
  int32_t pos_groups;        // 32-row position groups per workgroup
  int32_t hsubs;             // workgroups needed to cover one group's heads
  int32_t n_ptiles;          // position tiles of 32*pos_groups rows
  int32_t causal;
  float c;                   // softmax_scale * log2(e), rounded to fp32
  const int32_t* page_table; // paged mode: [B][max_pages] page ids; k and v are the pools
  int64_t num_pages;         // paged mode: pages in each pool [num_pages][Hkv][P][D]
  int32_t log2_P;            // paged mode: log2 of the page size (P >= 4)
  int32_t max_pages;         // paged mode: table row length
  int32_t n_emit;            // emit mode: number of owned blocks
  uint16_t emit_blocks[kMaxParts];
};

// Sequences whose lengths (and unit prefix sums) travel with the decode
// launches instead of being read from device memory.
constexpr int kDecodeTableSeqs = 256;

// How a decode launch finds each sequence's length and each workgroup's unit.
enum DecodeLenMode : int32_t {
  kLensDevice = 0,   // ctx_lens in device memory; grid Bd x max_units, idle units exit
  kLensUniform = 1,  // every sequence has uniform_len keys; grid of exactly the units needed
  kLensTable = 2,    // lens[] / unit_start[] below; grid of exactly the units needed
};

// Paged decode, pass 1: one workgroup per (kv head, unit of consecutive KV
// blocks of one sequence).  Each sequence has one head unit, blocks
// [0, min(nb, head_blocks)), which folds its blocks' partial states in
// registers from the empty state and writes either the final output (the
// head covers the sequence) or the running state; then tail units of up to
// unit_blocks blocks each write every block's partial state for the group's
// q heads.  The grid holds every head unit first (Bd per kv head; with the
// length table, longest sequence first, so the long heads start together and
// the short ones leave room for tails early), then the tail units.
struct DecodeArgs {
  const uint16_t* q;          // [Bd][Hq][D]
  const uint16_t* k_pool;     // [num_pages][Hkv][P][D]
  const uint16_t* v_pool;
  const int32_t* page_table;  // [Bd][max_pages]; null: page i of sequence s is s*max_pages + i
  const int32_t* ctx_lens;    // [Bd] (kLensDevice only)
  float* items_out;           // [Bd][max_blocks][Hq][D]; a head's running acc in block slot 0
  float* items_lse;           // [Bd][max_blocks][Hq]; a head's running m, l in block slots 0, 1
  void* out;                  // [Bd][Hq][D] bf16 or fp32: written by head units that cover their sequence
  float* lse;                 // [Bd][Hq]
  int64_t num_pages;
  int32_t P, max_pages, Bd, Hq, Hkv, G, max_blocks, len_cap;
  int32_t log2_P;             // page size is a power of two (it divides the block)
  int32_t unit_blocks;        // KV blocks per tail unit
  int32_t head_blocks;        // KV blocks of a head unit (at most kDecodeIdsCap * P / block)
  int32_t len_mode;           // DecodeLenMode
  int64_t n_units;            // units in the grid (per kv head): Bd heads, then the tails
  int32_t uniform_len;        // kLensUniform: context length of every sequence
  float c;
  int32_t lens[kDecodeTableSeqs];            // kLensTable: length of sequence s (validated, <= len_cap)
  int32_t unit_start[kDecodeTableSeqs + 1];  // kLensTable: first tail unit of sequence s; [Bd] = all tails
  int16_t head_order[kDecodeTableSeqs];     // kLensTable: sequence of head unit u (longest first)
};

// Fold of per-block partial states in ascending block order (decode pass 2)
// or in a given order over an explicit list of parts (merge).
struct FoldArgs {
  const float* part_out;      // merge: [n_parts][rows][Hq][D]; decode: items
  const float* part_lse;
  const int32_t* ctx_lens;    // decode, kLensDevice: [Bd] (block count per row); merge: null
  int32_t uniform_len;        // decode, kLensUniform: length of every row
  int32_t len_mode;           // decode: DecodeLenMode (kLensTable: lens[] below)
  void* out;                  // [rows][Hq][D] bf16 or fp32
  float* lse;                 // [rows][Hq]
  int64_t rows;
  int32_t Hq;
  int32_t n_parts;            // merge: parts to fold; decode: max_blocks
  int32_t block;              // decode: keys per block; merge: unused
  int32_t head_blocks;        // decode: blocks folded by each sequence's head unit
  int32_t len_cap;            // decode: clamp on context lengths
  uint16_t order[kMaxParts];  // merge: part indices in fold order
  int32_t lens[kDecodeTableSeqs];  // decode, kLensTable: length of row s
};

// Backward (dQ, dK, dV of Out).  Query row t of batch b sits at position
// pos0 + t and attends keys [0, kv_len) (key <= position when causal).
// q, out, dout, dq share q's layout (b*q_bstride + (t*Hq + h)*D); k, v, dk, dv
// share k's layout (b*kv_bstride + (key*Hkv + hk)*D).  ws: [B][Hq][2][Sq_pad]
// scratch (LSE*log2 e, then Delta, per row).
struct BackwardArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* out;           // forward Out, bf16 or fp32
  const float* lse;          // forward LSE [B][Sq][Hq], natural log
  const uint16_t* dout;      // gradient of Out, bf16
  float* ws;
  void* dq;                  // fp32 or bf16 (grad_bf16)
  void* dk;                  // fp32 (read first when accumulate is set) or bf16
  void* dv;
  int64_t q_bstride;
  int64_t kv_bstride;
  int64_t pos0;
  int64_t kv_len;
  int32_t B, Sq, Sq_pad, Hq, Hkv, G;
  int32_t hpw;               // dQ kernel: q heads per workgroup (min(G, 4))
  int32_t hsubs;             // dQ kernel: workgroups per group (G / hpw)
  int32_t n_qtiles;          // ceil(Sq / 64)
  int32_t n_kblocks;         // dK/dV kernel: ceil(kv_len / 128)
  int32_t causal;
  int32_t accumulate;
  int32_t grad_bf16;         // write dQ/dK/dV as bf16 (RNE of the fp32 result); never with accumulate
  float c;                   // softmax_scale * log2(e), rounded to fp32
  float scale;               // softmax_scale
};

// Selected log-probabilities through an FP32 lm_head: x [T][H] (bf16 or
// fp32), w [V][H] fp32, tokens [T]; part [T][n_vblocks][2] and zsel [T] are
// scratch; logp [T], logz [T] (may be null) outputs.
struct LmHeadArgs {
  const void* x;
  const float* w;
  const int32_t* tokens;
  float* part;
  float* zsel;
  float* logp;
  float* logz;
  int32_t T, H, V;
  int32_t n_vblocks;   // vocabulary blocks (set by launch_lm_head)
  int32_t n_tgroups;   // token groups (set by launch_lm_head)
};

hipError_t launch_prefill(const PrefillArgs& a, int block, bool out_f32, bool emit, hipStream_t s);
// Scratch floats launch_lm_head needs for T tokens over V rows (part + zsel).
size_t lm_head_scratch_floats(int T, int V);
hipError_t launch_lm_head(LmHeadArgs a, bool x_f32, hipStream_t s);
// The dQ and dK/dV launches of the backward, in that order on s.
hipError_t launch_backward(const BackwardArgs& a, bool out_f32, hipStream_t s);
// Fused prefill with K/V gathered from paged pools (a.page_table etc. set).
hipError_t launch_prefill_paged(const PrefillArgs& a, int block, bool out_f32, hipStream_t s);
hipError_t launch_decode_items(const DecodeArgs& a, int block, bool out_f32, hipStream_t s);
// Size of the fixed device array behind rla_attn_decode_paged_static: the
// decode items of 64 sequences of 16384 keys with 32 q heads (129 MiB) fit.
constexpr size_t kStaticDecodeScratchBytes = size_t{132} << 20;
// Device address of that array on the current device (looked up once per
// device); null with *err set on failure.
void* static_decode_scratch(hipError_t* err);
hipError_t launch_fold(const FoldArgs& a, bool decode, bool out_f32, hipStream_t s);

}  // namespace rla
