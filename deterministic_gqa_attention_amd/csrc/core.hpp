// Canonical arithmetic of the deterministic attention core (gfx950).
//
// Every kernel of the library includes this header and computes each
// (query row, KV block) partial state and each merge step with exactly the
// operations written here, in this order.  That is what makes the result
// independent of how work is cut up (batch makeup, chunk size, page layout,
// context-parallel split, arrival order of partial states): the pages
// ("WS2 Attention PR5 Drift Benchmark", sections "Scope" and "Transformer
// Engine Reuse"; "[WS2][Attention] H100 validation and reproduction guide",
// section "Status") require FP32 accumulation, per-block partial states
// (out_i, lse_i, global_block_index_i) merged in ascending global block index,
// and a downcast to bf16 only when the final output is written.
//
// The contract, per query row q and KV block b (keys [b*Bk, (b+1)*Bk) counted
// from sequence position 0):
//   dot_j = MFMA bf16 chain over D in 8 fixed 16-wide steps, FP32 accumulate;
//           masked keys -> -inf (select)
//   m_t   = fl(max_j dot_j * c) with c = fl32(scale * log2 e)  (block max in
//           the log2 domain; equal to max_j fl(dot_j * c) since c > 0)
//   p_j   = 2^fma(dot_j, c, -m_t)                (v_exp_f32)
//   l_b   = fixed tree over the 16 values a lane holds per 32-key sub-tile,
//           plus its partner lane, then a fixed tree over the sub-tiles
//   acc_b = MFMA chain over the block's keys from zero, P rounded to bf16
//           (FP32-output mode: P = hi + lo, two MFMAs per key step)
//   O_b   = acc_b * r_b with r_b = v_rcp_f32(l_b) (within 1 ulp of 1 / l_b);
//           L_b = (m_t + log2 l_b) * ln 2
//   empty row (no unmasked key) -> (O_b, L_b) = (0, -inf)
// Fold over blocks in ascending index from the empty state (m, l, acc) =
// (-inf, 0, 0), with a lazily moved reference m (tau = 8, natural-log units).
// Every step is acc = fma(O_b, beta, acc * alpha) with:
//   empty item (L_b = -inf):  alpha = 1, beta = 0          (state unchanged)
//   first non-empty item:     alpha = 1, beta = 1, m = L_b, l = 1
//   L_b <= m + tau ("add"):   alpha = 1, beta = e^(L_b - m), l = l + beta
//   L_b >  m + tau ("move"):  alpha = e^(m - L_b), beta = 1,
//                             l = l*alpha + 1, m = L_b
//   (acc * 1 is exact, so a kernel may skip that multiply when no lane of the
//   wave moves; weights stay below e^tau, so nothing overflows, and the
//   reference moves only on large jumps, so almost every step is one fma)
// Finalize: O = acc * (1 / l), LSE = m + log2(l) * ln 2 (natural log);
//           no item at all -> (0, -inf).
// The library is compiled with -ffp-contract=off, so no multiply-add is fused
// unless written as fmaf() here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kDSteps = kHeadDim / 16;     // MFMA steps over the head dimension
constexpr int kDTiles = kHeadDim / 32;     // 32-row output tiles over the head dimension
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
// e^x as used by the fold: one rounding for the scaling, then v_exp_f32.
__device__ __forceinline__ float fold_exp(float x) { return hw_exp2(x * kLog2e); }

// Block max in the log2 domain from the max raw dot (-inf when the row has no
// visible key in the block), and the offset used by the exponentials (0 for
// an empty row, so masked scores give exactly 0 instead of NaN).
__device__ __forceinline__ float block_m(float max_dot, float c) {
  return max_dot == kNegInf ? kNegInf : max_dot * c;
}
__device__ __forceinline__ float block_m_use(float m_t) { return m_t == kNegInf ? 0.0f : m_t; }
// Unnormalised probability of a (masked-to--inf) raw dot.
__device__ __forceinline__ float block_p(float dot, float c, float m_use) { return hw_exp2(fmaf(dot, c, -m_use)); }

// v_mfma_f32_32x32x16_bf16.  A is 32 (rows) x 16 (k), B is 16 (k) x 32 (cols).
// Lane l supplies A row l%32 and B column l%32, k values 8*(l/32)+0..7 of the
// step; accumulator register v of lane l is row 8*(v/4) + 4*(l/32) + v%4,
// column l%32.
__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int v, int half) { return 8 * (v >> 2) + 4 * half + (v & 3); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// fp32 -> bf16 round-to-nearest-even (v_cvt_pk_bf16_f32), two values per word.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Combine a value with the one held by the lane 32 apart (same accumulator
// column, other row half) without going through LDS: v_permlane32_swap swaps
// the upper half of one register with the lower half of another, so with two
// copies of x every lane ends up holding {x[l mod 32], x[l mod 32 + 32]}.
// max and + are commutative, so both halves get the same bits.  (Inline asm:
// the compiler builtin for this instruction returns only one of its two
// results.  The leading s_nop covers a VALU write of the operands just before.)
__device__ __forceinline__ void lane_pair(float x, float& lo, float& hi) {
  uint32_t a = __builtin_bit_cast(uint32_t, x);
  uint32_t b = a;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo = __builtin_bit_cast(float, a);
  hi = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float pair_max(float x) {
  float a, b;
  lane_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  lane_pair(x, a, b);
  return a + b;
}

// Canonical sum of the 16 values one lane holds for one 32-key sub-tile:
// a fixed pairwise tree in register order.
__device__ __forceinline__ float tree16(const f32x16& p) {
  float a0 = p[0] + p[1], a1 = p[2] + p[3], a2 = p[4] + p[5], a3 = p[6] + p[7];
  float a4 = p[8] + p[9], a5 = p[10] + p[11], a6 = p[12] + p[13], a7 = p[14] + p[15];
  float b0 = a0 + a1, b1 = a2 + a3, b2 = a4 + a5, b3 = a6 + a7;
  return (b0 + b1) + (b2 + b3);
}

// Canonical combination of the per-sub-tile sums (each already including the
// partner lane) into the block sum l_b.
template <int NKT>
__device__ __forceinline__ float combine_subtiles(const float* s) {
  static_assert(NKT == 2 || NKT == 4, "block must be 64 or 128 keys");
  if constexpr (NKT == 2) {
    return s[0] + s[1];
  } else {
    return (s[0] + s[1]) + (s[2] + s[3]);
  }
}

// Block item scalars from the block max (log2 domain) and block sum.
struct ItemScalars {
  float r;    // v_rcp_f32(l_b) (1 ulp), or 0 for an empty row
  float L;    // natural-log LSE of the block, or -inf for an empty row
};
__device__ __forceinline__ ItemScalars item_scalars(float m_t, float l_b) {
  ItemScalars s;
  if (m_t == kNegInf) {
    s.r = 0.0f;
    s.L = kNegInf;
  } else {
    s.r = __builtin_amdgcn_rcpf(l_b);
    float lg = hw_log2(l_b);
    float t = m_t + lg;
    s.L = t * kLn2;
  }
  return s;
}
// O_b element; an empty row gives exactly 0 (acc_b is 0 there).
__device__ __forceinline__ float item_out(float acc_b, const ItemScalars& s) { return acc_b * s.r; }

// Running fold state of one row.
struct FoldState {
  float m;  // running max of the item LSEs (natural log); -inf while empty
  float l;  // running sum of exp(L_i - m)
};

// Distance (natural log) the block LSE must exceed the reference by before
// the reference moves.
constexpr float kFoldTau = 8.0f;

struct FoldStep {
  float alpha;  // "move": e^(m_old - L); else 1
  float beta;   // "add": e^(L - m); "move", first item: 1; empty item: 0
  bool move;
};

// Scalar part of one fold step (updates m and l), with every case computed
// as a select rather than a branch: the one exponential takes (m - L) for a
// move and (L - m) otherwise, and each case picks its results from it.  The
// step sits on the dependent chain of every sequential fold (the fused
// prefill kernel, a decode head unit, the fold pass), which branches lengthen.
__device__ __forceinline__ FoldStep fold_scalars(FoldState& st, float L) {
  const bool empty = L == kNegInf;
  const bool first = !empty && st.m == kNegInf;
  const bool mv = !empty && !first && L > st.m + kFoldTau;
  const bool add = !empty && !first && !mv;
  const float x = mv ? st.m : L;
  const float y = mv ? L : st.m;
  const float e = fold_exp(x - y);  // unused (and possibly not finite) for empty and first
  const float la = st.l * e;
  FoldStep f;
  f.move = mv;
  f.alpha = mv ? e : 1.0f;                            // move: e^(m - L)
  f.beta = empty ? 0.0f : (add ? e : 1.0f);           // add: e^(L - m)
  const float l_add = st.l + e;                       // add: l + beta
  const float l_move = la + 1.0f;                     // move: l * alpha + 1
  st.l = first ? 1.0f : (mv ? l_move : (add ? l_add : st.l));
  st.m = (first || mv) ? L : st.m;
  return f;
}

// Element part of one fold step.
__device__ __forceinline__ float fold_elem(const FoldStep& f, float acc, float o) {
  return fmaf(o, f.beta, acc * f.alpha);
}
// The same when alpha == 1 (no lane of the wave moves): acc * 1 is exact.
__device__ __forceinline__ float fold_elem_nomove(const FoldStep& f, float acc, float o) {
  return fmaf(o, f.beta, acc);
}

// Finalize scalars: O = acc * r, LSE natural log.
struct Final {
  float r;
  float lse;
};
__device__ __forceinline__ Final finalize(const FoldState& st) {
  Final f;
  if (st.m == kNegInf) {
    f.r = 0.0f;
    f.lse = kNegInf;
  } else {
    f.r = 1.0f / st.l;
    float lg = hw_log2(st.l);
    float t = lg * kLn2;
    f.lse = st.m + t;
  }
  return f;
}

}  // namespace rla
