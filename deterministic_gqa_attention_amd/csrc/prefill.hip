// Prefill / chunked-prefill kernels for gfx950: fused mode (fold every KV
// block of the row in ascending global block index and write Out/LSE) and
// emit mode (write the per-block partial states of a set of owned blocks,
// which is how a context-parallel shard is emulated on one GPU).
//
// Work decomposition: a workgroup of 8 waves (two per SIMD) takes one kv head
// hk of one batch row and a tile of query positions; each wave owns 32
// consecutive positions of one q head of the group (an MFMA column tile).
// Each KV block is staged in LDS once per workgroup by direct global->LDS
// loads and read by all waves.
//
// Per wave and block there are four phases:
//   scores   S^T = K Q^T                      (matrix cores, K from LDS)
//   softmax  mask, max, p, sum, bf16 P        (vector ALU)
//   pv       acc_b = V^T P^T per dim tile     (matrix cores, V from LDS)
//   fold     O_b = acc_b / l_b into the running state (vector ALU)
// with the operations of core.hpp.  The bf16-output kernel
// (prefill_pp_kernel, contiguous and paged caches) runs the two halves of
// the workgroup one stage apart (ping-pong), so on every SIMD a scores stage
// (matrix cores) overlaps a softmax + PV + fold stage (vector ALU) of the
// other wave.  The fp32-output kernel runs scores | softmax | pv+fold one
// after the other.  K/V blocks arrive by direct buffer->LDS loads; each
// kernel names the buffer being read and the buffer being filled as separate
// arrays (or restrict pointers), so the compiler knows they do not overlap
// and never stalls an LDS read on the in-flight loads (it would otherwise
// wait for every outstanding direct load before the first read).  No atomics and no split
// of a block across workgroups, so nothing depends on scheduling.
#include <type_traits>

#include "kernels.hpp"
#include "tile.hpp"

namespace rla {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

// ---------------------------------------------------------------- phases --

// S^T = K Q^T for one staged block: NKT sub-tiles of 32 keys x 32 queries.
// K fragments are read one head-dim step ahead.
// (lane: this lane's index, passed in so a caller can make it opaque)
template <int BK>
__device__ __forceinline__ void block_scores(const char* kreg, const bf16x8 (&qf)[kDSteps], f32x16 (&s)[BK / 32],
                                             int lane = static_cast<int>(threadIdx.x & 63)) {
  constexpr int NKT = BK / 32;
  const KReads<BK> kr(kreg, lane);
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) s[kt] = f32x16{};
  bf16x8 kf[2][NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) kf[0][kt] = kr.frag(kt, 0);
#pragma unroll
  for (int ds = 0; ds < kDSteps; ++ds) {
    if (ds + 1 < kDSteps) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) kf[(ds + 1) & 1][kt] = kr.frag(kt, ds + 1);
    }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) s[kt] = mfma(kf[ds & 1][kt], qf[ds], s[kt]);
    sched_fence();
  }
}

// The same one key sub-tile at a time (each sub-tile's chain over the head
// dimension in the same order, so the same bits), with K fragments read R-1
// MFMAs ahead through a ring of R registers, from prebuilt fragment addresses.
template <int BK, int R>
__device__ __forceinline__ void block_scores_kr(const KReads<BK>& kr, const bf16x8 (&qf)[kDSteps],
                                                f32x16 (&s)[BK / 32]) {
  constexpr int NKT = BK / 32;
  constexpr int N = NKT * kDSteps;
  bf16x8 kf[R];
#pragma unroll
  for (int i = 0; i < R - 1; ++i) kf[i] = kr.frag(i / kDSteps, i % kDSteps);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int kt = i / kDSteps;
    const int ds = i % kDSteps;
    if (i + R - 1 < N) kf[(i + R - 1) % R] = kr.frag((i + R - 1) / kDSteps, (i + R - 1) % kDSteps);
    s[kt] = mfma(kf[i % R], qf[ds], ds == 0 ? f32x16{} : s[kt]);
    sched_fence();
  }
}

// Softmax result of one block for one wave: P as MFMA B-fragments per
// 16-key step, and the block scalars.
template <int BK, bool F32>
struct BlockP {
  static constexpr int NKT = BK / 32;
  u32x4 ph[NKT][2];  // P rounded to bf16
  u32x4 pl[NKT][2];  // P - bf16(P) rounded to bf16 (fp32-output mode only)
  float m_t;         // block max, log2 domain (-inf: no visible key)
  float l_b;         // block sum of p
};

// Causal / kv_len mask of a score block (only for blocks on the causal
// diagonal or past kv_len): key = key0 + 4*half + kt*32 + 8*(v/4) + v%4 is
// visible iff key <= limit; masked scores become -inf.  Positions are
// 32-bit (sequence lengths stay below 2^31).
template <int BK>
__device__ __forceinline__ void apply_mask(f32x16 (&s)[BK / 32], int key0, int kv_len, int causal, int qpos) {
  constexpr int NKT = BK / 32;
  const int half = (threadIdx.x & 63) >> 5;
  const int limit = causal ? min(kv_len - 1, qpos) : kv_len - 1;
  const int room = limit - (key0 + 4 * half);
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int off = kt * 32 + 8 * (v >> 2) + (v & 3);
      s[kt][v] = off <= room ? s[kt][v] : kNegInf;
    }
  }
}

// Block max (log2 domain) of a masked score block.
template <int BK>
__device__ __forceinline__ float block_max(const f32x16 (&s)[BK / 32], float c) {
  float mx = kNegInf;
#pragma unroll
  for (int kt = 0; kt < BK / 32; ++kt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kt][v]);
  }
  return block_m(pair_max(mx), c);
}

// p = 2^fma(s, c, -m), canonical sum, bf16 P of a masked score block.
template <int BK, bool F32>
__device__ __forceinline__ void softmax_core(f32x16 (&s)[BK / 32], float c, BlockP<BK, F32>& P) {
  constexpr int NKT = BK / 32;
  P.m_t = block_max<BK>(s, c);
  const float mu = block_m_use(P.m_t);
  float sub[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) s[kt][v] = block_p(s[kt][v], c, mu);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = s[kt][8 * st + 2 * w];
        const float p1 = s[kt][8 * st + 2 * w + 1];
        const uint32_t h = pack_bf16(p0, p1);
        P.ph[kt][st][w] = h;
        if constexpr (F32) P.pl[kt][st][w] = pack_bf16(p0 - bf16_lo_to_f32(h), p1 - bf16_hi_to_f32(h));
      }
    }
    sub[kt] = pair_sum(tree16(s[kt]));
  }
  P.l_b = combine_subtiles<NKT>(sub);
}

template <int BK, bool F32>
__device__ __forceinline__ void block_softmax(f32x16 (&s)[BK / 32], bool need_mask, int key0, int kv_len, int causal,
                                              int qpos, float c, BlockP<BK, F32>& P) {
  if (need_mask) apply_mask<BK>(s, key0, kv_len, causal, qpos);  // wave-uniform
  softmax_core<BK, F32>(s, c, P);
}

// One output dim tile of the block: acc_b tile = V^T P^T, an MFMA chain
// over the block's 16-key steps from zero.  V fragments come from a ring of
// R registers filled R-1 MFMAs ahead; the ring runs on across tiles when the
// caller passes the same ring to consecutive tiles.
template <int BK, bool F32, int R>
struct VRing {
  static constexpr int NS = BK / 16;  // 16-key steps per tile
  static constexpr int N = NS * kDTiles;
  bf16x8 f[R];
  __device__ __forceinline__ static bf16x8 load(const VReads<BK>& vr, int i) {
    const int n = i % NS;
    return vr.frag(i / NS, n >> 1, n & 1);
  }
  __device__ __forceinline__ void start(const VReads<BK>& vr) {
#pragma unroll
    for (int i = 0; i < R - 1; ++i) f[i] = load(vr, i);
  }
  // MFMAs of tile dt (global MFMA index i = dt*NS + n).
  __device__ __forceinline__ f32x16 tile(const VReads<BK>& vr, const BlockP<BK, F32>& P, int dt) {
    f32x16 ab = f32x16{};
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      const int i = dt * NS + n;
      const int j = i + R - 1;
      if (j < N) f[j % R] = load(vr, j);
      ab = mfma(f[i % R], as_bf16x8(P.ph[n >> 1][n & 1]), ab);
      if constexpr (F32) ab = mfma(f[i % R], as_bf16x8(P.pl[n >> 1][n & 1]), ab);
      sched_fence();
    }
    return ab;
  }
};

// Fold of one block item into the running state (core.hpp): the acc * alpha
// multiply is skipped when no lane of the wave moves its reference (alpha is
// then 1 on every lane and the multiply exact).
struct FoldIn {
  float r;      // 1 / l_b (0 for an empty row)
  FoldStep f;
  bool any_move;
};

__device__ __forceinline__ FoldIn fold_prepare(FoldState& fs, float m_t, float l_b) {
  const ItemScalars sc = item_scalars(m_t, l_b);
  FoldIn in;
  in.r = sc.r;
  in.f = fold_scalars(fs, sc.L);
  in.any_move = __any(in.f.move);
  return in;
}

__device__ __forceinline__ void fold_tile(f32x16& acc, const f32x16& ab, const FoldIn& in) {
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] = fold_elem_nomove(in.f, acc[v], ab[v] * in.r);
}

// PV of the block fused with its fold: tile dt's MFMAs are issued, then tile
// dt-1 (already finished) is folded while they run.
template <int BK, bool F32>
__device__ __forceinline__ void block_pv_fold(const VReads<BK>& vr, const BlockP<BK, F32>& P, const FoldIn& in,
                                              f32x16 (&acc)[kDTiles]) {
  if (in.any_move) {
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[dt][v] = acc[dt][v] * in.f.alpha;
    }
  }
  VRing<BK, F32, 3> ring;
  ring.start(vr);
  f32x16 ab0 = ring.tile(vr, P, 0);
  f32x16 ab1 = ring.tile(vr, P, 1);
  fold_tile(acc[0], ab0, in);
  sched_fence();
  ab0 = ring.tile(vr, P, 2);
  fold_tile(acc[1], ab1, in);
  sched_fence();
  ab1 = ring.tile(vr, P, 3);
  fold_tile(acc[2], ab0, in);
  fold_tile(acc[3], ab1, in);
}

// ------------------------------------------------------------ work map --

struct TileMap {
  int b, hk, head, t0, t, tile_t1, t_last;
  bool q_ok, wave_has_rows;
  int64_t qpos;
};

__device__ __forceinline__ TileMap map_tile(const PrefillArgs& a, int64_t wg) {
  TileMap m;
  // wave index made provably uniform, so per-wave decisions are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int col = threadIdx.x & 31;
  const int n_bh = a.B * a.Hkv * a.hsubs;
  int bh, ptile;
  heavy_first_tile(wg, n_bh, a.n_ptiles, bh, ptile);
  m.b = bh / (a.Hkv * a.hsubs);
  m.hk = (bh / a.hsubs) % a.Hkv;
  const int hs = bh % a.hsubs;
  const int tile_rows = 32 * a.pos_groups;
  const int tile_t0 = ptile * tile_rows;
  m.tile_t1 = min(a.Sq, tile_t0 + tile_rows) - 1;
  const bool wave_used = wave < a.heads_per_wg * a.pos_groups;  // 8 % G != 0 leaves waves idle
  m.head = m.hk * a.G + hs * a.heads_per_wg + (wave % a.heads_per_wg);
  m.t0 = tile_t0 + 32 * (wave / a.heads_per_wg);
  m.t = m.t0 + col;
  m.wave_has_rows = wave_used && m.t0 < a.Sq;
  m.q_ok = m.wave_has_rows && m.t < a.Sq;
  m.qpos = a.pos0 + m.t;
  m.t_last = min(a.Sq, m.t0 + 32) - 1;
  return m;
}

// Common per-wave set-up of both kernels.
struct WaveCtx {
  TileMap tm;
  __amdgpu_buffer_rsrc_t krs;  // keys [0, kv_len) of this kv head
  __amdgpu_buffer_rsrc_t vrs;
  int64_t row_stride;
  bf16x8 qf[kDSteps];
};

__device__ __forceinline__ void wave_setup(const PrefillArgs& a, int64_t wg, WaveCtx& w) {
  const int half = (threadIdx.x & 63) >> 5;
  w.tm = map_tile(a, wg);
  const int64_t kvoff = static_cast<int64_t>(w.tm.b) * a.kv_bstride + static_cast<int64_t>(w.tm.hk) * kHeadDim;
  w.row_stride = static_cast<int64_t>(a.Hkv) * kHeadDim;
  w.krs = head_rsrc(a.k + kvoff, a.kv_len, static_cast<int>(w.row_stride * 2));
  w.vrs = head_rsrc(a.v + kvoff, a.kv_len, static_cast<int>(w.row_stride * 2));
  const uint16_t* qrow = a.q + static_cast<int64_t>(w.tm.b) * a.q_bstride +
                         (static_cast<int64_t>(w.tm.t) * a.Hq + w.tm.head) * kHeadDim + 8 * half;
#pragma unroll
  for (int ds = 0; ds < kDSteps; ++ds)
    w.qf[ds] = as_bf16x8(w.tm.q_ok ? gload16(qrow + 16 * ds) : u32x4{0, 0, 0, 0});
}

// Does block blk hold a key some row of this wave may see?
template <int BK>
__device__ __forceinline__ bool wave_sees(const PrefillArgs& a, const TileMap& tm, int64_t blk) {
  return tm.wave_has_rows && blk * BK < a.kv_len && (!a.causal || blk * BK <= a.pos0 + tm.t_last);
}
// Is every key of block blk visible to every row of this wave?
template <int BK>
__device__ __forceinline__ bool wave_full(const PrefillArgs& a, const TileMap& tm, int64_t blk) {
  return (blk + 1) * BK <= a.kv_len && (!a.causal || (blk + 1) * BK - 1 <= a.pos0 + tm.t0);
}

// ----------------------------------------------------------- fused mode --

// Epilogue of both fused kernels: O = acc / l, LSE.
template <bool F32>
__device__ __forceinline__ void write_out(const PrefillArgs& a, const TileMap& tm, const FoldState& fs,
                                          const f32x16 (&acc)[kDTiles]) {
  const int half = (threadIdx.x & 63) >> 5;
  const Final fin = finalize(fs);
  const int64_t out_row = static_cast<int64_t>(tm.b) * a.Sq + tm.t;  // row index in [B*Sq]
  const int64_t orow = (out_row * a.Hq + tm.head) * kHeadDim;
#pragma unroll
  for (int dt = 0; dt < kDTiles; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = dt * 32 + 8 * g + 4 * half;
      const float o0 = acc[dt][4 * g] * fin.r;
      const float o1 = acc[dt][4 * g + 1] * fin.r;
      const float o2 = acc[dt][4 * g + 2] * fin.r;
      const float o3 = acc[dt][4 * g + 3] * fin.r;
      if constexpr (F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + orow + d) = f32x4{o0, o1, o2, o3};
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + orow + d) =
            u32x2{pack_bf16(o0, o1), pack_bf16(o2, o3)};
      }
    }
  }
  if (half == 0) a.lse[out_row * a.Hq + tm.head] = fin.lse;
}

// bf16 output, ping-pong schedule.  Waves w and w+4 of the workgroup share a
// SIMD.  Each wave's work is cut into two kinds of stage that use different
// units:
//   matrix stage A_j: PV of block j-1 with its fold (block_pv_fold), then
//                     S_j = K_j Q^T (block_scores)  -- 64 MFMAs and the fold
//   vector stage B_j: the softmax of S_j (block_softmax, fold_prepare)
// and a wave runs A_0, B_0, A_1, B_1, ..., A_n (n blocks; A_0 has no PV, A_n
// no scores).  The two halves of the workgroup (waves 0-3 and 4-7) run this
// sequence one stage apart: time is cut into half-steps ended by a workgroup
// barrier, and in half-step h a wave of group g is at stage h - g, so on
// every SIMD one wave issues matrix work while the other issues vector work.
// K_j is read in half-steps 2j (group 0) and 2j+1 (group 1), V_j in 2j+2 and
// 2j+3.  Group 1 issues all loads, at the start of each of its vector stages
// (which read no LDS): in half-step 2i it loads K_{i+1} and V_i, and it waits
// for them at the end of half-step 2i+1, so every load has two half-steps to
// land.  K and V are double-buffered in four separate LDS arrays, and the
// block loop is unrolled by two so that each stage names its arrays at
// compile time: the compiler then sees that the matrix stage's fragment reads
// and the loads in flight touch different arrays, and does not make the
// reads wait.  Q stays in registers.  Per block and wave the operations are
// those of the other fused kernels, so the result is the same bits.
template <int BK, int PG>
__global__ __launch_bounds__(kThreads) void prefill_pp_kernel(const PrefillArgs a) {
  using L = TileLayout<BK>;
  using Ld = BlockLoader<BK, kWaves / 2>;  // the waves of group 1
  using P = BlockP<BK, false>;
  constexpr int NKT = BK / 32;
  __shared__ __attribute__((aligned(16))) char kb0[L::kKBytes];
  __shared__ __attribute__((aligned(16))) char kb1[L::kKBytes];
  __shared__ __attribute__((aligned(16))) char vb0[L::kVBytes];
  __shared__ __attribute__((aligned(16))) char vb1[L::kVBytes];

  WaveCtx w;
  wave_setup(a, blockIdx.x, w);
  const TileMap& tm = w.tm;
  // 32-bit block indices and positions (the host keeps one head's rows below 2 GiB)
  const int kvl32 = static_cast<int>(a.kv_len);
  const int n_kv_blocks = (kvl32 + BK - 1) / BK;
  const int last_pos = static_cast<int>(a.pos0) + tm.tile_t1;
  const int nblk = a.causal ? min(n_kv_blocks, last_pos / BK + 1) : n_kv_blocks;
  const int first_pos = static_cast<int>(a.pos0) + tm.t0;
  const int wave_last = static_cast<int>(a.pos0) + tm.t_last;
  // does block j hold a key a row of this wave may see / do all rows see all its keys
  auto sees = [&](int j) { return tm.wave_has_rows && j * BK < kvl32 && (!a.causal || j * BK <= wave_last); };
  auto full = [&](int j) { return (j + 1) * BK <= kvl32 && (!a.causal || (j + 1) * BK - 1 <= first_pos); };
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int group = wave >> 2;

  FoldState fs{kNegInf, 0.0f};
  f32x16 acc[kDTiles];
#pragma unroll
  for (int dt = 0; dt < kDTiles; ++dt) acc[dt] = f32x16{};

  sched_fence();  // the Q loads of wave_setup stay ahead of the direct loads
  Ld ld;
  ld.init(static_cast<int>(w.row_stride), wave & 3);
  // Paged (PG != 0): group 1 gathers K and V through the page table (PG > 0:
  // the page size is 2^PG, fixed at compile time; PG < 0: any page size).
  PagedBufLoader<BK, kWaves / 2, (PG > 0 ? PG : 0)> pl;
  if constexpr (PG != 0)
    pl.init(a.page_table + static_cast<int64_t>(tm.b) * a.max_pages, a.log2_P, a.kv_len, a.num_pages, a.Hkv, tm.hk,
            wave & 3);
  auto issue_k = [&](char* dst, int key0) {
    if constexpr (PG != 0) {
      pl.template issue<false>(dst, a.k, key0);
    } else {
      ld.issue_k(dst, w.krs, key0);
    }
  };
  auto issue_v = [&](char* dst, int key0) {
    if constexpr (PG != 0) {
      pl.template issue<true>(dst, a.v, key0);
    } else {
      ld.issue_v(dst, w.vrs, key0);
    }
  };

  const int kvl = static_cast<int>(a.kv_len);
  const int qpos = static_cast<int>(tm.qpos);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // Fragment addresses of buffer 0 of each pair, computed once; buffer 1 of a
  // pair sits at a fixed distance, so every read is one register + immediate.
  const KReads<BK> kr0(kb0, opaque_lane());
  const VReads<BK> vr0(vb0, opaque_lane());
  // Loads of half-step 2i (group 1): K_{i+1} into the K array of parity
  // (i+1)&1 and V_i into the V array of parity i&1.  par = i & 1.
  auto loads = [&](auto par, int i) {
    constexpr int p = decltype(par)::value;
    if (i + 1 < nblk) issue_k(p ? kb0 : kb1, (i + 1) * BK);
    if (i < nblk) issue_v(p ? vb1 : vb0, i * BK);
  };
  // Matrix stage A_j (par = j & 1): PV + fold of block j-1 from the V array of
  // parity (j-1)&1, then the scores of block j from the K array of parity j&1.
  // The matrix stage is the one the SIMD's throughput depends on, so its wave
  // gets the higher issue priority.
  auto stage_a = [&](auto par, int j, f32x16 (&s)[NKT], const P& pp, const FoldIn& inp) {
    constexpr int p = decltype(par)::value;
    KReads<BK> kr = kr0;
    kr.reg = p ? kb1 : kb0;
    VReads<BK> vr = vr0;
    vr.reg = p ? vb0 : vb1;
    __builtin_amdgcn_s_setprio(2);
    if (j > 0 && sees(j - 1)) block_pv_fold<BK, false>(vr, pp, inp, acc);
    sched_fence();
    if (j < nblk && sees(j)) {
      block_scores_kr<BK, 3>(kr, w.qf, s);
    } else {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) s[kt] = f32x16{};  // defined on every path (unused)
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Vector stage B_j: softmax of S_j, fold scalars of block j.
  auto stage_b = [&](int j, f32x16 (&s)[NKT], P& pn, FoldIn& inn) {
    if (!sees(j)) {
      pn = P{};  // defined on every path, so the previous block's P is dead after its PV
      inn = FoldIn{};
      return;
    }
    block_softmax<BK, false>(s, !full(j), j * BK, kvl, a.causal, qpos, a.c, pn);
    inn = fold_prepare(fs, pn.m_t, pn.l_b);
  };
  // End of a half-step: (group 1, when it has loads in flight) wait for
  // them, then the barrier.
  auto end_half = [&]() {
    sched_fence();
    lds_barrier();
  };
  auto end_half_wait = [&]() {
    sched_fence();
    wait_direct_loads();
    lds_barrier();
  };

  P pb{};        // softmax result of the block whose PV is pending
  FoldIn ib{};   // and its fold scalars
  if (group == 0) {
    lds_barrier();  // prologue: K_0 landed
    int j = 0;
    for (; j + 2 <= nblk; j += 2) {
      {
        f32x16 s[NKT];
        stage_a(I0{}, j, s, pb, ib);  // half-step 2j
        end_half();
        stage_b(j, s, pb, ib);        // 2j+1
        end_half();
      }
      {
        f32x16 s[NKT];
        stage_a(I1{}, j + 1, s, pb, ib);
        end_half();
        stage_b(j + 1, s, pb, ib);
        end_half();
      }
    }
    if (j < nblk) {
      f32x16 s[NKT];
      stage_a(I0{}, j, s, pb, ib);
      end_half();
      stage_b(j, s, pb, ib);
      end_half();
    }
    {
      f32x16 s[NKT];
      if (nblk & 1) {
        stage_a(I1{}, nblk, s, pb, ib);  // half-step 2n: PV of the last block
      } else {
        stage_a(I0{}, nblk, s, pb, ib);
      }
      end_half();
    }
    end_half();  // half-step 2n+1
  } else {
    // prologue: K_0 (and the Q rows) landed; then the loads of half-step 0
    // (K_1, V_0), with nothing else in flight, so the compiler's wait
    // counting stays exact
    if (nblk > 0) issue_k(kb0, 0);
    wait_direct_loads();
    lds_barrier();
    loads(I0{}, 0);
    end_half();  // half-step 0
    int j = 0;
    for (; j + 2 <= nblk; j += 2) {
      {
        f32x16 s[NKT];
        stage_a(I0{}, j, s, pb, ib);  // half-step 2j+1
        end_half_wait();
        loads(I1{}, j + 1);           // half-step 2j+2
        stage_b(j, s, pb, ib);
        end_half();
      }
      {
        f32x16 s[NKT];
        stage_a(I1{}, j + 1, s, pb, ib);
        end_half_wait();
        loads(I0{}, j + 2);
        stage_b(j + 1, s, pb, ib);
        end_half();
      }
    }
    if (j < nblk) {
      f32x16 s[NKT];
      stage_a(I0{}, j, s, pb, ib);
      end_half_wait();
      loads(I1{}, j + 1);
      stage_b(j, s, pb, ib);
      end_half();
    }
    {
      f32x16 s[NKT];
      if (nblk & 1) {
        stage_a(I1{}, nblk, s, pb, ib);  // half-step 2n+1
      } else {
        stage_a(I0{}, nblk, s, pb, ib);
      }
      end_half_wait();
    }
  }

  if (!tm.q_ok) return;
  write_out<false>(a, tm, fs, acc);
}

// fp32 output (P carried as bf16 hi + lo, two MFMAs per key step): the
// phases run one after the other, one barrier after each.  K_{j+2} is loaded
// into the K buffer of block j in the third phase of block j and V_{j+1}
// into the other V buffer in the second phase, so each load has about four
// phases to land.
template <int BK, bool F32, bool PAGED>
__global__ __launch_bounds__(kThreads) void prefill_fused_kernel(const PrefillArgs a) {
  using L = TileLayout<BK>;
  using Ld = BlockLoader<BK, kWaves>;
  __shared__ __attribute__((aligned(16))) char kbuf[2 * L::kKBytes];
  __shared__ __attribute__((aligned(16))) char vbuf[2 * L::kVBytes];

  WaveCtx w;
  wave_setup(a, blockIdx.x, w);
  const TileMap& tm = w.tm;
  const int64_t n_kv_blocks = (a.kv_len + BK - 1) / BK;
  const int64_t nblk = a.causal ? min(n_kv_blocks, (a.pos0 + tm.tile_t1) / BK + 1) : n_kv_blocks;

  FoldState fs{kNegInf, 0.0f};
  f32x16 acc[kDTiles];
#pragma unroll
  for (int dt = 0; dt < kDTiles; ++dt) acc[dt] = f32x16{};

  sched_fence();  // the Q loads of wave_setup stay ahead of the direct loads
  Ld ld;
  ld.init(static_cast<int>(w.row_stride));
  PagedLoader<BK, kWaves> pl;
  if constexpr (PAGED)
    pl.init(a.page_table + static_cast<int64_t>(tm.b) * a.max_pages, a.log2_P, a.kv_len, a.num_pages, a.Hkv, tm.hk);
  auto issue_k = [&](char* dst, int64_t key0) {
    if constexpr (PAGED) {
      pl.template issue<false>(dst, a.k, key0);
    } else {
      ld.issue_k(dst, w.krs, key0);
    }
  };
  auto issue_v = [&](char* dst, int64_t key0) {
    if constexpr (PAGED) {
      pl.template issue<true>(dst, a.v, key0);
    } else {
      ld.issue_v(dst, w.vrs, key0);
    }
  };
  auto cnt = [&](int64_t blk) { return blk < nblk ? Ld::NI : 0; };  // loads of one region of blk
  if (nblk > 0) {
    issue_k(kbuf, 0);
    issue_v(vbuf, 0);
  }
  if (nblk > 1) issue_k(kbuf + L::kKBytes, BK);
  wait_direct_loads();  // Q, K_0, V_0, K_1
  lds_barrier();

  const int kvl = static_cast<int>(a.kv_len);
  const int qpos = static_cast<int>(tm.qpos);

  // kc: K of blk (read, then refilled with blk+2); vc: V of blk; vn: V buffer
  // being filled with blk+1.  The three do not overlap.
  auto step = [&](int64_t blk, char* __restrict__ kc, const char* __restrict__ vc, char* __restrict__ vn) {
    const bool sees = wave_sees<BK>(a, tm, blk);
    f32x16 s[BK / 32];
    BlockP<BK, F32> P;
    if (sees) block_scores<BK>(kc, w.qf, s);
    sched_fence();
    lds_barrier();
    if (blk + 1 < nblk) issue_v(vn, (blk + 1) * BK);
    FoldIn in{};
    if (sees) {
      block_softmax<BK, F32>(s, !wave_full<BK>(a, tm, blk), static_cast<int>(blk * BK), kvl, a.causal, qpos, a.c, P);
      in = fold_prepare(fs, P.m_t, P.l_b);
    }
    sched_fence();
    wait_loads_leq<Ld::NI>(cnt(blk + 1) + cnt(blk + 1));  // V of blk landed
    if constexpr (PAGED) {
      if ((blk + 1) * BK > a.kv_len) pl.clear_tail(const_cast<char*>(vc), blk * BK, a.kv_len);
    }
    lds_barrier();
    if (blk + 2 < nblk) issue_k(kc, (blk + 2) * BK);
    if (sees) block_pv_fold<BK, F32>(VReads<BK>(vc), P, in, acc);
    sched_fence();
    wait_loads_leq<Ld::NI>(cnt(blk + 1) + cnt(blk + 2));  // K of blk+1 landed
    lds_barrier();
  };
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int cb = static_cast<int>(blk & 1);
    step(blk, kbuf + cb * L::kKBytes, vbuf + cb * L::kVBytes, vbuf + (cb ^ 1) * L::kVBytes);
  }

  if (!tm.q_ok) return;
  write_out<F32>(a, tm, fs, acc);
}

// ------------------------------------------------------------ emit mode --

// One workgroup per (owned block, tile): stage the block, compute its item
// (O_b, L_b) for every row of the tile and write it.
template <int BK, bool F32>
__global__ __launch_bounds__(kThreads) void prefill_emit_kernel(const PrefillArgs a) {
  using L = TileLayout<BK>;
  __shared__ __attribute__((aligned(16))) char k0[L::kKBytes];
  __shared__ __attribute__((aligned(16))) char v0[L::kVBytes];

  const int half = (threadIdx.x & 63) >> 5;
  int64_t wg = blockIdx.x;
  const int pidx = static_cast<int>(wg % a.n_emit);
  wg /= a.n_emit;
  WaveCtx w;
  wave_setup(a, wg, w);
  const TileMap& tm = w.tm;

  const int64_t blk = a.emit_blocks[pidx];
  const bool tile_sees = blk * BK < a.kv_len && (!a.causal || blk * BK <= a.pos0 + tm.tile_t1);
  const bool active = tile_sees && wave_sees<BK>(a, tm, blk);
  f32x16 ab[kDTiles];
  BlockP<BK, F32> P;
  if (tile_sees) {  // uniform over the workgroup
    BlockLoader<BK, kWaves> ld;
    ld.init(static_cast<int>(w.row_stride));
    ld.issue_k(k0, w.krs, blk * BK);
    ld.issue_v(v0, w.vrs, blk * BK);
    wait_direct_loads();
    lds_barrier();
    if (active) {
      f32x16 s[BK / 32];
      block_scores<BK>(k0, w.qf, s);
      block_softmax<BK, F32>(s, !wave_full<BK>(a, tm, blk), static_cast<int>(blk * BK), static_cast<int>(a.kv_len),
                             a.causal, static_cast<int>(tm.qpos), a.c, P);
      const VReads<BK> vr(v0);
      VRing<BK, F32, 3> ring;
      ring.start(vr);
#pragma unroll
      for (int dt = 0; dt < kDTiles; ++dt) ab[dt] = ring.tile(vr, P, dt);
    }
  }
  const ItemScalars sc = active ? item_scalars(P.m_t, P.l_b) : ItemScalars{0.0f, kNegInf};
  if (!tm.q_ok) return;
  const int64_t out_row = static_cast<int64_t>(tm.b) * a.Sq + tm.t;
  const int64_t prow = static_cast<int64_t>(pidx) * a.B * a.Sq + out_row;
  float* po = a.part_out + (prow * a.Hq + tm.head) * kHeadDim;
#pragma unroll
  for (int dt = 0; dt < kDTiles; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = dt * 32 + 8 * g + 4 * half;
      f32x4 o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (active)
        o = f32x4{item_out(ab[dt][4 * g], sc), item_out(ab[dt][4 * g + 1], sc), item_out(ab[dt][4 * g + 2], sc),
                  item_out(ab[dt][4 * g + 3], sc)};
      *reinterpret_cast<f32x4*>(po + d) = o;
    }
  }
  if (half == 0) a.part_lse[prow * a.Hq + tm.head] = sc.L;
}

template <int BK, bool F32, bool EMIT, bool PAGED = false>
hipError_t launch_t(PrefillArgs a, hipStream_t s) {
  // tile = up to 8 column tiles of 32 positions: heads of the group first
  // (the largest divisor of G that fits), then positions
  int hpw = a.G < kWaves ? a.G : kWaves;
  while (a.G % hpw != 0) --hpw;
  a.heads_per_wg = hpw;
  a.pos_groups = kWaves / hpw;
  a.hsubs = a.G / hpw;
  const int tile_rows = 32 * a.pos_groups;
  a.n_ptiles = (a.Sq + tile_rows - 1) / tile_rows;
  int64_t grid = static_cast<int64_t>(a.n_ptiles) * a.B * a.Hkv * a.hsubs;
  if (EMIT) grid *= a.n_emit;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if constexpr (EMIT) {
    hipLaunchKernelGGL((prefill_emit_kernel<BK, F32>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  } else if constexpr (F32) {
    hipLaunchKernelGGL((prefill_fused_kernel<BK, F32, PAGED>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s,
                       a);
  } else {
    if (!PAGED) {
      hipLaunchKernelGGL((prefill_pp_kernel<BK, 0>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
    } else if (a.log2_P == 4) {  // 16-key pages
      hipLaunchKernelGGL((prefill_pp_kernel<BK, 4>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL((prefill_pp_kernel<BK, -1>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
    }
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int block, bool out_f32, bool emit, hipStream_t s) {
  if (block == 128) {
    if (out_f32) return emit ? launch_t<128, true, true>(a, s) : launch_t<128, true, false>(a, s);
    return emit ? launch_t<128, false, true>(a, s) : launch_t<128, false, false>(a, s);
  }
  if (block == 64) {
    if (out_f32) return emit ? launch_t<64, true, true>(a, s) : launch_t<64, true, false>(a, s);
    return emit ? launch_t<64, false, true>(a, s) : launch_t<64, false, false>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_paged(const PrefillArgs& a, int block, bool out_f32, hipStream_t s) {
  if (a.page_table == nullptr || a.log2_P < 2 || (1 << a.log2_P) > block) return hipErrorInvalidValue;
  if (block == 128) return out_f32 ? launch_t<128, true, false, true>(a, s) : launch_t<128, false, false, true>(a, s);
  if (block == 64) return out_f32 ? launch_t<64, true, false, true>(a, s) : launch_t<64, false, false, true>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace rla
