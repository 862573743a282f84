// Prefill / chunked-prefill kernel for gfx950: fused mode (fold every KV block
// of the row in ascending global block index and write Out/LSE) and emit mode
// (write the per-block partial states of a set of owned blocks, which is how a
// context-parallel shard is emulated on one GPU).
//
// Work decomposition: a workgroup of 8 waves (two per SIMD) takes one kv head
// hk of one batch row and a tile of query positions; each wave owns 32
// consecutive positions of one q head of the group (an MFMA column tile).
// Each KV block is staged in LDS once per workgroup by direct global->LDS
// loads and read by all waves.  In fused mode the LDS is double-buffered: the
// loads of block b+1 are issued before block b is computed, and one barrier
// per block hands the buffers over.
// Per wave and block: S^T = K Q^T (bf16 MFMA 32x32x16, fp32 accumulate), the
// block softmax on the score registers, and per 32-dim output tile
// acc_b = V^T P^T (bf16 MFMA), the block item O_b = acc_b / l_b and, in fused
// mode, its fold into the running state — all with the operations of
// core.hpp.  Fragment loads are software-pipelined one step ahead and fenced
// so the live register set stays within two waves per SIMD.  The fold of dim
// tile dt-1 is issued after the MFMAs of tile dt so the VALU work overlaps the
// matrix core.  No atomics and no split of a block across workgroups, so
// nothing depends on scheduling.
#include "kernels.hpp"
#include "tile.hpp"

namespace rla {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;

// Block softmax state of one wave for one staged block.
template <int BK, bool F32>
struct BlockCore {
  static constexpr int NKT = BK / 32;
  u32x4 ph[NKT][2];  // P (bf16 hi) as B-fragments per 16-key step
  u32x4 pl[NKT][2];  // P residual (bf16 lo), fp32-output mode only
  float m_t;         // block max, log2 domain (-inf: no visible key)
  float l_b;         // block sum of p

  // S^T, mask, max, p = 2^fma(s, c, -m), canonical sum, bf16 P.
  // Positions are 32-bit (sequence lengths stay below 2^31).
  __device__ __forceinline__ void softmax(const char* lds, const bf16x8 (&qf)[kDSteps], int key0, int kv_len,
                                          int causal, int qpos, bool need_mask, float c) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
    const int half = lane >> 5;
    f32x16 s[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) s[kt] = f32x16{};
    bf16x8 kf[2][NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) kf[0][kt] = k_frag<BK>(lds, kt, 0, col, half);
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) {
      if (ds + 1 < kDSteps) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) kf[(ds + 1) & 1][kt] = k_frag<BK>(lds, kt, ds + 1, col, half);
      }
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) s[kt] = mfma(kf[ds & 1][kt], qf[ds], s[kt]);
      sched_fence();
    }
    float mx = kNegInf;
    if (need_mask) {  // wave-uniform: only blocks on the causal diagonal or past kv_len
      const int kbase = key0 + 4 * half;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kbase + kt * 32 + 8 * (v >> 2) + (v & 3);
          const bool ok = key < kv_len && (!causal || key <= qpos);
          s[kt][v] = ok ? s[kt][v] : kNegInf;
          mx = fmaxf(mx, s[kt][v]);
        }
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kt][v]);
      }
    }
    mx = fmaxf(mx, partner(mx));
    m_t = block_m(mx, c);
    const float mu = block_m_use(m_t);
    float sub[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kt][v] = block_p(s[kt][v], c, mu);
      const float a = tree16(s[kt]);
      sub[kt] = a + partner(a);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float p0 = s[kt][8 * st + 2 * w];
          const float p1 = s[kt][8 * st + 2 * w + 1];
          const uint32_t h = pack_bf16(p0, p1);
          ph[kt][st][w] = h;
          if constexpr (F32) pl[kt][st][w] = pack_bf16(p0 - bf16_lo_to_f32(h), p1 - bf16_hi_to_f32(h));
        }
      }
    }
    l_b = combine_subtiles<NKT>(sub);
  }

  // Issue the PV MFMAs of output dim tile dt (chain over the block's keys in
  // 16-key steps from zero); V fragments prefetched one step ahead.
  __device__ __forceinline__ f32x16 pv(const char* lds, int dt) const {
    f32x16 acc = f32x16{};
    constexpr int NS = NKT * 2;
    bf16x8 vf[2];
    const char* vbase = lds + TileLayout<BK>::kKBytes;
    vf[0] = v_frag<BK>(vbase, dt, 0, 0);
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      if (n + 1 < NS) vf[(n + 1) & 1] = v_frag<BK>(vbase, dt, (n + 1) >> 1, (n + 1) & 1);
      const int kt = n >> 1, st = n & 1;
      acc = mfma(vf[n & 1], as_bf16x8(ph[kt][st]), acc);
      if constexpr (F32) acc = mfma(vf[n & 1], as_bf16x8(pl[kt][st]), acc);
      sched_fence();
    }
    return acc;
  }
};

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
  const int bh = static_cast<int>(wg % n_bh);
  const int ptile = a.n_ptiles - 1 - static_cast<int>(wg / n_bh);  // heaviest tiles first
  m.b = bh / (a.Hkv * a.hsubs);
  m.hk = (bh / a.hsubs) % a.Hkv;
  const int hs = bh % a.hsubs;
  const int tile_rows = 32 * a.pos_groups;
  const int tile_t0 = ptile * tile_rows;
  m.tile_t1 = min(a.Sq, tile_t0 + tile_rows) - 1;
  m.head = m.hk * a.G + hs * a.heads_per_wg + (wave % a.heads_per_wg);
  m.t0 = tile_t0 + 32 * (wave / a.heads_per_wg);
  m.t = m.t0 + col;
  m.q_ok = m.t < a.Sq;
  m.qpos = a.pos0 + m.t;
  m.t_last = min(a.Sq, m.t0 + 32) - 1;
  m.wave_has_rows = m.t0 < a.Sq;
  return m;
}

// One fold step of output dim tile dt (acc_b -> O_b -> running acc).  When
// every lane of the wave takes the "add" step (the common case) the select
// of fold_elem is skipped; the arithmetic is the same.
__device__ __forceinline__ void fold_tile(f32x16& acc, const f32x16& ab, const ItemScalars& sc, const FoldStep& f,
                                          bool all_add) {
  if (all_add) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = fold_add(acc[v], item_out(ab[v], sc), f.beta);
  } else {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = fold_elem(f, acc[v], item_out(ab[v], sc));
  }
}

template <int BK, bool F32, bool EMIT>
__global__ __launch_bounds__(kThreads) void prefill_kernel(const PrefillArgs a) {
  using L = TileLayout<BK>;
  constexpr int NBUF = EMIT ? 1 : 2;
  __shared__ __attribute__((aligned(16))) char lds[NBUF * L::kBytes];

  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;

  int64_t wg = blockIdx.x;
  int pidx = 0;
  if constexpr (EMIT) {
    pidx = static_cast<int>(wg % a.n_emit);
    wg /= a.n_emit;
  }
  const TileMap tm = map_tile(a, wg);

  const uint16_t* kb = a.k + static_cast<int64_t>(tm.b) * a.kv_bstride + static_cast<int64_t>(tm.hk) * kHeadDim;
  const uint16_t* vb = a.v + static_cast<int64_t>(tm.b) * a.kv_bstride + static_cast<int64_t>(tm.hk) * kHeadDim;
  const int64_t row_stride = static_cast<int64_t>(a.Hkv) * kHeadDim;

  bf16x8 qf[kDSteps];
  {
    const uint16_t* qrow = a.q + static_cast<int64_t>(tm.b) * a.q_bstride +
                           (static_cast<int64_t>(tm.t) * a.Hq + tm.head) * kHeadDim + 8 * half;
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds)
      qf[ds] = as_bf16x8(tm.q_ok ? gload16(qrow + 16 * ds) : u32x4{0, 0, 0, 0});
  }

  // Does block blk hold a key some row of this wave may see?
  auto wave_sees = [&](int64_t blk) {
    return tm.wave_has_rows && blk * BK < a.kv_len && (!a.causal || blk * BK <= a.pos0 + tm.t_last);
  };
  // Is every key of block blk visible to every row of this wave?
  auto wave_full = [&](int64_t blk) {
    return (blk + 1) * BK <= a.kv_len && (!a.causal || (blk + 1) * BK - 1 <= a.pos0 + tm.t0);
  };
  const int64_t out_row = static_cast<int64_t>(tm.b) * a.Sq + tm.t;  // row index in [B*Sq]

  if constexpr (EMIT) {
    const int64_t blk = a.emit_blocks[pidx];
    const bool tile_sees = blk * BK < a.kv_len && (!a.causal || blk * BK <= a.pos0 + tm.tile_t1);
    const bool active = tile_sees && wave_sees(blk);
    BlockCore<BK, F32> bc;
    if (tile_sees) {
      BlockLoader<BK, kWaves> ld;
      ld.init(static_cast<int>(row_stride));
      ld.issue(lds, kb, vb, row_stride, blk * BK, a.kv_len);
      wait_direct_loads();
      __syncthreads();
      if (active)
        bc.softmax(lds, qf, static_cast<int>(blk * BK), static_cast<int>(a.kv_len), a.causal,
                   static_cast<int>(tm.qpos), !wave_full(blk), a.c);
    }
    const ItemScalars sc = active ? item_scalars(bc.m_t, bc.l_b) : ItemScalars{0.0f, kNegInf};
    const int64_t prow = static_cast<int64_t>(pidx) * a.B * a.Sq + out_row;
    float* po = a.part_out + (prow * a.Hq + tm.head) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) {
      const f32x16 ob = active ? bc.pv(lds, dt) : f32x16{};
      if (tm.q_ok) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = dt * 32 + 8 * g + 4 * half;
          *reinterpret_cast<f32x4*>(po + d) = f32x4{item_out(ob[4 * g], sc), item_out(ob[4 * g + 1], sc),
                                                    item_out(ob[4 * g + 2], sc), item_out(ob[4 * g + 3], sc)};
        }
      }
    }
    if (tm.q_ok && half == 0) a.part_lse[prow * a.Hq + tm.head] = sc.L;
    return;
  } else {
    const int64_t n_kv_blocks = (a.kv_len + BK - 1) / BK;
    const int64_t last_blk = a.causal ? min(n_kv_blocks - 1, (a.pos0 + tm.tile_t1) / BK) : n_kv_blocks - 1;
    FoldState fs{kNegInf, 0.0f};
    f32x16 acc[kDTiles];
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) acc[dt] = f32x16{};

    BlockLoader<BK, kWaves> ld;
    ld.init(static_cast<int>(row_stride));
    if (last_blk >= 0) ld.issue(lds, kb, vb, row_stride, 0, a.kv_len);
    wait_direct_loads();
    __syncthreads();

    for (int64_t blk = 0; blk <= last_blk; ++blk) {
      const char* cur = lds + (blk & 1) * L::kBytes;
      if (blk + 1 <= last_blk)
        ld.issue(lds + ((blk + 1) & 1) * L::kBytes, kb, vb, row_stride, (blk + 1) * BK, a.kv_len);
      if (wave_sees(blk)) {
        BlockCore<BK, F32> bc;
        bc.softmax(cur, qf, static_cast<int>(blk * BK), static_cast<int>(a.kv_len), a.causal,
                   static_cast<int>(tm.qpos), !wave_full(blk), a.c);
        const ItemScalars sc = item_scalars(bc.m_t, bc.l_b);
        const FoldStep f = fold_scalars(fs, sc.L);
        const bool all_add = __all(f.mode == kFoldAdd);
        f32x16 ab0 = bc.pv(cur, 0);
        f32x16 ab1 = bc.pv(cur, 1);
        fold_tile(acc[0], ab0, sc, f, all_add);
        ab0 = bc.pv(cur, 2);
        fold_tile(acc[1], ab1, sc, f, all_add);
        ab1 = bc.pv(cur, 3);
        fold_tile(acc[2], ab0, sc, f, all_add);
        fold_tile(acc[3], ab1, sc, f, all_add);
      }
      wait_direct_loads();
      __syncthreads();
    }

    if (!tm.q_ok) return;
    const Final fin = finalize(fs);
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
}

template <int BK, bool F32, bool EMIT>
hipError_t launch_t(PrefillArgs a, hipStream_t s) {
  // tile = 8 column tiles of 32 positions: heads of the group first, then positions
  a.heads_per_wg = a.G < kWaves ? a.G : kWaves;
  a.pos_groups = kWaves / a.heads_per_wg;
  a.hsubs = a.G / a.heads_per_wg;
  const int tile_rows = 32 * a.pos_groups;
  a.n_ptiles = (a.Sq + tile_rows - 1) / tile_rows;
  int64_t grid = static_cast<int64_t>(a.n_ptiles) * a.B * a.Hkv * a.hsubs;
  if (EMIT) grid *= a.n_emit;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_kernel<BK, F32, EMIT>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
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

}  // namespace rla
