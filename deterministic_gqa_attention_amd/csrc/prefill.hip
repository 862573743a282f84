// Prefill / chunked-prefill kernel for gfx950: fused mode (fold every KV block
// of the row in ascending global block index and write Out/LSE) and emit mode
// (write the per-block partial states of a set of owned blocks, which is how a
// context-parallel shard is emulated on one GPU).
//
// Work decomposition: a workgroup of 4 waves takes one kv head hk of one batch
// row and a tile of query positions; wave w owns 32 consecutive positions of
// one q head of the group (an MFMA column tile).  The workgroup stages each
// KV block in LDS once (K key-major, V transposed) and all four waves read it.
// Per wave and block: S^T = K Q^T (bf16 MFMA 32x32x16, fp32 accumulate), the
// block softmax on the score registers, acc_b = V^T P^T (bf16 MFMA), the block
// item (O_b, L_b) and, in fused mode, the fold into the running state — all
// with the operations of core.hpp.  No atomics, no split of a block across
// workgroups, so nothing depends on scheduling.
#include "kernels.hpp"
#include "tile.hpp"

namespace rla {

namespace {

constexpr int kThreads = 256;

template <int BK>
__device__ __forceinline__ void stage_block(char* lds, const uint16_t* kb, const uint16_t* vb,
                                            int64_t row_stride, int64_t key0, int64_t kv_len) {
  using L = TileLayout<BK>;
  const int tid = threadIdx.x;
  char* lk = lds;
  char* lv = lds + L::kKBytes;
  // K: 16-byte chunk c of key row r; 16 consecutive threads cover one row.
  constexpr int KIT = BK / 16;
  const int c = tid & 15;
  const int r0 = tid >> 4;
  u32x4 kx[KIT];
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int64_t key = key0 + r0 + 16 * i;
    kx[i] = key < kv_len ? gload16(kb + key * row_stride + c * 8) : u32x4{0, 0, 0, 0};
  }
  // V: 4-key x 8-dim sub-block (key group kg, dim chunk dc).
  constexpr int VIT = BK / 64;
  const int dc = tid & 15;
  const int kg0 = tid >> 4;
  u32x4 vx[VIT][4];
#pragma unroll
  for (int i = 0; i < VIT; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t key = key0 + 4 * (kg0 + 16 * i) + j;
      vx[i][j] = key < kv_len ? gload16(vb + key * row_stride + dc * 8) : u32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int i = 0; i < KIT; ++i) lds_store16(lk, L::k_off(r0 + 16 * i, c), kx[i]);
#pragma unroll
  for (int i = 0; i < VIT; ++i) {
    u32x2 t[8];
    transpose4x8(vx[i], t);
    const int kg = kg0 + 16 * i;
#pragma unroll
    for (int ii = 0; ii < 8; ++ii) lds_store8(lv, L::v_off(8 * dc + ii, kg), t[ii]);
  }
}

// One wave, one staged block: block item for the wave's 32 query columns.
// Returns O_b in ob[] (output layout of the PV MFMA) and the item scalars.
template <int BK, bool F32>
__device__ __forceinline__ ItemScalars wave_block_item(const char* lds, const bf16x8 (&qf)[kDSteps],
                                                      int64_t key0, int64_t kv_len, int causal,
                                                      int64_t qpos, bool need_mask, float cscale,
                                                      f32x16 (&ob)[kDTiles]) {
  using L = TileLayout<BK>;
  constexpr int NKT = BK / 32;
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const char* lk = lds;
  const char* lv = lds + L::kKBytes;

  // S^T sub-tiles: chain over the head dimension in 8 fixed steps.
  f32x16 s[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) s[kt] = f32x16{};
#pragma unroll
  for (int ds = 0; ds < kDSteps; ++ds) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) s[kt] = mfma(k_frag<BK>(lk, kt, ds, col, half), qf[ds], s[kt]);
  }

  // t = dot * c, masked keys -> -inf by select; block max.
  float mx = kNegInf;
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float t = s[kt][v] * cscale;
      if (need_mask) {
        const int64_t key = key0 + kt * 32 + acc_row(v, half);
        const bool ok = key < kv_len && (!causal || key <= qpos);
        t = ok ? t : kNegInf;
      }
      s[kt][v] = t;
      mx = fmaxf(mx, t);
    }
  }
  const float m_t = fmaxf(mx, partner(mx));
  const float m_use = (m_t == kNegInf) ? 0.0f : m_t;

  // p = 2^(t - m), block sum by the canonical tree, P to bf16 (hi/lo).
  float sub[NKT];
  u32x4 ph[NKT][2];
  u32x4 pl[NKT][2];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) s[kt][v] = hw_exp2(s[kt][v] - m_use);
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
        if constexpr (F32) {
          const float r0 = p0 - bf16_lo_to_f32(h);
          const float r1 = p1 - bf16_hi_to_f32(h);
          pl[kt][st][w] = pack_bf16(r0, r1);
        }
      }
    }
  }
  const float l_b = combine_subtiles<NKT>(sub);

  // acc_b = V^T P^T from zero, chain over the block's keys in 16-key steps.
#pragma unroll
  for (int dt = 0; dt < kDTiles; ++dt) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 vf = v_frag<BK>(lv, dt, kt, st, col, half);
        acc = mfma(vf, as_bf16x8(ph[kt][st]), acc);
        if constexpr (F32) acc = mfma(vf, as_bf16x8(pl[kt][st]), acc);
      }
    }
    ob[dt] = acc;
  }
  const ItemScalars sc = item_scalars(m_t, l_b);
#pragma unroll
  for (int dt = 0; dt < kDTiles; ++dt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) ob[dt][v] = item_out(ob[dt][v], sc);
  }
  return sc;
}

template <int BK, bool F32, bool EMIT>
__global__ __launch_bounds__(kThreads) void prefill_kernel(const PrefillArgs a) {
  using L = TileLayout<BK>;
  __shared__ __attribute__((aligned(16))) char lds[L::kBytes];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  int64_t wg = blockIdx.x;
  int pidx = 0;
  if constexpr (EMIT) {
    pidx = static_cast<int>(wg % a.n_emit);
    wg /= a.n_emit;
  }
  const int n_bh = a.B * a.Hkv * a.hsubs;
  const int bh = static_cast<int>(wg % n_bh);
  const int ptile = a.n_ptiles - 1 - static_cast<int>(wg / n_bh);  // heaviest tiles first
  const int b = bh / (a.Hkv * a.hsubs);
  const int hk = (bh / a.hsubs) % a.Hkv;
  const int hs = bh % a.hsubs;

  const int tile_rows = 32 * a.pos_groups;
  const int tile_t0 = ptile * tile_rows;
  const int tile_t1 = min(a.Sq, tile_t0 + tile_rows) - 1;  // last valid row of the tile
  const int head = hk * a.G + hs * a.heads_per_wg + (wave % a.heads_per_wg);
  const int t0 = tile_t0 + 32 * (wave / a.heads_per_wg);     // first row of this wave
  const int t = t0 + col;
  const bool q_ok = t < a.Sq;
  const int64_t qpos = a.pos0 + t;
  const int t_last = min(a.Sq, t0 + 32) - 1;                 // last valid row of this wave
  const bool wave_has_rows = t0 < a.Sq;

  const uint16_t* kb = a.k + static_cast<int64_t>(b) * a.kv_bstride + static_cast<int64_t>(hk) * kHeadDim;
  const uint16_t* vb = a.v + static_cast<int64_t>(b) * a.kv_bstride + static_cast<int64_t>(hk) * kHeadDim;
  const int64_t row_stride = static_cast<int64_t>(a.Hkv) * kHeadDim;

  bf16x8 qf[kDSteps];
  {
    const uint16_t* qrow = a.q + static_cast<int64_t>(b) * a.q_bstride +
                           (static_cast<int64_t>(t) * a.Hq + head) * kHeadDim + 8 * half;
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) qf[ds] = as_bf16x8(q_ok ? gload16(qrow + 16 * ds) : u32x4{0, 0, 0, 0});
  }

  const int64_t n_kv_blocks = (a.kv_len + BK - 1) / BK;
  // Does block blk hold a key some row of this wave may see?
  auto wave_sees = [&](int64_t blk) {
    return wave_has_rows && blk * BK < a.kv_len && (!a.causal || blk * BK <= a.pos0 + t_last);
  };
  // Is every key of block blk visible to every row of this wave?
  auto wave_full = [&](int64_t blk) {
    return (blk + 1) * BK <= a.kv_len && (!a.causal || (blk + 1) * BK - 1 <= a.pos0 + t0);
  };

  const int64_t out_row = static_cast<int64_t>(b) * a.Sq + t;  // row index in [B*Sq]

  if constexpr (EMIT) {
    const int64_t blk = a.emit_blocks[pidx];
    const bool tile_sees = blk * BK < a.kv_len && (!a.causal || blk * BK <= a.pos0 + tile_t1);
    f32x16 ob[kDTiles];
    ItemScalars sc{0.0f, kNegInf};
    if (tile_sees) {
      stage_block<BK>(lds, kb, vb, row_stride, blk * BK, a.kv_len);
      __syncthreads();
      if (wave_sees(blk)) {
        sc = wave_block_item<BK, F32>(lds, qf, blk * BK, a.kv_len, a.causal, qpos, !wave_full(blk), a.c, ob);
      } else {
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt) ob[dt] = f32x16{};
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < kDTiles; ++dt) ob[dt] = f32x16{};
    }
    if (q_ok) {
      const int64_t prow = static_cast<int64_t>(pidx) * a.B * a.Sq + out_row;
      float* po = a.part_out + (prow * a.Hq + head) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < kDTiles; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = dt * 32 + 8 * g + 4 * half;
          *reinterpret_cast<f32x4*>(po + d) =
              f32x4{ob[dt][4 * g], ob[dt][4 * g + 1], ob[dt][4 * g + 2], ob[dt][4 * g + 3]};
        }
      }
      if (half == 0) a.part_lse[prow * a.Hq + head] = sc.L;
    }
    return;
  } else {
    // Fused: fold every visible block in ascending global block index.
    const int64_t last_blk = a.causal ? min(n_kv_blocks - 1, (a.pos0 + tile_t1) / BK) : n_kv_blocks - 1;
    FoldState st{kNegInf, 0.0f};
    f32x16 acc[kDTiles];
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) acc[dt] = f32x16{};

    for (int64_t blk = 0; blk <= last_blk; ++blk) {
      __syncthreads();
      stage_block<BK>(lds, kb, vb, row_stride, blk * BK, a.kv_len);
      __syncthreads();
      if (!wave_sees(blk)) continue;
      f32x16 ob[kDTiles];
      const ItemScalars sc =
          wave_block_item<BK, F32>(lds, qf, blk * BK, a.kv_len, a.causal, qpos, !wave_full(blk), a.c, ob);
      const FoldStep f = fold_scalars(st, sc.L);
      if (__all(f.mode == kFoldCombine && f.alpha == 1.0f)) {
        // acc * 1 == acc exactly: same bits as the general combine below.
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[dt][v] = fmaf(ob[dt][v], f.beta, acc[dt][v]);
      } else if (__all(f.mode == kFoldCombine)) {
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[dt][v] = fold_combine(acc[dt][v], ob[dt][v], f.alpha, f.beta);
      } else {
#pragma unroll
        for (int dt = 0; dt < kDTiles; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[dt][v] = fold_elem(f, acc[dt][v], ob[dt][v]);
      }
    }

    if (!q_ok) return;
    const Final fin = finalize(st);
    const int64_t orow = (out_row * a.Hq + head) * kHeadDim;
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
    if (half == 0) a.lse[out_row * a.Hq + head] = fin.lse;
  }
}

template <int BK, bool F32, bool EMIT>
hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
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
