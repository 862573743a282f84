// Backward of deterministic attention for gfx950: dQ, dK and dV of Out.
//
// For a query row i of q head h, key j of its kv head, and the forward's
// natural-log LSE_i:
//   P_ij  = 2^fma(dot(q_i, k_j), c, -LSE_i * log2 e)   (c = scale * log2 e)
//   dP_ij = dot(dOut_i, v_j)
//   Delta_i = sum_d dOut_i[d] * Out_i[d]
//   dS_ij = (P_ij * (dP_ij - Delta_i)) * scale,  rounded to bf16
//   dV_j += bf16(P_ij) dOut_i,  dK_j += dS_ij q_i,  dQ_i += dS_ij k_j
// (the chain rule through softmax; the gradient reaching LSE is taken as
// zero).  Dot products are bf16 MFMA chains over D with FP32 accumulation,
// the same 32x32x16 shape and D-step order as the forward.
//
// Determinism.  No atomics and no reduction whose order depends on the
// schedule: every output element is one MFMA accumulation chain in a fixed
// order.
//  * dK and dV of a key: query tiles of 64 rows (counted from the first row of
//    the call) in ascending order; inside a tile, the q heads of the group in
//    ascending order; inside a head, the 64 rows in four 16-row MFMA steps in
//    ascending order.  One workgroup owns 128 keys for the whole walk.
//  * dQ of a row: KV blocks of 64 keys in ascending order from key 0, each in
//    four 16-key MFMA steps.
// Two launches: the dQ kernel, which also computes Delta per row (a fixed
// tree over the 128 products) and writes it with LSE * log2 e to a per-row
// scratch, then the dK/dV kernel.  Chunked replay: with accumulate set, dK/dV start from the
// values already in the output buffers, so calls over consecutive query
// chunks whose boundaries are multiples of 64 rows continue the chains of a
// single call over all rows and give its exact bits.
//
// Pages: "[WS2][Attention] H100 validation and reproduction guide for #235
// PR1-PR8", sections "PR stack" (the prefill/chunked-prefill backward leg for
// dQ/dK/dV), "Status" and "Acceptance" (dQ, dK, dV bitwise equal across
// decompositions, max abs 0.0).
#include "kernels.hpp"
#include "tile.hpp"

namespace rla {

namespace {

constexpr int kQT = 64;   // query rows per tile
constexpr int kKB = 128;  // keys per dK/dV workgroup (4 waves x 32 keys)
constexpr int kQB = 64;   // keys per KV block streamed by the dQ kernel

// Row-fragment reads (ds_read_b128) of a region of 256-byte rows stored with
// the V swizzle of TileLayout: MFMA A-fragment of row tile rt (rows
// 32rt..32rt+31), head-dim step ds.  v_swz depends on the row's low four bits
// only, so row 32rt + col sits at the address of row col plus 32rt*256.
struct RowReadsV {
  const char* reg;
  int ref;
  int a[kDSteps];
  __device__ __forceinline__ explicit RowReadsV(const char* r) : reg(r), ref(lds_address(r)) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
    const int half = lane >> 5;
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) a[ds] = opaque_add(TileLayout<64>::v_rel(col, 2 * ds + half), ref);
  }
  __device__ __forceinline__ bf16x8 frag(int rt, int ds) const {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(reg + (a[ds] - ref + rt * 32 * 256)));
  }
};

// Four consecutive gradient values at element idx of an fp32 or bf16 (RNE,
// the only rounding of the result) output.
__device__ __forceinline__ void store_grad4(void* base, int64_t idx, float x0, float x1, float x2, float x3, bool bf) {
  if (bf) {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + idx) = u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)};
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx) = f32x4{x0, x1, x2, x3};
  }
}

// Eight accumulator registers 8s..8s+7 rounded to bf16 as one MFMA
// B-fragment (element j = register 8s + j).
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int s) {
  u32x4 w;
  w[0] = pack_bf16(x[8 * s + 0], x[8 * s + 1]);
  w[1] = pack_bf16(x[8 * s + 2], x[8 * s + 3]);
  w[2] = pack_bf16(x[8 * s + 4], x[8 * s + 5]);
  w[3] = pack_bf16(x[8 * s + 6], x[8 * s + 7]);
  return as_bf16x8(w);
}

// ----------------------------------------------------------------- dQ --

// One workgroup of 8 waves per (b, kv head, head subgroup, query tile of 64
// rows); wave w takes q head slot w % hpw and rows 32*(w / hpw).. of the
// tile.  KV blocks of 64 keys are staged in LDS (K with the V swizzle: row
// reads for S^T and transposed reads for dQ^T; V with the K swizzle: row
// reads for dP^T), double-buffered.
constexpr int kDqWaves = 8;

template <bool OUT_F32>
__global__ __launch_bounds__(kDqWaves * 64) void bwd_dq_kernel(const BackwardArgs a) {
  using Ld = BlockLoader<kQB, kDqWaves>;
  constexpr int kRegion = kQB * kHeadDim * 2;
  __shared__ __attribute__((aligned(16))) char kbuf[2 * kRegion];
  __shared__ __attribute__((aligned(16))) char vbuf[2 * kRegion];

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  const int n_bh = a.B * a.Hkv * a.hsubs;
  const int64_t wg = blockIdx.x;
  int bh, ptile;
  heavy_first_tile(wg, n_bh, a.n_qtiles, bh, ptile);
  const int b = bh / (a.Hkv * a.hsubs);
  const int hk = (bh / a.hsubs) % a.Hkv;
  const int hs = bh % a.hsubs;
  const int tile_t0 = ptile * kQT;
  const int tile_t1 = min(a.Sq, tile_t0 + kQT) - 1;
  const bool wave_used = wave < 2 * a.hpw;
  const int head = hk * a.G + hs * a.hpw + (wave % a.hpw);
  const int t0 = tile_t0 + 32 * (wave / a.hpw);
  const int t = t0 + col;
  const bool wave_has_rows = wave_used && t0 < a.Sq;
  const bool q_ok = wave_has_rows && t < a.Sq;
  const int t_last = min(a.Sq, t0 + 32) - 1;
  const int64_t qpos = a.pos0 + t;

  // Q and dOut B-fragments of this lane's row; the row's LSE*log2e and Delta.
  bf16x8 qf[kDSteps], of[kDSteps];
  {
    const int64_t e = static_cast<int64_t>(b) * a.q_bstride + (static_cast<int64_t>(t) * a.Hq + head) * kHeadDim + 8 * half;
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) {
      qf[ds] = as_bf16x8(q_ok ? gload16(a.q + e + 16 * ds) : u32x4{0, 0, 0, 0});
      of[ds] = as_bf16x8(q_ok ? gload16(a.dout + e + 16 * ds) : u32x4{0, 0, 0, 0});
    }
  }
  // Delta of the lane's row: the products dOut * Out of the dims the lane
  // holds (16ds + 8half + 0..7) in a fixed tree per D-step, the eight step
  // sums in a fixed tree, then the partner lane's sum (the other half of the
  // row).  LSE * log2 e and Delta go to the scratch for the dK/dV kernel
  // (zeros for rows past Sq).
  float lse2 = 0.0f, delta = 0.0f;
  {
    float part = 0.0f;
    if (q_ok) {
      const int64_t e = static_cast<int64_t>(b) * a.q_bstride + (static_cast<int64_t>(t) * a.Hq + head) * kHeadDim + 8 * half;
      float st[kDSteps];
#pragma unroll
      for (int ds = 0; ds < kDSteps; ++ds) {
        float o[8];
        if constexpr (OUT_F32) {
          const f32x4 o0 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.out) + e + 16 * ds);
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.out) + e + 16 * ds + 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o[i] = o0[i];
            o[4 + i] = o1[i];
          }
        } else {
          const u32x4 ow = gload16(static_cast<const uint16_t*>(a.out) + e + 16 * ds);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            o[2 * i] = bf16_lo_to_f32(ow[i]);
            o[2 * i + 1] = bf16_hi_to_f32(ow[i]);
          }
        }
        const u32x4 gw = __builtin_bit_cast(u32x4, of[ds]);
        float p[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[2 * i] = bf16_lo_to_f32(gw[i]) * o[2 * i];
          p[2 * i + 1] = bf16_hi_to_f32(gw[i]) * o[2 * i + 1];
        }
        st[ds] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      }
      part = ((st[0] + st[1]) + (st[2] + st[3])) + ((st[4] + st[5]) + (st[6] + st[7]));
      lse2 = a.lse[(static_cast<int64_t>(b) * a.Sq + t) * a.Hq + head] * kLog2e;
    }
    delta = pair_sum(part);
    if (wave_used && half == 0) {
      float* row = a.ws + (static_cast<int64_t>(b) * a.Hq + head) * 2 * a.Sq_pad;
      row[t] = lse2;
      row[a.Sq_pad + t] = delta;
    }
  }

  const int64_t n_kv_blocks = (a.kv_len + kQB - 1) / kQB;
  const int64_t nblk = a.causal ? min(n_kv_blocks, (a.pos0 + tile_t1) / kQB + 1) : n_kv_blocks;
  const int kvl = static_cast<int>(a.kv_len);
  const int limit = !q_ok ? -1 : (a.causal ? min(kvl - 1, static_cast<int>(qpos)) : kvl - 1);

  f32x16 acc[kDTiles];
#pragma unroll
  for (int dt = 0; dt < kDTiles; ++dt) acc[dt] = f32x16{};

  const int64_t kvoff = static_cast<int64_t>(b) * a.kv_bstride + static_cast<int64_t>(hk) * kHeadDim;
  const int row_stride = a.Hkv * kHeadDim;
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k + kvoff, a.kv_len, row_stride * 2);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(a.v + kvoff, a.kv_len, row_stride * 2);
  Ld ld;
  ld.init(row_stride);
  auto issue = [&](int64_t blk) {
    const int buf = static_cast<int>(blk & 1);
    ld.issue_v(kbuf + buf * kRegion, krs, blk * kQB);  // K: V swizzle
    ld.issue_k(vbuf + buf * kRegion, vrs, blk * kQB);  // V: K swizzle
  };
  if (nblk > 0) issue(0);

  for (int64_t blk = 0; blk < nblk; ++blk) {
    wait_direct_loads();
    lds_barrier();  // block blk staged; every wave is done with block blk-1
    if (blk + 1 < nblk) issue(blk + 1);
    const int buf = static_cast<int>(blk & 1);
    const char* kreg = kbuf + buf * kRegion;
    const char* vreg = vbuf + buf * kRegion;
    const int key0 = static_cast<int>(blk * kQB);
    const bool sees = wave_has_rows && key0 < kvl && (!a.causal || key0 <= a.pos0 + t_last);
    if (!sees) continue;
    const bool full = key0 + kQB <= kvl && (!a.causal || key0 + kQB - 1 <= a.pos0 + t0) && t_last == t0 + 31;

    // S^T = K Q^T and dP^T = V dOut^T, fragments read one D-step ahead.
    f32x16 s[2], dp[2];
    {
      const RowReadsV kr(kreg);
      const KReads<kQB> vr(vreg);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[kt] = f32x16{};
        dp[kt] = f32x16{};
      }
      bf16x8 fa[2][4];
      auto rd = [&](int ds, int slot) {
        fa[slot][0] = kr.frag(0, ds);
        fa[slot][1] = kr.frag(1, ds);
        fa[slot][2] = vr.frag(0, ds);
        fa[slot][3] = vr.frag(1, ds);
      };
      rd(0, 0);
#pragma unroll
      for (int ds = 0; ds < kDSteps; ++ds) {
        if (ds + 1 < kDSteps) rd(ds + 1, (ds + 1) & 1);
        s[0] = mfma(fa[ds & 1][0], qf[ds], s[0]);
        s[1] = mfma(fa[ds & 1][1], qf[ds], s[1]);
        dp[0] = mfma(fa[ds & 1][2], of[ds], dp[0]);
        dp[1] = mfma(fa[ds & 1][3], of[ds], dp[1]);
        sched_fence();
      }
    }
    // P and dS (into s) of register v of key sub-tile kt, whose key is
    // key0 + 32kt + 8(v/4) + 4half + v%4.
    const int room = limit - (key0 + 4 * half);
    auto grad = [&](int kt, int v) {
      const int off = kt * 32 + 8 * (v >> 2) + (v & 3);
      const float p = hw_exp2(fmaf(s[kt][v], a.c, -lse2));
      const float pm = (full || off <= room) ? p : 0.0f;
      const float d = dp[kt][v] - delta;
      const float g = pm * d;
      s[kt][v] = g * a.scale;
    };
#pragma unroll
    for (int v = 0; v < 16; ++v) grad(0, v);
    // dQ^T += K^T dS^T in 16 steps (key sub-tile kt, 16-key step st, dim tile
    // dt), transposed K fragments read two steps ahead; the vector work of
    // sub-tile 1 runs between the MFMAs of sub-tile 0.
    {
      const VReads<kQB> ktr(kreg);
      bf16x8 fk[3];
      auto rd = [&](int step, int slot) { fk[slot] = ktr.frag(step & 3, step >> 3, (step >> 2) & 1); };
      rd(0, 0);
      rd(1, 1);
      bf16x8 bf;
#pragma unroll
      for (int step = 0; step < 16; ++step) {
        if (step + 2 < 16) rd(step + 2, (step + 2) % 3);
        const int kt = step >> 3, st = (step >> 2) & 1, dt = step & 3;
        if (dt == 0) bf = pack8(s[kt], st);
        acc[dt] = mfma(fk[step % 3], bf, acc[dt]);
        if (step < 8) {
          grad(1, 2 * step);
          grad(1, 2 * step + 1);
        }
        sched_fence();
      }
    }
  }

  if (!q_ok) return;
  // acc[dt] register v: dim 32dt + 8(v/4) + 4half + v%4 of row t.
  const int64_t dst = static_cast<int64_t>(b) * a.q_bstride + (static_cast<int64_t>(t) * a.Hq + head) * kHeadDim + 4 * half;
  const bool gbf = a.grad_bf16 != 0;
#pragma unroll
  for (int dt = 0; dt < kDTiles; ++dt) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_grad4(a.dq, dst + 32 * dt + 8 * j, acc[dt][4 * j], acc[dt][4 * j + 1], acc[dt][4 * j + 2], acc[dt][4 * j + 3],
                  gbf);
  }
}

// -------------------------------------------------------------- dK / dV --

// One workgroup of 4 waves per (key block of 128, b, kv head); wave w owns
// keys 32w..32w+31 of the block, with their K and V rows as MFMA
// B-fragments in registers and their dK^T, dV^T accumulators.  The walk
// stages, for each query tile and q head, the tile's Q and dOut rows (V
// swizzle: row reads for S and dP, transposed reads for dV^T and dK^T) and
// its LSE*log2e and Delta, double-buffered.
constexpr int kKvWaves = 4;

struct KvStage {
  static constexpr int kRows = kQT * kHeadDim * 2;  // 16 KiB
  static constexpr int kQ = 0;
  static constexpr int kO = kRows;
  static constexpr int kL = 2 * kRows;
  static constexpr int kD = 2 * kRows + kQT * 4;
  static constexpr int kBytes = 2 * kRows + 2 * kQT * 4;
};

__global__ __launch_bounds__(kKvWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(const BackwardArgs a) {
  using Ld = BlockLoader<kQT, kKvWaves>;
  __shared__ __attribute__((aligned(16))) char stage[2 * KvStage::kBytes];

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  const int n_bh = a.B * a.Hkv;
  const int64_t wg = blockIdx.x;
  const int kb = static_cast<int>(wg / n_bh);  // key block 0 first: the longest walk under a causal mask
  const int bh = static_cast<int>(wg % n_bh);
  const int b = bh / a.Hkv;
  const int hk = bh % a.Hkv;
  const int kvl = static_cast<int>(a.kv_len);
  const int kw0 = kb * kKB + 32 * wave;
  const int key = kw0 + col;
  const bool key_ok = key < kvl;

  // K and V rows of this lane's key as B-fragments.
  bf16x8 kf[kDSteps], vf[kDSteps];
  {
    const int64_t e = static_cast<int64_t>(b) * a.kv_bstride + (static_cast<int64_t>(key) * a.Hkv + hk) * kHeadDim + 8 * half;
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) {
      kf[ds] = as_bf16x8(key_ok ? gload16(a.k + e + 16 * ds) : u32x4{0, 0, 0, 0});
      vf[ds] = as_bf16x8(key_ok ? gload16(a.v + e + 16 * ds) : u32x4{0, 0, 0, 0});
    }
  }
  // dK^T, dV^T accumulators: register v of tile dt is dim 32dt + 8(v/4) + 4half + v%4.
  const int64_t gout = static_cast<int64_t>(b) * a.kv_bstride + (static_cast<int64_t>(key) * a.Hkv + hk) * kHeadDim + 4 * half;
  f32x16 dk[kDTiles], dv[kDTiles];
#pragma unroll
  for (int dt = 0; dt < kDTiles; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
    if (a.accumulate && key_ok) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.dk) + gout + 32 * dt + 8 * j);
        const f32x4 y = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.dv) + gout + 32 * dt + 8 * j);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dk[dt][4 * j + i] = x[i];
          dv[dt][4 * j + i] = y[i];
        }
      }
    }
  }

  // Query tiles with a row at or after the block's first key (causal); all
  // tiles otherwise.
  const int64_t first_row = a.causal ? static_cast<int64_t>(kb) * kKB - a.pos0 : 0;
  const int t_first = first_row > 0 ? static_cast<int>(first_row / kQT) : 0;
  const int n_iter = (a.n_qtiles - t_first) * a.G;

  Ld ld;
  ld.init(a.Hq * kHeadDim);
  const int qrow_bytes = a.Hq * kHeadDim * 2;
  auto issue = [&](int i) {
    const int tile = t_first + i / a.G;
    const int h = hk * a.G + i % a.G;
    char* dst = stage + (i & 1) * KvStage::kBytes;
    const int64_t qoff = static_cast<int64_t>(b) * a.q_bstride + static_cast<int64_t>(h) * kHeadDim;
    const __amdgpu_buffer_rsrc_t qrs = head_rsrc(a.q + qoff, a.Sq, qrow_bytes);
    const __amdgpu_buffer_rsrc_t ors = head_rsrc(a.dout + qoff, a.Sq, qrow_bytes);
    ld.issue_v(dst + KvStage::kQ, qrs, static_cast<int64_t>(tile) * kQT);
    ld.issue_v(dst + KvStage::kO, ors, static_cast<int64_t>(tile) * kQT);
    if (wave < 2) {  // 64 floats of LSE*log2e (wave 0) or Delta (wave 1), 4 bytes per lane
      const float* src = a.ws + (static_cast<int64_t>(b) * a.Hq + h) * 2 * a.Sq_pad + wave * a.Sq_pad +
                         static_cast<int64_t>(tile) * kQT + lane;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + KvStage::kL + wave * kQT * 4), 4, 0, 0);
    }
  };
  if (n_iter > 0) issue(0);

  const float c = a.c;
  const float scale = a.scale;
  for (int i = 0; i < n_iter; ++i) {
    wait_direct_loads();
    lds_barrier();  // stage i staged; every wave is done with stage i-1
    if (i + 1 < n_iter) issue(i + 1);
    const int tile = t_first + i / a.G;
    const int tr0 = tile * kQT;  // first row of the tile
    const int rows_left = a.Sq - tr0;
    const int64_t pos_last = a.pos0 + min(a.Sq, tr0 + kQT) - 1;
    const bool sees = kw0 < kvl && (!a.causal || kw0 <= pos_last);
    if (!sees) continue;
    const char* base = stage + (i & 1) * KvStage::kBytes;
    const char* qreg = base + KvStage::kQ;
    const char* oreg = base + KvStage::kO;

    // LSE*log2e and Delta of the lane's rows: register v of row tile qt is
    // row r = 32qt + 8(v/4) + 4half + v%4 of the tile.
    f32x4 Lr[2][4], Dr[2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = 32 * qt + 8 * j + 4 * half;
        Lr[qt][j] = *reinterpret_cast<const f32x4*>(base + KvStage::kL + r0 * 4);
        Dr[qt][j] = *reinterpret_cast<const f32x4*>(base + KvStage::kD + r0 * 4);
      }
    }
    // Rows r of the tile that see this lane's key: rmin <= r < rmax (row in
    // range, key in range, and causally key <= pos0 + tr0 + r).
    const int rmax = key_ok ? rows_left : 0;
    const int rmin = a.causal ? max(0, key - static_cast<int>(a.pos0 + tr0)) : 0;

    // S = Q K^T and dP = dOut V^T, fragments read one D-step ahead.
    f32x16 s[2], dp[2];
    {
      const RowReadsV qr(qreg);
      const RowReadsV orr(oreg);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        s[qt] = f32x16{};
        dp[qt] = f32x16{};
      }
      bf16x8 fa[3][4];
      auto rd = [&](int ds, int slot) {
        fa[slot][0] = qr.frag(0, ds);
        fa[slot][1] = qr.frag(1, ds);
        fa[slot][2] = orr.frag(0, ds);
        fa[slot][3] = orr.frag(1, ds);
      };
      rd(0, 0);
      rd(1, 1);
#pragma unroll
      for (int ds = 0; ds < kDSteps; ++ds) {
        if (ds + 2 < kDSteps) rd(ds + 2, (ds + 2) % 3);
        s[0] = mfma(fa[ds % 3][0], kf[ds], s[0]);
        s[1] = mfma(fa[ds % 3][1], kf[ds], s[1]);
        dp[0] = mfma(fa[ds % 3][2], vf[ds], dp[0]);
        dp[1] = mfma(fa[ds % 3][3], vf[ds], dp[1]);
        sched_fence();
      }
    }
    // P (into s) and dS (into dp) of register v of row tile qt.
    auto grad = [&](int qt, int v) {
      const int j = v >> 2;
      const int e = v & 3;
      const int r = 32 * qt + 8 * j + 4 * half + e;
      const bool vis = (r >= rmin) & (r < rmax);
      const float p = hw_exp2(fmaf(s[qt][v], c, -Lr[qt][j][e]));
      const float pm = vis ? p : 0.0f;
      const float d = dp[qt][v] - Dr[qt][j][e];
      const float g = pm * d;
      s[qt][v] = pm;
      dp[qt][v] = g * scale;
    };
#pragma unroll
    for (int v = 0; v < 16; ++v) grad(0, v);
    // dV^T += dOut^T P and dK^T += Q^T dS in 16 steps (row tile qt, 16-row
    // step st, dim tile dt), transposed fragments read two steps ahead; the
    // vector work of row tile 1 runs between the MFMAs of row tile 0.
    {
      const VReads<kQT> otr(oreg);
      const VReads<kQT> qtr(qreg);
      bf16x8 fo[4], fq[4];
      auto rd = [&](int step, int slot) {
        const int qt = step >> 3, st = (step >> 2) & 1, dt = step & 3;
        fo[slot] = otr.frag(dt, qt, st);
        fq[slot] = qtr.frag(dt, qt, st);
      };
      rd(0, 0);
      rd(1, 1);
      rd(2, 2);
      bf16x8 pb, db;
#pragma unroll
      for (int step = 0; step < 16; ++step) {
        if (step + 3 < 16) rd(step + 3, (step + 3) % 4);
        const int qt = step >> 3, st = (step >> 2) & 1, dt = step & 3;
        if (dt == 0) {
          pb = pack8(s[qt], st);
          db = pack8(dp[qt], st);
        }
        dv[dt] = mfma(fo[step % 4], pb, dv[dt]);
        dk[dt] = mfma(fq[step % 4], db, dk[dt]);
        if (step < 8) {
          grad(1, 2 * step);
          grad(1, 2 * step + 1);
        }
        sched_fence();
      }
    }
  }

  if (!key_ok) return;
  const bool gbf = a.grad_bf16 != 0;
#pragma unroll
  for (int dt = 0; dt < kDTiles; ++dt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t e = gout + 32 * dt + 8 * j;
      store_grad4(a.dk, e, dk[dt][4 * j], dk[dt][4 * j + 1], dk[dt][4 * j + 2], dk[dt][4 * j + 3], gbf);
      store_grad4(a.dv, e, dv[dt][4 * j], dv[dt][4 * j + 1], dv[dt][4 * j + 2], dv[dt][4 * j + 3], gbf);
    }
  }
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, bool out_f32, hipStream_t s) {
  // dQ (also writes LSE * log2 e and Delta per row), then dK / dV
  const int64_t g1 = static_cast<int64_t>(a.B) * a.Hkv * a.hsubs * a.n_qtiles;
  if (g1 <= 0 || g1 > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (out_f32) {
    hipLaunchKernelGGL(bwd_dq_kernel<true>, dim3(static_cast<unsigned>(g1)), dim3(kDqWaves * 64), 0, s, a);
  } else {
    hipLaunchKernelGGL(bwd_dq_kernel<false>, dim3(static_cast<unsigned>(g1)), dim3(kDqWaves * 64), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t g2 = static_cast<int64_t>(a.B) * a.Hkv * a.n_kblocks;
  if (g2 <= 0) return hipSuccess;
  if (g2 > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(static_cast<unsigned>(g2)), dim3(kKvWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace rla
