// Paged-KV decode, pass 1 (gfx950): one workgroup per (kv head, unit of
// consecutive KV blocks of one sequence) computes each block's partial state
// for the q heads of the group.  A sequence's head unit (its first blocks, up
// to 64 of them) folds those states in registers, in block order from the
// empty state, with the fold pass's own steps, and writes the finished row
// (when it covers the sequence) or its running state; the tail units write
// every block's state to the caller's workspace, and pass 2 (fold.hip)
// continues the fold from the head's state over them in ascending block
// index.  Folding in the head unit saves most of the item writes (which cost
// far more than their share of the bytes) and most of the per-workgroup
// set-up.  The cut into units is fixed by the lengths alone and never changes
// what any block's state holds or the order it is folded in.  Decode is bound
// by reading the KV cache, so each workgroup keeps two register sets of blocks
// (K as MFMA A-fragments, V rows bound for LDS) and refills a set with the
// block two ahead as soon as its registers are free: V right after it is
// staged in LDS, K right after the score MFMAs have read it.  Two workgroups
// share a CU.
//
// Keys are gathered through the page table: key j of sequence s is slot j % P
// of page page_table[s][j / P] in a pool laid out [page][kv head][slot][dim].
// The per-(row, block) arithmetic is the same as in the prefill kernel (same
// fragments, MFMA shape and operand order, softmax tree and PV chain), only
// split over the four waves: wave w computes score sub-tile w and output dim
// tile w, and the block max, sub-tile sums and bf16 P go through LDS.  Rows
// are the group's q heads for the one query token (columns >= G are zero).
#include <mutex>

#include "kernels.hpp"
#include "tile.hpp"

namespace rla {

namespace {

constexpr int kThreads = 256;

template <int BK, bool F32>
struct DecodeLds {
  static constexpr int NKT = BK / 32;
  static constexpr int kPBytesPerTile = 64 * 32 * (F32 ? 2 : 1);  // 64 lanes x 16 bf16 (x2 hi/lo)
  static constexpr int kMaxUnitPages = kDecodeIdsCap;              // page ids of one unit
  static constexpr int kVOff = 0;                                 // V region only (no K in LDS)
  static constexpr int kPOff = TileLayout<BK>::kVBytes;
  static constexpr int kMaxOff = kPOff + NKT * kPBytesPerTile;
  static constexpr int kSumOff = kMaxOff + NKT * 32 * 4;
  static constexpr int kPageOff = kSumOff + NKT * 32 * 4;
  // a tail unit's items: [block of the unit][head of the group][D] fp32, then
  // the LSEs [block][head]
  static constexpr int kStageOff = kPageOff + kMaxUnitPages * 4;
  static constexpr int kStageLseOff = kStageOff + kDecodeUnitBlocks * kDecodeStageHeads * kHeadDim * 4;
  static constexpr int kBytes = kStageLseOff + kDecodeUnitBlocks * kDecodeStageHeads * 4;
};

// The unit's slice of the page table, copied to LDS once so that the per-row
// page lookups are LDS reads and never wait behind the KV loads in flight
// (vector loads retire in order).
struct UnitPages {
  const int32_t* ids;  // LDS: page ids of pages first .. first+count-1 of the sequence
  int first;
};

// Element offset of key `key` (a key of the unit, key < len) of kv head hk in
// the pool.  Page ids outside [0, num_pages) are clamped into the pool, so a
// bad table cannot fault (its result is unspecified).
__device__ __forceinline__ int64_t page_row_off(const DecodeArgs& a, const UnitPages& up, int hk, int key) {
  int page = up.ids[(key >> a.log2_P) - up.first];
  page = page < 0 ? 0 : (page >= a.num_pages ? static_cast<int>(a.num_pages - 1) : page);
  const int64_t row = ((static_cast<int64_t>(page) * a.Hkv + hk) << a.log2_P) + (key & ((1 << a.log2_P) - 1));
  return row * kHeadDim;
}

// Registers holding one KV block in flight: the calling wave's K sub-tile as
// MFMA A-fragments (waves < NKT) and this thread's share of V rows.  Rows past
// len read key len-1 instead (their scores are masked, their weights are 0).
template <int BK>
struct BlockRegs {
  static constexpr int NKT = BK / 32;
  static constexpr int VIT = BK * 16 / kThreads;  // 16-byte V chunks per thread
  u32x4 k[kDSteps];
  u32x4 v[VIT];

  __device__ __forceinline__ void load(const DecodeArgs& a, const UnitPages& up, int hk, int key0, int len) {
    load_k(a, up, hk, key0, len);
    load_v(a, up, hk, key0, len);
  }
  __device__ __forceinline__ void load_k(const DecodeArgs& a, const UnitPages& up, int hk, int key0, int len) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    if (wave < NKT) {
      const int key = min(key0 + wave * 32 + (lane & 31), len - 1);
      const uint16_t* row = a.k_pool + page_row_off(a, up, hk, key) + 8 * (lane >> 5);
#pragma unroll
      for (int ds = 0; ds < kDSteps; ++ds) k[ds] = gload16(row + 16 * ds);
    }
  }
  __device__ __forceinline__ void load_v(const DecodeArgs& a, const UnitPages& up, int hk, int key0, int len) {
    const int tid = threadIdx.x;
    const int c = tid & 15;
    int64_t off[VIT];
#pragma unroll
    for (int i = 0; i < VIT; ++i) off[i] = page_row_off(a, up, hk, min(key0 + (tid >> 4) + (kThreads / 16) * i, len - 1));
#pragma unroll
    for (int i = 0; i < VIT; ++i) v[i] = gload16(a.v_pool + off[i] + 8 * c);
  }

  // V rows into the (key-major, swizzled) V region of TileLayout.
  __device__ __forceinline__ void store_v(char* lv) const {
    using L = TileLayout<BK>;
    const int tid = threadIdx.x;
    const int c = tid & 15;
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int r = (tid >> 4) + (kThreads / 16) * i;
      *reinterpret_cast<u32x4*>(lv + L::v_rel(r, c)) = v[i];
    }
  }
};

__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int seq) {
  const int len = a.len_mode == kLensDevice ? a.ctx_lens[seq] : a.uniform_len;
  return len < 0 ? 0 : (len > a.len_cap ? a.len_cap : len);
}

// Map a unit index to (sequence, first block, end block, head or tail);
// false for an idle unit.  Units [0, Bd) are the sequences' head units
// (kLensTable: in head_order), blocks [0, min(nb, head_blocks)); the rest are
// tail units of up to
// unit_blocks blocks from head_blocks on.  kLensTable: a tail's sequence is
// the last one whose first tail unit (unit_start, a prefix sum the host built
// from the lengths) is <= its index, found by a binary search over the launch
// arguments, so no workgroup waits on a device-memory read before its first
// KV load.  kLensUniform: every sequence has the same number of tails.
// kLensDevice: tail t is tail t / Bd of sequence t % Bd (the grid covers
// max_context_len; tails past a sequence's length are idle).
template <int BK>
__device__ __forceinline__ bool locate_unit(const DecodeArgs& a, uint32_t u, int& seq, int& blk0, int& blk1, int& len,
                                            bool& head) {
  const int U = a.unit_blocks;
  const int H = a.head_blocks;
  const uint32_t bd = static_cast<uint32_t>(a.Bd);
  head = u < bd;
  uint32_t k = 0;  // tail index within the sequence
  if (head) {
    seq = a.len_mode == kLensTable ? a.head_order[u] : static_cast<int>(u);
    len = a.len_mode == kLensTable ? a.lens[seq] : clamp_len(a, seq);
  } else {
    const uint32_t t = u - bd;
    if (a.len_mode == kLensTable) {
      int lo = 0, hi = a.Bd;  // unit_start[lo] <= t < unit_start[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (static_cast<uint32_t>(a.unit_start[mid]) <= t) {
          lo = mid;
        } else {
          hi = mid;
        }
      }
      seq = lo;
      len = a.lens[lo];
      k = t - static_cast<uint32_t>(a.unit_start[lo]);
    } else if (a.len_mode == kLensUniform) {
      len = clamp_len(a, 0);
      const int nb = (len + BK - 1) / BK;
      const uint32_t per = static_cast<uint32_t>(nb > H ? (nb - H + U - 1) / U : 0);
      if (per == 0) return false;
      seq = static_cast<int>(t / per);
      k = t - static_cast<uint32_t>(seq) * per;
    } else {
      seq = static_cast<int>(t % bd);
      len = clamp_len(a, seq);
      k = t / bd;
    }
  }
  const int nb = (len + BK - 1) / BK;
  if (head) {
    blk0 = 0;
    blk1 = min(nb, H);
  } else {
    blk0 = H + static_cast<int>(k) * U;
    blk1 = min(blk0 + U, nb);
  }
  return blk0 < blk1;
}

// Running fold of a head unit, per lane: the state of the lane's column
// (q head) and the accumulator of its 16 output elements.
struct HeadFold {
  FoldState st;
  float acc[16];
};

// One block's partial states for the group's heads, from the K fragments in
// registers (waves < NKT) and the V tile in LDS.  A head unit folds them into
// hf (the fold pass's scalar and element steps, in block order); a tail unit
// writes them to the items.
template <int BK, bool F32>
__device__ __forceinline__ void decode_block(const DecodeArgs& a, char* lds, BlockRegs<BK>& br,
                                             const bf16x8 (&qf)[kDSteps], int seq, int hk, int blk, int len,
                                             const UnitPages& up, int next_key0, bool head, HeadFold& hf,
                                             int slot) {
  using Lay = DecodeLds<BK, F32>;
  constexpr int NKT = Lay::NKT;
  const char* lv = lds + Lay::kVOff;  // V rows at lv + TileLayout::v_rel(...)
  char* lp = lds + Lay::kPOff;
  float* red_max = reinterpret_cast<float*>(lds + Lay::kMaxOff);
  float* red_sum = reinterpret_cast<float*>(lds + Lay::kSumOff);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int key0 = blk * BK;

  // ---- scores of sub-tile kt = wave (waves < NKT)
  f32x16 s = f32x16{};
  if (wave < NKT) {
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) s = mfma(as_bf16x8(br.k[ds]), qf[ds], s);
    // K of the block two ahead, into the registers the MFMAs just read (the
    // fp32-output instance, short of registers, loads it after the block)
    if constexpr (!F32) {
      if (next_key0 >= 0) br.load_k(a, up, hk, next_key0, len);
    }
    float m_lane = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kk = key0 + wave * 32 + acc_row(v, half);
      const float d = kk < len ? s[v] : kNegInf;
      s[v] = d;
      m_lane = fmaxf(m_lane, d);
    }
    m_lane = pair_max(m_lane);
    if (half == 0) red_max[wave * 32 + col] = m_lane;
  }
  lds_barrier();

  float mx = red_max[col];
#pragma unroll
  for (int kt = 1; kt < NKT; ++kt) mx = fmaxf(mx, red_max[kt * 32 + col]);
  const float m_t = block_m(mx, a.c);
  const float m_use = block_m_use(m_t);

  if (wave < NKT) {
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = block_p(s[v], a.c, m_use);
    const float aa = tree16(s);
    const float sum = pair_sum(aa);
    if (half == 0) red_sum[wave * 32 + col] = sum;
    u32x4 ph[2], pl[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = s[8 * st + 2 * w];
        const float p1 = s[8 * st + 2 * w + 1];
        const uint32_t h = pack_bf16(p0, p1);
        ph[st][w] = h;
        if constexpr (F32) pl[st][w] = pack_bf16(p0 - bf16_lo_to_f32(h), p1 - bf16_hi_to_f32(h));
      }
    }
    char* my = lp + wave * Lay::kPBytesPerTile + lane * (F32 ? 64 : 32);
    *reinterpret_cast<u32x4*>(my) = ph[0];
    *reinterpret_cast<u32x4*>(my + 16) = ph[1];
    if constexpr (F32) {
      *reinterpret_cast<u32x4*>(my + 32) = pl[0];
      *reinterpret_cast<u32x4*>(my + 48) = pl[1];
    }
  }
  lds_barrier();

  float sub[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) sub[kt] = red_sum[kt * 32 + col];
  const float l_b = combine_subtiles<NKT>(sub);

  // ---- PV for output dim tile dt = wave
  const int dt = wave;
  f32x16 acc = f32x16{};
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const char* pp = lp + kt * Lay::kPBytesPerTile + lane * (F32 ? 64 : 32);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const bf16x8 vf = v_frag<BK>(lv, dt, kt, st);
      acc = mfma(vf, as_bf16x8(lds_load16(pp, 16 * st)), acc);
      if constexpr (F32) acc = mfma(vf, as_bf16x8(lds_load16(pp, 32 + 16 * st)), acc);
    }
  }
  const ItemScalars sc = item_scalars(m_t, l_b);
  if (head) {
    const FoldStep f = fold_scalars(hf.st, sc.L);
#pragma unroll
    for (int i = 0; i < 16; ++i) hf.acc[i] = fold_elem(f, hf.acc[i], item_out(acc[i], sc));
  } else if (col < a.G) {
    // tail unit: the items wait in LDS for the unit's end (written after the
    // block loop)
    float* so = reinterpret_cast<float*>(lds + Lay::kStageOff) + (slot * kDecodeStageHeads + col) * kHeadDim;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = dt * 32 + 8 * g + 4 * half;
      *reinterpret_cast<f32x4*>(so + d) = f32x4{item_out(acc[4 * g], sc), item_out(acc[4 * g + 1], sc),
                                                item_out(acc[4 * g + 2], sc), item_out(acc[4 * g + 3], sc)};
    }
    float* sl = reinterpret_cast<float*>(lds + Lay::kStageLseOff);
    if (wave == 0 && half == 0) sl[slot * kDecodeStageHeads + col] = sc.L;
  }
  if constexpr (F32) {
    if (next_key0 >= 0) br.load_k(a, up, hk, next_key0, len);
  }
}

// Blocks of the unit are processed in pairs so that the two register sets
// have static indices: while block b is computed, block b+1 is already in
// registers (or in flight) and block b+2 is being loaded into the set of b.
template <int BK, bool F32>
__global__ __launch_bounds__(kThreads, 2) void decode_items_kernel(const DecodeArgs a) {
  using Lay = DecodeLds<BK, F32>;
  __shared__ __attribute__((aligned(16))) char lds[Lay::kBytes];
  char* lv = lds + Lay::kVOff;

  const uint32_t x = blockIdx.x;
  const uint32_t hkv = static_cast<uint32_t>(a.Hkv);
  const int hk = static_cast<int>(x % hkv);
  int seq;
  int blk0, blk1, len;
  bool head;
  if (!locate_unit<BK>(a, x / hkv, seq, blk0, blk1, len, head)) return;  // uniform across the workgroup

  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  // page ids covering the unit's keys [blk0*BK, min(blk1*BK, len))
  UnitPages up;
  {
    int32_t* ids = reinterpret_cast<int32_t*>(lds + Lay::kPageOff);
    up.ids = ids;
    up.first = (blk0 * BK) >> a.log2_P;
    const int kend = min(blk1 * BK, len);
    const int count = ((kend + a.P - 1) >> a.log2_P) - up.first;
    const int32_t* row = a.page_table + static_cast<int64_t>(seq) * a.max_pages + up.first;
    const int32_t id0 = seq * a.max_pages + up.first;  // no table: page i of sequence s is s*max_pages + i
    for (int t = threadIdx.x; t < count; t += kThreads)
      ids[t] = a.page_table != nullptr ? row[t] : id0 + static_cast<int32_t>(t);
    __syncthreads();
  }

  BlockRegs<BK> r0, r1;
  r0.load(a, up, hk, blk0 * BK, len);
  if (blk0 + 1 < blk1) r1.load(a, up, hk, (blk0 + 1) * BK, len);

  // Q fragments of the group's heads (columns >= G are zero)
  bf16x8 qf[kDSteps];
  {
    const bool qok = col < a.G;
    const uint16_t* qrow = a.q + (static_cast<int64_t>(seq) * a.Hq + hk * a.G + (qok ? col : 0)) * kHeadDim + 8 * half;
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) qf[ds] = as_bf16x8(qok ? gload16(qrow + 16 * ds) : u32x4{0, 0, 0, 0});
  }

  HeadFold hf;
  hf.st = FoldState{kNegInf, 0.0f};
#pragma unroll
  for (int i = 0; i < 16; ++i) hf.acc[i] = 0.0f;

  for (int blk = blk0; blk < blk1; blk += 2) {
    const int n0 = blk + 2 < blk1 ? (blk + 2) * BK : -1;
    r0.store_v(lv);
    if (n0 >= 0) r0.load_v(a, up, hk, n0, len);
    lds_barrier();  // V of blk visible
    decode_block<BK, F32>(a, lds, r0, qf, seq, hk, blk, len, up, n0, head, hf, blk - blk0);
    lds_barrier();  // everyone done with V / P of blk
    if (blk + 1 < blk1) {
      const int n1 = blk + 3 < blk1 ? (blk + 3) * BK : -1;
      r1.store_v(lv);
      if (n1 >= 0) r1.load_v(a, up, hk, n1, len);
      lds_barrier();
      decode_block<BK, F32>(a, lds, r1, qf, seq, hk, blk + 1, len, up, n1, head, hf, blk + 1 - blk0);
      lds_barrier();
    }
  }

  // A tail unit writes its items now, after its last wait for KV loads: item
  // stores count in the same in-order counter as the loads, so a store issued
  // between blocks would make the next block's wait for its KV data also wait
  // for the store's completion, which under the full read stream is slow.
  // (The loop's last barrier made the staged items visible.)
  if (!head) {
    const int per = a.G * (kHeadDim / 4);  // 16-byte chunks of one block's items
    const int n = (blk1 - blk0) * per;
    const char* so = lds + Lay::kStageOff;
    for (int c = threadIdx.x; c < n; c += kThreads) {
      const int j = c / per;
      const int r = c - j * per;
      const int64_t item0 = (static_cast<int64_t>(seq) * a.max_blocks + blk0 + j) * a.Hq + hk * a.G;
      *reinterpret_cast<f32x4*>(a.items_out + item0 * kHeadDim + 4 * r) =
          *reinterpret_cast<const f32x4*>(so + (j * kDecodeStageHeads * kHeadDim + 4 * r) * 4);
    }
    const float* sl = reinterpret_cast<const float*>(lds + Lay::kStageLseOff);
    for (int c = threadIdx.x; c < (blk1 - blk0) * a.G; c += kThreads) {
      const int j = c / a.G;
      const int h = c - j * a.G;
      a.items_lse[(static_cast<int64_t>(seq) * a.max_blocks + blk0 + j) * a.Hq + hk * a.G + h] =
          sl[j * kDecodeStageHeads + h];
    }
  }

  // A head unit that covers its sequence finalizes it as the fold pass would
  // (O = acc * (1 / l), rounded once at this write); otherwise it leaves its
  // running state for the fold pass: acc in block slot 0, m and l in the LSE
  // of block slots 0 and 1.
  if (head && col < a.G) {
    const int wave = threadIdx.x >> 6;
    const int hq = hk * a.G + col;
    const bool last = blk1 * BK >= len;
    if (last) {
      const Final fin = finalize(hf.st);
      const int64_t row = (static_cast<int64_t>(seq) * a.Hq + hq) * kHeadDim;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = wave * 32 + 8 * g + 4 * half;
        const float o0 = hf.acc[4 * g] * fin.r, o1 = hf.acc[4 * g + 1] * fin.r;
        const float o2 = hf.acc[4 * g + 2] * fin.r, o3 = hf.acc[4 * g + 3] * fin.r;
        if constexpr (F32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row + d) = f32x4{o0, o1, o2, o3};
        } else {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + row + d) = u32x2{pack_bf16(o0, o1), pack_bf16(o2, o3)};
        }
      }
      if (wave == 0 && half == 0) a.lse[static_cast<int64_t>(seq) * a.Hq + hq] = fin.lse;
    } else {
      const int64_t item0 = static_cast<int64_t>(seq) * a.max_blocks * a.Hq + hq;  // block slot 0
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = wave * 32 + 8 * g + 4 * half;
        *reinterpret_cast<f32x4*>(a.items_out + item0 * kHeadDim + d) =
            f32x4{hf.acc[4 * g], hf.acc[4 * g + 1], hf.acc[4 * g + 2], hf.acc[4 * g + 3]};
      }
      if (wave == 0 && half == 0) {
        a.items_lse[item0] = hf.st.m;
        a.items_lse[item0 + a.Hq] = hf.st.l;  // block slot 1
      }
    }
  }
}

template <int BK, bool F32>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  const int64_t grid = a.n_units * a.Hkv;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_items_kernel<BK, F32>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Block items of rla_attn_decode_paged_static (callers that cannot allocate):
// a fixed device array, one copy per GPU the library runs on, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it only stands for the symbol); it uses the address
// hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) char scratch[kStaticDecodeScratchBytes];

void* static_decode_scratch(hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    ptrs[dev] = ptr;
  }
  *err = hipSuccess;
  return ptrs[dev];
}

hipError_t launch_decode_items(const DecodeArgs& a, int block, bool out_f32, hipStream_t s) {
  if (block == 128) return out_f32 ? launch_t<128, true>(a, s) : launch_t<128, false>(a, s);
  if (block == 64) return out_f32 ? launch_t<64, true>(a, s) : launch_t<64, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace rla
