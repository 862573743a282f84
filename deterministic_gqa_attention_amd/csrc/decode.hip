// Paged-KV decode, pass 1 (gfx950): one workgroup per (sequence, kv head,
// KV block) computes the block's partial state for the q heads of the group
// and writes it to the caller's workspace; pass 2 (fold.hip) folds the items
// of each row in ascending block index.
//
// Keys are gathered through the page table: key j of sequence s is slot j % P
// of page page_table[s][j / P] in a pool laid out [page][kv head][slot][dim];
// the workgroup stages the block in LDS with direct global->LDS loads whose
// per-lane source addresses do the gather.  The per-(row, block) arithmetic is
// the same as in the prefill kernel (same LDS layout and fragments, same MFMA
// shape and operand order, same softmax tree, same PV chain), only split over
// the four waves: wave w computes score sub-tile w and output dim tile w, and
// the block max, sub-tile sums and bf16 P go through LDS.  Rows are the
// group's q heads for the one query token (columns >= G are zero padding).
#include "kernels.hpp"
#include "tile.hpp"

namespace rla {

namespace {

constexpr int kThreads = 256;

template <int BK, bool F32>
struct DecodeLds {
  static constexpr int NKT = BK / 32;
  static constexpr int kPBytesPerTile = 64 * 32 * (F32 ? 2 : 1);  // 64 lanes x 16 bf16 (x2 hi/lo)
  static constexpr int kPOff = TileLayout<BK>::kBytes;
  static constexpr int kMaxOff = kPOff + NKT * kPBytesPerTile;
  static constexpr int kSumOff = kMaxOff + NKT * 32 * 4;
  static constexpr int kBytes = kSumOff + NKT * 32 * 4;
};

// Element offset of key `key` of sequence `seq`, kv head hk, in the pool.
// key < len <= len_cap <= max_pages * P keeps the table read in its row; a
// page id outside [0, num_pages) is never dereferenced (ok = false).
__device__ __forceinline__ int64_t page_row_off(const DecodeArgs& a, int seq, int hk, int64_t key, bool& ok) {
  const int32_t page = a.page_table[static_cast<int64_t>(seq) * a.max_pages + key / a.P];
  ok = page >= 0 && page < a.num_pages;
  return ((static_cast<int64_t>(ok ? page : 0) * a.Hkv + hk) * a.P + key % a.P) * kHeadDim;
}

// Direct global->LDS loads of one KV block gathered through the page table,
// in the layout of TileLayout (rows past len load key len-1: masked).
template <int BK>
__device__ __forceinline__ void issue_paged_loads(char* buf, const DecodeArgs& a, int seq, int hk, int64_t key0,
                                                  int64_t len) {
  using L = TileLayout<BK>;
  constexpr int NW = kThreads / 64;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int p = lane & 15;
#pragma unroll
  for (int i = 0; i < L::kLoadsPerRegion / NW; ++i) {
    const int n = wave + NW * i;
    const int r = 4 * n + (lane >> 4);
    int64_t key = key0 + r;
    key = key < len ? key : len - 1;
    bool ok;
    const int64_t off = page_row_off(a, seq, hk, key, ok);  // ok == false: page 0 row (masked or caller error)
    direct_load16(a.k_pool + off + ((p ^ L::k_swz(r)) << 3), buf + n * 1024);
    direct_load16(a.v_pool + off + ((p ^ L::v_swz(r)) << 3), buf + L::kKBytes + n * 1024);
  }
}

template <int BK, bool F32>
__global__ __launch_bounds__(kThreads) void decode_items_kernel(const DecodeArgs a) {
  using Lay = DecodeLds<BK, F32>;
  constexpr int NKT = Lay::NKT;
  __shared__ __attribute__((aligned(16))) char lds[Lay::kBytes];
  char* lp = lds + Lay::kPOff;
  float* red_max = reinterpret_cast<float*>(lds + Lay::kMaxOff);
  float* red_sum = reinterpret_cast<float*>(lds + Lay::kSumOff);

  const int64_t x = blockIdx.x;
  const int hk = static_cast<int>(x % a.Hkv);
  const int seq = static_cast<int>((x / a.Hkv) % a.Bd);
  const int64_t blk = x / (static_cast<int64_t>(a.Hkv) * a.Bd);
  int64_t len = a.ctx_lens[seq];
  len = len < 0 ? 0 : (len > a.len_cap ? a.len_cap : len);
  const int64_t nb = (len + BK - 1) / BK;
  if (blk >= nb) return;  // uniform across the workgroup
  const int64_t key0 = blk * BK;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  issue_paged_loads<BK>(lds, a, seq, hk, key0, len);

  // Q fragments of the group's heads (columns >= G are zero)
  bf16x8 qf[kDSteps];
  {
    const bool qok = col < a.G;
    const uint16_t* qrow = a.q + (static_cast<int64_t>(seq) * a.Hq + hk * a.G + (qok ? col : 0)) * kHeadDim + 8 * half;
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) qf[ds] = as_bf16x8(qok ? gload16(qrow + 16 * ds) : u32x4{0, 0, 0, 0});
  }
  wait_direct_loads();
  __syncthreads();

  // ---- scores of sub-tile kt = wave (waves < NKT)
  f32x16 s = f32x16{};
  if (wave < NKT) {
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) s = mfma(k_frag<BK>(lds, wave, ds, col, half), qf[ds], s);
    float m_lane = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t kk = key0 + wave * 32 + acc_row(v, half);
      const float d = kk < len ? s[v] : kNegInf;
      s[v] = d;
      m_lane = fmaxf(m_lane, d);
    }
    m_lane = fmaxf(m_lane, partner(m_lane));
    if (half == 0) red_max[wave * 32 + col] = m_lane;
  }
  __syncthreads();

  float mx = red_max[col];
#pragma unroll
  for (int kt = 1; kt < NKT; ++kt) mx = fmaxf(mx, red_max[kt * 32 + col]);
  const float m_t = block_m(mx, a.c);
  const float m_use = block_m_use(m_t);

  if (wave < NKT) {
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = block_p(s[v], a.c, m_use);
    const float aa = tree16(s);
    const float sum = aa + partner(aa);
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
  __syncthreads();

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
      const bf16x8 vf = v_frag<BK>(lds, dt, kt, st);
      acc = mfma(vf, as_bf16x8(lds_load16(pp, 16 * st)), acc);
      if constexpr (F32) acc = mfma(vf, as_bf16x8(lds_load16(pp, 32 + 16 * st)), acc);
    }
  }
  const ItemScalars sc = item_scalars(m_t, l_b);
  if (col < a.G) {
    const int head = hk * a.G + col;
    const int64_t item = (static_cast<int64_t>(seq) * a.max_blocks + blk) * a.Hq + head;
    float* po = a.items_out + item * kHeadDim;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = dt * 32 + 8 * g + 4 * half;
      *reinterpret_cast<f32x4*>(po + d) = f32x4{item_out(acc[4 * g], sc), item_out(acc[4 * g + 1], sc),
                                                item_out(acc[4 * g + 2], sc), item_out(acc[4 * g + 3], sc)};
    }
    if (wave == 0 && half == 0) a.items_lse[item] = sc.L;
  }
}

template <int BK, bool F32>
hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
  const int64_t grid = static_cast<int64_t>(a.max_blocks) * a.Bd * a.Hkv;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_items_kernel<BK, F32>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_items(const DecodeArgs& a, int block, bool out_f32, hipStream_t s) {
  if (block == 128) return out_f32 ? launch_t<128, true>(a, s) : launch_t<128, false>(a, s);
  if (block == 64) return out_f32 ? launch_t<64, true>(a, s) : launch_t<64, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace rla
