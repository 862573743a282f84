// Fold of per-block partial states (gfx950): the merge of emulated
// context-parallel shards and pass 2 of paged decode.
//
// One wave per (row, q head): lane l owns dims 2l and 2l+1.  The items are
// folded with the scalar and element steps of core.hpp in the order given
// (merge: the part order sorted by global block index on the host; decode:
// ascending block index, continuing from the running state the sequence's
// head unit left after its blocks, or nothing at all when the head unit
// covered the sequence and wrote the row itself), then finalized and written
// (bf16 RNE or fp32) with the natural-log LSE.  These are the same operations, in the same order, as
// the fold inside the fused prefill kernel, so a merge of per-block states
// reproduces the fused result bit for bit.
#include "kernels.hpp"
#include "core.hpp"

namespace rla {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kBatch = 32;  // items in flight per wave

template <bool DECODE, bool F32>
__global__ __launch_bounds__(kThreads) void fold_kernel(const FoldArgs a) {
  // wave index made provably uniform: the row, its item count and every
  // per-item condition below are then scalar, and the conditions scalar
  // branches
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kWaves + wave;  // row * Hq + head
  if (item >= a.rows * a.Hq) return;
  const int64_t row = item / a.Hq;
  const int head = static_cast<int>(item % a.Hq);

  int n;
  int start = 0;  // first item to fold
  FoldState st{kNegInf, 0.0f};
  float acc0 = 0.0f, acc1 = 0.0f;
  if constexpr (DECODE) {
    int64_t len = a.uniform_len;
    if (a.len_mode == kLensTable) len = a.lens[row];
    if (a.len_mode == kLensDevice) len = a.ctx_lens[row];
    len = len < 0 ? 0 : (len > a.len_cap ? a.len_cap : len);
    n = __builtin_amdgcn_readfirstlane(static_cast<int>((len + a.block - 1) / a.block));  // one row per wave
    // The sequence's head unit folded blocks [0, head_blocks) already: it
    // wrote the final row itself when that was all of them, else its running
    // state (acc in block slot 0, m and l in the LSE of slots 0 and 1).
    if (n > 0 && n <= a.head_blocks) return;
    if (n > a.head_blocks) {
      const int64_t i0 = row * a.n_parts * a.Hq + head;
      st.m = a.part_lse[i0];
      st.l = a.part_lse[i0 + a.Hq];
      const float2 x = *reinterpret_cast<const float2*>(a.part_out + i0 * kHeadDim + 2 * lane);
      acc0 = x.x;
      acc1 = x.y;
      start = a.head_blocks;
    }
  } else {
    n = a.n_parts;
  }

  // Items are loaded kBatch at a time (all loads in flight together), then
  // folded one by one in order.
  for (int i0 = start; i0 < n; i0 += kBatch) {
    float L[kBatch];
    float2 o[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + j;
      L[j] = kNegInf;
      o[j] = float2{0.0f, 0.0f};
      if (i < n) {
        int64_t idx;  // index of the item's (row, head) record
        if constexpr (DECODE) {
          idx = (row * a.n_parts + i) * a.Hq + head;
        } else {
          idx = (static_cast<int64_t>(a.order[i]) * a.rows + row) * a.Hq + head;
        }
        L[j] = a.part_lse[idx];
        o[j] = *reinterpret_cast<const float2*>(a.part_out + idx * kHeadDim + 2 * lane);
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (i0 + j < n) {
        const FoldStep f = fold_scalars(st, L[j]);
        acc0 = fold_elem(f, acc0, o[j].x);
        acc1 = fold_elem(f, acc1, o[j].y);
      }
    }
  }
  const Final fin = finalize(st);
  const float o0 = acc0 * fin.r;
  const float o1 = acc1 * fin.r;
  const int64_t base = item * kHeadDim + 2 * lane;
  if constexpr (F32) {
    *reinterpret_cast<float2*>(static_cast<float*>(a.out) + base) = float2{o0, o1};
  } else {
    *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.out) + base) = pack_bf16(o0, o1);
  }
  if (lane == 0) a.lse[item] = fin.lse;
}

template <bool DECODE, bool F32>
hipError_t launch_t(const FoldArgs& a, hipStream_t s) {
  const int64_t items = a.rows * a.Hq;
  const int64_t grid = (items + kWaves - 1) / kWaves;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fold_kernel<DECODE, F32>), dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fold(const FoldArgs& a, bool decode, bool out_f32, hipStream_t s) {
  if (decode) return out_f32 ? launch_t<true, true>(a, s) : launch_t<true, false>(a, s);
  return out_f32 ? launch_t<false, true>(a, s) : launch_t<false, false>(a, s);
}

}  // namespace rla
