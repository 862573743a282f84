// Selected log-probability through an FP32 lm_head (gfx950): for active
// token t with attention output x_t (its Out row, all q heads side by side)
// and token id y_t,
//   z_tv = sum_h x_th W_vh,   logp_t = z_{t,y_t} - ln sum_v exp(z_tv).
// The pages ("WS2 Attention PR5 Drift Benchmark", section "Scope") project
// both attention outputs of a drift comparison through one deterministic
// synthetic FP32 lm_head and compare the active tokens' selected log-probs;
// "[WS2][Attention] H100 validation and reproduction guide", section
// "Status", reports that drift as max abs 0.0 between decode and prefill.
//
// Determinism: every logit is one FP32 MFMA (32x32x2) chain over the hidden
// dimension in a fixed order (visits of 32 values in ascending order; inside
// visit J the pairs (32J + 4c + i, 32J + 16 + 4c + i) for c, i = 0..3; a
// hidden size that is not a multiple of 128 finishes with groups of 8, pairs
// (8j + i, 8j + 4 + i)), and a token's logit depends only on its own MFMA
// column, so batch makeup changes nothing.  Each wave owns 32 vocabulary rows
// and 64 tokens; its lanes read 64 contiguous bytes of a W row per visit (the
// two halves of the wave cover a 128-byte line), three visits ahead of the
// MFMAs.  Pass 1 writes, per (32-row vocabulary block, token), the block max
// and the fixed-tree sum of exp(z - max) (and the selected logit from the
// block that holds y_t); pass 2 folds the blocks: M = max of the block
// maxima, S = sum_b s_b exp(m_b - M) in a fixed order (four contiguous
// quarters, lanes strided in ascending order inside each, fixed trees
// across lanes and quarters), logZ = M + ln S.
#include <type_traits>

#include "kernels.hpp"
#include "core.hpp"

namespace rla {

namespace {

constexpr int kRowsPerWave = 32;  // vocabulary rows per wave (one 32-row MFMA tile)
constexpr int kNRT = kRowsPerWave / 32;
constexpr int kTokPerWave = 64;   // tokens per wave (two 32-column MFMA tiles)
constexpr int kWaves = 4;

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Raw bits of four consecutive x values of token row t from h (t is clamped
// into [0, T): columns of tokens past T are computed from a valid row and
// never written), and their fp32 values.  Loading and widening are separate
// so a load can be issued long before its values are needed.
template <bool XF32>
struct XRaw {
  using T = typename std::conditional<XF32, f32x4, u32x2>::type;
};
template <bool XF32>
__device__ __forceinline__ typename XRaw<XF32>::T load_x4(const LmHeadArgs& a, int t, int h) {
  const int64_t e = static_cast<int64_t>(min(t, a.T - 1)) * a.H + h;
  if constexpr (XF32) {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + e);
  } else {
    return *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.x) + e);
  }
}
__device__ __forceinline__ float x_val(const f32x4& r, int i) { return r[i]; }
__device__ __forceinline__ float x_val(const u32x2& r, int i) {
  return (i & 1) ? bf16_hi_to_f32(r[i >> 1]) : bf16_lo_to_f32(r[i >> 1]);
}

// Pass 1.  Grid: (vocabulary group of 4 x 32 rows) x (token group of 64),
// token groups fastest so neighbouring workgroups read the same W rows.
template <bool XF32>
__global__ __launch_bounds__(kWaves * 64) void lmh_partial_kernel(const LmHeadArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int tg = static_cast<int>(blockIdx.x % a.n_tgroups);
  const int vg = static_cast<int>(blockIdx.x / a.n_tgroups);
  const int vblk = vg * kWaves + wave;  // 32-row vocabulary block of this wave
  if (vblk >= a.n_vblocks) return;
  const int v0 = vblk * kRowsPerWave;
  const int t0 = tg * kTokPerWave;

  // Lane l reads W row v0 + l%32 and x rows t0 + l%32, t0 + 32 + l%32, four
  // values from 8j + 4half each, two groups ahead of the MFMAs.
  const int r0 = min(v0 + col, a.V - 1);  // rows past V read row V-1 (masked below)
  const float* w0 = a.w + static_cast<int64_t>(r0) * a.H + 4 * half;
  const int ta = t0 + col, tb = t0 + 32 + col;

  f32x16 acc[kNRT][2];
  acc[0][0] = f32x16{};
  acc[0][1] = f32x16{};
  // Per visit of 32 hidden values, lane l reads 16 consecutive W values of
  // its row (64 bytes, so the two halves cover a 128-byte line) and the same
  // 16 x values of its two token rows; MFMA step (c, i) of visit J contracts
  // the pair (32J + 4c + i, 32J + 16 + 4c + i).  Visits run three ahead
  // through a ring of four register slots (indices clamped, so every step
  // issues the same loads); hidden sizes that are not a multiple of 128 end
  // with groups of 8 (pairs (8j + i, 8j + 4 + i)).
  constexpr int kRing = 4, kAhead = 3;
  const int n_vis = a.H / 32;
  const int n_main = (n_vis / kRing) * kRing;
  const float* w0v = a.w + static_cast<int64_t>(r0) * a.H + 16 * half;
  f32x4 wq[kRing][4];
  typename XRaw<XF32>::T xaq[kRing][4], xbq[kRing][4];
  auto load = [&](int slot, int J) {
    const int h = 32 * J + 16 * half;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      wq[slot][c] = *reinterpret_cast<const f32x4*>(w0v + 32 * J + 4 * c);
      xaq[slot][c] = load_x4<XF32>(a, ta, h + 4 * c);
      xbq[slot][c] = load_x4<XF32>(a, tb, h + 4 * c);
    }
  };
  if (n_main > 0) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) load(u, min(u, n_main - 1));
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int J0 = 0; J0 < n_main; J0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      load((u + kAhead) % kRing, min(J0 + u + kAhead, n_main - 1));
      __builtin_amdgcn_sched_barrier(0);  // keep the loads here, ahead of their use
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[0][0] = mfma32(wq[u][c][i], x_val(xaq[u][c], i), acc[0][0]);
          acc[0][1] = mfma32(wq[u][c][i], x_val(xbq[u][c], i), acc[0][1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  for (int j = 4 * n_main; j < a.H / 8; ++j) {
    const int h = 8 * j + 4 * half;
    const f32x4 wv = *reinterpret_cast<const f32x4*>(w0 + 8 * j);
    const auto xa = load_x4<XF32>(a, ta, h);
    const auto xb = load_x4<XF32>(a, tb, h);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[0][0] = mfma32(wv[i], x_val(xa, i), acc[0][0]);
      acc[0][1] = mfma32(wv[i], x_val(xb, i), acc[0][1]);
    }
  }

  // acc[rt][tt] register v: vocabulary row v0 + 32rt + 8(v/4) + 4half + v%4,
  // token t0 + 32tt + col.
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = t0 + 32 * tt + col;
    float mx = kNegInf;
#pragma unroll
    for (int rt = 0; rt < kNRT; ++rt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = v0 + 32 * rt + 8 * (v >> 2) + 4 * half + (v & 3);
        if (row >= a.V) acc[rt][tt][v] = kNegInf;
        mx = fmaxf(mx, acc[rt][tt][v]);
      }
    }
    const float m = pair_max(mx);
    float sub[kNRT];
#pragma unroll
    for (int rt = 0; rt < kNRT; ++rt) {
      f32x16 e;
#pragma unroll
      for (int v = 0; v < 16; ++v) e[v] = hw_exp2((acc[rt][tt][v] - m) * kLog2e);
      sub[rt] = pair_sum(tree16(e));
    }
    float s = sub[0];
#pragma unroll
    for (int rt = 1; rt < kNRT; ++rt) s = s + sub[rt];
    if (t < a.T) {
      if (half == 0) {
        float* part = a.part + (static_cast<int64_t>(t) * a.n_vblocks + vblk) * 2;
        *reinterpret_cast<float2*>(part) = float2{m, s};
      }
      const int y = a.tokens[t];
      const int rr = y - v0;
      if (rr >= 0 && rr < kRowsPerWave) {
        const int rt = rr >> 5, rem = rr & 31;
        if (((rem >> 2) & 1) == half) {
          const int v = 4 * (rem >> 3) + (rem & 3);
          float zy = 0.0f;
#pragma unroll
          for (int q = 0; q < kNRT; ++q) {
#pragma unroll
            for (int u = 0; u < 16; ++u) zy = (q == rt && u == v) ? acc[q][tt][u] : zy;  // static register indices
          }
          a.zsel[t] = zy;
        }
      }
    }
  }
}

// Pass 2: one workgroup of 4 waves per token.  Wave w takes the blocks
// [w*n/4, (w+1)*n/4), lane l of it blocks l, l+64, ... of that range in
// ascending order; the lanes' sums meet in a fixed butterfly and the four
// wave sums as (s0 + s1) + (s2 + s3).
__global__ __launch_bounds__(256) void lmh_fold_kernel(const LmHeadArgs a) {
  __shared__ float red[8];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = static_cast<int>(blockIdx.x);
  const float* part = a.part + static_cast<int64_t>(t) * a.n_vblocks * 2;
  const int lo = static_cast<int>(static_cast<int64_t>(a.n_vblocks) * wave / 4);
  const int hi = static_cast<int>(static_cast<int64_t>(a.n_vblocks) * (wave + 1) / 4);
  float mx = kNegInf;
  for (int b = lo + lane; b < hi; b += 64) mx = fmaxf(mx, part[2 * b]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = 0.0f;
  for (int b = lo + lane; b < hi; b += 64) {
    const float2 p = *reinterpret_cast<const float2*>(part + 2 * b);
    const float w = hw_exp2((p.x - mx) * kLog2e);
    const float term = p.y * w;
    s = s + term;
  }
  // Butterfly: lanes i and i^m add the same two values, so all lanes agree.
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s = s + __shfl_xor(s, m, 64);
  if (lane == 0) red[4 + wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float tot = (red[4] + red[5]) + (red[6] + red[7]);
    const float lz = mx + hw_log2(tot) * kLn2;
    const int y = a.tokens[t];
    const float lp = (y >= 0 && y < a.V) ? a.zsel[t] - lz : __builtin_nanf("");
    a.logp[t] = lp;
    if (a.logz != nullptr) a.logz[t] = lz;
  }
}

}  // namespace

size_t lm_head_scratch_floats(int T, int V) {
  const size_t blocks = (static_cast<size_t>(V) + kRowsPerWave - 1) / kRowsPerWave;
  return blocks * static_cast<size_t>(T) * 2 + static_cast<size_t>(T);
}

hipError_t launch_lm_head(LmHeadArgs a, bool x_f32, hipStream_t s) {
  a.n_vblocks = (a.V + kRowsPerWave - 1) / kRowsPerWave;
  a.n_tgroups = (a.T + kTokPerWave - 1) / kTokPerWave;
  a.zsel = a.part + static_cast<size_t>(a.n_vblocks) * a.T * 2;
  const int64_t n_vgroups = (static_cast<int64_t>(a.n_vblocks) + kWaves - 1) / kWaves;
  const int64_t g1 = n_vgroups * a.n_tgroups;
  if (g1 <= 0 || g1 > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (x_f32) {
    hipLaunchKernelGGL(lmh_partial_kernel<true>, dim3(static_cast<unsigned>(g1)), dim3(kWaves * 64), 0, s, a);
  } else {
    hipLaunchKernelGGL(lmh_partial_kernel<false>, dim3(static_cast<unsigned>(g1)), dim3(kWaves * 64), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lmh_fold_kernel, dim3(static_cast<unsigned>(a.T)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace rla
