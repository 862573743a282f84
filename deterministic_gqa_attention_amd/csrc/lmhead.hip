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
// dimension in a fixed order (groups of 8 in ascending order; inside a group
// the pairs (8j+i, 8j+4+i) for i = 0..3), and a token's logit depends only on
// its own MFMA column, so batch makeup changes nothing.  Pass 1 writes, per
// (64-row vocabulary block, token), the block max and the fixed-tree sum of
// exp(z - max) (and the selected logit from the block that holds y_t); pass 2
// folds the blocks in ascending order: M = max of the block maxima,
// S = sum_b s_b exp(m_b - M) with lane l taking blocks l, l+64, ... in order
// and a fixed butterfly across lanes, logZ = M + ln S.
#include "kernels.hpp"
#include "core.hpp"

namespace rla {

namespace {

constexpr int kRowsPerWave = 64;  // vocabulary rows per wave (two 32-row MFMA tiles)
constexpr int kTokPerWave = 64;   // tokens per wave (two 32-column MFMA tiles)
constexpr int kWaves = 4;

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Four consecutive x values of token row t from h, widened to fp32 (zeros
// when the token is past T).
template <bool XF32>
__device__ __forceinline__ f32x4 load_x4(const LmHeadArgs& a, int t, int h) {
  if (t >= a.T) return f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t e = static_cast<int64_t>(t) * a.H + h;
  if constexpr (XF32) {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.x) + e);
  } else {
    const u32x2 w = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.x) + e);
    return f32x4{bf16_lo_to_f32(w[0]), bf16_hi_to_f32(w[0]), bf16_lo_to_f32(w[1]), bf16_hi_to_f32(w[1])};
  }
}

// Pass 1.  Grid: (vocabulary group of 4 x 64 rows) x (token group of 64),
// token groups fastest so neighbouring workgroups read the same W rows.
template <bool XF32>
__global__ __launch_bounds__(kWaves * 64) void lmh_partial_kernel(const LmHeadArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int tg = static_cast<int>(blockIdx.x % a.n_tgroups);
  const int vg = static_cast<int>(blockIdx.x / a.n_tgroups);
  const int vblk = vg * kWaves + wave;  // 64-row vocabulary block of this wave
  if (vblk >= a.n_vblocks) return;
  const int v0 = vblk * kRowsPerWave;
  const int t0 = tg * kTokPerWave;

  // Lane l reads W rows v0 + l%32 and v0 + 32 + l%32, and x rows t0 + l%32
  // and t0 + 32 + l%32, four values from 8j + 4half each.
  const int r0 = min(v0 + col, a.V - 1);  // rows past V read row V-1 (masked below)
  const int r1 = min(v0 + 32 + col, a.V - 1);
  const float* w0 = a.w + static_cast<int64_t>(r0) * a.H + 4 * half;
  const float* w1 = a.w + static_cast<int64_t>(r1) * a.H + 4 * half;
  const int ta = t0 + col, tb = t0 + 32 + col;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    acc[i][0] = f32x16{};
    acc[i][1] = f32x16{};
  }
  const int n_groups = a.H / 8;
  f32x4 wa = *reinterpret_cast<const f32x4*>(w0);
  f32x4 wb = *reinterpret_cast<const f32x4*>(w1);
  f32x4 xa = load_x4<XF32>(a, ta, 4 * half);
  f32x4 xb = load_x4<XF32>(a, tb, 4 * half);
  for (int j = 0; j < n_groups; ++j) {
    f32x4 nwa = wa, nwb = wb, nxa = xa, nxb = xb;
    if (j + 1 < n_groups) {  // next group's values, in flight during this group's MFMAs
      const int h = 8 * (j + 1);
      nwa = *reinterpret_cast<const f32x4*>(w0 + h);
      nwb = *reinterpret_cast<const f32x4*>(w1 + h);
      nxa = load_x4<XF32>(a, ta, h + 4 * half);
      nxb = load_x4<XF32>(a, tb, h + 4 * half);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[0][0] = mfma32(wa[i], xa[i], acc[0][0]);
      acc[0][1] = mfma32(wa[i], xb[i], acc[0][1]);
      acc[1][0] = mfma32(wb[i], xa[i], acc[1][0]);
      acc[1][1] = mfma32(wb[i], xb[i], acc[1][1]);
    }
    wa = nwa;
    wb = nwb;
    xa = nxa;
    xb = nxb;
  }

  // acc[rt][tt] register v: vocabulary row v0 + 32rt + 8(v/4) + 4half + v%4,
  // token t0 + 32tt + col.
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = t0 + 32 * tt + col;
    float mx = kNegInf;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = v0 + 32 * rt + 8 * (v >> 2) + 4 * half + (v & 3);
        if (row >= a.V) acc[rt][tt][v] = kNegInf;
        mx = fmaxf(mx, acc[rt][tt][v]);
      }
    }
    const float m = pair_max(mx);
    float sub[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      f32x16 e;
#pragma unroll
      for (int v = 0; v < 16; ++v) e[v] = hw_exp2((acc[rt][tt][v] - m) * kLog2e);
      sub[rt] = pair_sum(tree16(e));
    }
    const float s = sub[0] + sub[1];
    if (t < a.T) {
      if (half == 0) {
        float* part = a.part + (static_cast<int64_t>(vblk) * a.T + t) * 2;
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
          for (int q = 0; q < 2; ++q) {
#pragma unroll
            for (int u = 0; u < 16; ++u) zy = (q == rt && u == v) ? acc[q][tt][u] : zy;  // static register indices
          }
          a.zsel[t] = zy;
        }
      }
    }
  }
}

// Pass 2: one wave per token.
__global__ __launch_bounds__(256) void lmh_fold_kernel(const LmHeadArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = static_cast<int>(blockIdx.x) * 4 + static_cast<int>(threadIdx.x >> 6);
  if (t >= a.T) return;
  float mx = kNegInf;
  for (int b = lane; b < a.n_vblocks; b += 64) mx = fmaxf(mx, a.part[(static_cast<int64_t>(b) * a.T + t) * 2]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  float s = 0.0f;
  for (int b = lane; b < a.n_vblocks; b += 64) {
    const float2 p = *reinterpret_cast<const float2*>(a.part + (static_cast<int64_t>(b) * a.T + t) * 2);
    const float w = hw_exp2((p.x - mx) * kLog2e);
    const float term = p.y * w;
    s = s + term;
  }
  // Butterfly: lanes i and i^m add the same two values, so all lanes agree.
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s = s + __shfl_xor(s, m, 64);
  if (lane == 0) {
    const float lz = mx + hw_log2(s) * kLn2;
    const int y = a.tokens[t];
    const float lp = (y >= 0 && y < a.V) ? a.zsel[t] - lz : __builtin_nanf("");
    a.logp[t] = lp;
    if (a.logz != nullptr) a.logz[t] = lz;
  }
}

}  // namespace

hipError_t launch_lm_head(const LmHeadArgs& a, bool x_f32, hipStream_t s) {
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
  const int64_t g2 = (static_cast<int64_t>(a.T) + 3) / 4;
  hipLaunchKernelGGL(lmh_fold_kernel, dim3(static_cast<unsigned>(g2)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace rla
