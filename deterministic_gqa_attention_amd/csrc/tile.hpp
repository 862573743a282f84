// LDS layouts of one staged KV block (Bk keys x 128 dims, bf16) and the
// register transposition used to build the V^T layout.
//
// K is kept key-major, one 256-byte row per key, with its 16-byte chunks
// XOR-swizzled by the low 3 bits of the key so that the 32 rows an MFMA
// A-fragment read touches fall in distinct bank groups.
//
// V is kept transposed (dimension-major, keys contiguous) because the PV
// product contracts over keys: an A-fragment lane needs 8 keys of one
// dimension.  8-byte units (4 keys) are XOR-swizzled by f(d) below, which
// keeps both the transposing writes and the fragment reads free of bank
// conflicts.
#pragma once

#include "core.hpp"

namespace rla {

template <int BK>
struct TileLayout {
  static constexpr int kKBytes = BK * kHeadDim * 2;
  static constexpr int kVBytes = BK * kHeadDim * 2;
  static constexpr int kBytes = kKBytes + kVBytes;
  static constexpr int kVRowBytes = BK * 2;

  // byte offset of 16-byte chunk c (dims 8c..8c+7) of key row r
  __device__ static __forceinline__ int k_off(int r, int c) { return r * 256 + ((c ^ (r & 7)) << 4); }

  __device__ static __forceinline__ int v_swz(int d) { return (d & 15) ^ ((d >> 4) & 7); }
  // byte offset, within the V^T region, of 8-byte unit u (keys 4u..4u+3) of
  // dimension row d
  __device__ static __forceinline__ int v_off(int d, int u) {
    return d * kVRowBytes + ((u ^ v_swz(d)) << 3);
  }
};

// Transpose a 4-key x 8-dim bf16 sub-block: r[j] holds dims 8dc..8dc+7 of key
// 4kg+j.  Output o[i] holds keys 4kg..4kg+3 of dim 8dc+i.
__device__ __forceinline__ void transpose4x8(const u32x4 r[4], u32x2 o[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int w = i >> 1;
    uint32_t x01, x23;
    if ((i & 1) == 0) {
      x01 = (r[0][w] & 0xffffu) | (r[1][w] << 16);
      x23 = (r[2][w] & 0xffffu) | (r[3][w] << 16);
    } else {
      x01 = (r[0][w] >> 16) | (r[1][w] & 0xffff0000u);
      x23 = (r[2][w] >> 16) | (r[3][w] & 0xffff0000u);
    }
    o[i] = u32x2{x01, x23};
  }
}

__device__ __forceinline__ void lds_store16(char* lds, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(lds + off) = v;
}
__device__ __forceinline__ void lds_store8(char* lds, int off, u32x2 v) {
  *reinterpret_cast<u32x2*>(lds + off) = v;
}
__device__ __forceinline__ u32x4 lds_load16(const char* lds, int off) {
  return *reinterpret_cast<const u32x4*>(lds + off);
}
__device__ __forceinline__ u32x2 lds_load8(const char* lds, int off) {
  return *reinterpret_cast<const u32x2*>(lds + off);
}
__device__ __forceinline__ u32x4 gload16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// A-fragment of K for sub-tile kt, head-dim step ds (lane: key row kt*32+col,
// dims 16ds + 8*half + 0..7).  lds_k points at the K region.
template <int BK>
__device__ __forceinline__ bf16x8 k_frag(const char* lds_k, int kt, int ds, int col, int half) {
  return as_bf16x8(lds_load16(lds_k, TileLayout<BK>::k_off(kt * 32 + col, 2 * ds + half)));
}

// A-fragment of V^T for output dim tile dt and key step (kt, s): lane holds
// dim dt*32+col at keys kt*32+16s + {4h..4h+3} then {8+4h..8+4h+3}, h = half;
// this is the key order of the P^T B-fragment taken from accumulator
// registers 8s..8s+7 of the score sub-tile kt.  lds_v points at the V^T region.
template <int BK>
__device__ __forceinline__ bf16x8 v_frag(const char* lds_v, int dt, int kt, int s, int col, int half) {
  const int d = dt * 32 + col;
  const int u = 8 * kt + 4 * s + half;
  u32x2 a = lds_load8(lds_v, TileLayout<BK>::v_off(d, u));
  u32x2 b = lds_load8(lds_v, TileLayout<BK>::v_off(d, u + 2));
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

}  // namespace rla
