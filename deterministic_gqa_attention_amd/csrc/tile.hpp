// LDS layout of one staged KV block (Bk keys x 128 dims, bf16) and the
// fragment reads of it.
//
// Both K and V are kept key-major, one 256-byte row per key, filled straight
// from global memory by global_load_lds_dwordx4 (each wave instruction writes
// 1 KiB = 4 rows; the lane -> global address map applies the swizzle, so the
// LDS side is a plain contiguous write).  The 16-byte chunks of a row are
// XOR-swizzled:
//  * K rows by the low 4 bits of the key, so the 16 rows an MFMA A-fragment
//    read (ds_read_b128) touches per cycle land in 16 distinct bank groups;
//  * V rows by fV(r) = ((r & 3) << 2) ^ ((r >> 2) & 3), so the transposed
//    reads (ds_read_b64_tr_b16: four lanes read one 16-dim row segment of a
//    key, lane i of the 16-lane group receives dim i of four keys) of 4 keys
//    x 4 chunks hit 32 distinct bank pairs.
#pragma once

#include "core.hpp"

namespace rla {

template <int BK>
struct TileLayout {
  static constexpr int kKBytes = BK * kHeadDim * 2;
  static constexpr int kVBytes = BK * kHeadDim * 2;
  static constexpr int kBytes = kKBytes + kVBytes;
  static constexpr int kLoadsPerRegion = BK / 4;  // 1 KiB direct loads per region

  __device__ static __forceinline__ int k_swz(int r) { return r & 15; }
  __device__ static __forceinline__ int v_swz(int r) { return ((r & 3) << 2) ^ ((r >> 2) & 3); }
  // byte offset of logical 16-byte chunk c (dims 8c..8c+7) of key row r
  __device__ static __forceinline__ int k_off(int r, int c) { return r * 256 + ((c ^ k_swz(r)) << 4); }
  // the same within the V region alone, and from the start of the tile
  __device__ static __forceinline__ int v_rel(int r, int c) { return r * 256 + ((c ^ v_swz(r)) << 4); }
  __device__ static __forceinline__ int v_off(int r, int c) { return kKBytes + v_rel(r, c); }
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ u32x4 lds_load16(const char* lds, int off) {
  return *reinterpret_cast<const u32x4*>(lds + off);
}
__device__ __forceinline__ u32x4 gload16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// One 16-byte-per-lane direct load: lane i's 16 bytes at src land at
// lds_dst + 16*i (lds_dst must be the same for the whole wave).
__device__ __forceinline__ void direct_load16(const uint16_t* src, char* lds_dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (lds_void*)(lds_dst), 16, 0, 0);
#endif
}

// Direct global->LDS loads of KV blocks into a tile buffer: the calling wave
// issues loads wave, wave+NW, ... of each region (1 KiB = 4 key rows each).
// The lane's element offsets within a block are fixed, so they are computed
// once; a block that reaches past kv_len takes the clamped path, where rows
// past kv_len load the last valid key instead (always masked: score -inf,
// weight exactly 0).
template <int BK, int NW>
struct BlockLoader {
  using L = TileLayout<BK>;
  static constexpr int NI = L::kLoadsPerRegion / NW;
  static_assert(L::kLoadsPerRegion % NW == 0, "loads must divide over the waves");
  // Row of load i is r_i = 4*(wave + NW*i) + lane/16; both swizzles depend on
  // r_i only through bits that do not change with i (NW is a multiple of 4),
  // so offset i is offset 0 plus the uniform stride i * 4*NW rows.
  static_assert(NW % 4 == 0, "swizzle bits must not depend on the load index");
  int koff0;
  int voff0;
  int wave;

  __device__ __forceinline__ void init(int row_stride) {
    wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int p = lane & 15;
    const int r = 4 * wave + (lane >> 4);
    koff0 = r * row_stride + ((p ^ L::k_swz(r)) << 3);
    voff0 = r * row_stride + ((p ^ L::v_swz(r)) << 3);
  }

  __device__ __forceinline__ void issue(char* buf, const uint16_t* kb, const uint16_t* vb, int64_t row_stride,
                                        int64_t key0, int64_t kv_len) const {
    if (key0 + BK <= kv_len) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int n = wave + NW * i;
        const int64_t rows = key0 + 4 * NW * i;  // uniform
        direct_load16(kb + rows * row_stride + koff0, buf + n * 1024);
        direct_load16(vb + rows * row_stride + voff0, buf + L::kKBytes + n * 1024);
      }
    } else {
      const int lane = threadIdx.x & 63;
      const int p = lane & 15;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int n = wave + NW * i;
        const int r = 4 * n + (lane >> 4);
        int64_t key = key0 + r;
        key = key < kv_len ? key : kv_len - 1;
        direct_load16(kb + key * row_stride + ((p ^ L::k_swz(r)) << 3), buf + n * 1024);
        direct_load16(vb + key * row_stride + ((p ^ L::v_swz(r)) << 3), buf + L::kKBytes + n * 1024);
      }
    }
  }
};

// Wait until this wave's direct loads have landed in LDS (vmcnt(0)).
__device__ __forceinline__ void wait_direct_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A-fragment of K for sub-tile kt, head-dim step ds (lane: key row kt*32+col,
// dims 16ds + 8*half + 0..7).
template <int BK>
__device__ __forceinline__ bf16x8 k_frag(const char* lds, int kt, int ds, int col, int half) {
  return as_bf16x8(lds_load16(lds, TileLayout<BK>::k_off(kt * 32 + col, 2 * ds + half)));
}

// A-fragment of V^T for output dim tile dt and key step (kt, s): lane l holds
// dim dt*32 + l%32 at keys kb + {4h..4h+3} then kb + {8+4h..8+4h+3},
// kb = kt*32 + 16s, h = l/32 — the key order of the P^T B-fragment taken from
// accumulator registers 8s..8s+7 of score sub-tile kt.  Two transposed reads:
// in each 16-lane group, lane 4k+j reads dims d0+4j..d0+4j+3 of key row
// base+k and receives dim d0+i of the four rows.  vbase points at the V region.
template <int BK>
__device__ __forceinline__ bf16x8 v_frag(const char* vbase, int dt, int kt, int s) {
  using L = TileLayout<BK>;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15;
  const int g = lane >> 4;
  const int h = g >> 1;
  const int k = i >> 2;
  const int j = i & 3;
  const int c = dt * 4 + 2 * (g & 1) + (j >> 1);
  const int r1 = kt * 32 + 16 * s + 4 * h + k;
  const int r2 = r1 + 8;
  const char* p1 = vbase + L::v_rel(r1, c) + (j & 1) * 8;
  const char* p2 = vbase + L::v_rel(r2, c) + (j & 1) * 8;
  v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p1));
  v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p2));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  v8i16 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations
// (lgkmcnt) and meets the other waves, but leaves global loads in flight, so
// register prefetches of the next KV block keep streaming across it.  (A full
// __syncthreads() would also wait for every outstanding global load.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace rla
