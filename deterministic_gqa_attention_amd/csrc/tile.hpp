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

// Buffer resource over the keys [0, kv_len) of one kv head: key r at byte
// r * row_bytes.  Reads at or past num_records return zeros, which is how
// the rows of a block past kv_len are filled (they are always masked: score
// -inf, weight exactly 0, and 0 * 0 adds nothing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, int64_t kv_len, int row_bytes) {
  const int64_t bytes = kv_len > 0 ? (kv_len - 1) * row_bytes + kHeadDim * 2 : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// Direct buffer->LDS loads of one KV block into one region: the calling wave
// issues loads wave, wave+NW, ... (1 KiB = 4 key rows each).  The per-lane
// offset is fixed (one register); the block and load offsets are uniform
// (scalar soffset).  Offsets are 32-bit: callers keep kv_len * row_bytes
// below 2^31.
template <int BK, int NW>
struct BlockLoader {
  using L = TileLayout<BK>;
  static constexpr int NI = L::kLoadsPerRegion / NW;
  static_assert(L::kLoadsPerRegion % NW == 0, "loads must divide over the waves");
  // Row of load i is r_i = 4*(wave + NW*i) + lane/16; both swizzles depend on
  // r_i only through bits that do not change with i (NW is a multiple of 4),
  // so load i is load 0 moved by the uniform 4*NW*i rows.
  static_assert(NW % 4 == 0, "swizzle bits must not depend on the load index");
  int kbyte0;  // lane's byte offset of load 0 within the block (K swizzle)
  int vbyte0;  // the same with the V swizzle
  int wave;
  int row_bytes;

  __device__ __forceinline__ void init(int row_stride) {
    init(row_stride, __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6)));
  }
  // The same for a loading team of NW waves whose member index (0..NW-1) is
  // w, e.g. the upper half of a workgroup.
  __device__ __forceinline__ void init(int row_stride, int w) {
    wave = w;
    row_bytes = row_stride * 2;
    const int lane = threadIdx.x & 63;
    const int p = lane & 15;
    const int r = 4 * wave + (lane >> 4);
    kbyte0 = r * row_bytes + ((p ^ L::k_swz(r)) << 4);
    vbyte0 = r * row_bytes + ((p ^ L::v_swz(r)) << 4);
  }

  template <bool V>
  __device__ __forceinline__ void issue(char* dst, __amdgpu_buffer_rsrc_t rs, int64_t key0) const {
    const int off0 = V ? vbyte0 : kbyte0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = wave + NW * i;
      const int soff = static_cast<int>(key0 + 4 * NW * i) * row_bytes;  // uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + n * 1024), 16, off0, soff, 0, 0);
    }
  }
  __device__ __forceinline__ void issue_k(char* dst, __amdgpu_buffer_rsrc_t rs, int64_t key0) const {
    issue<false>(dst, rs, key0);
  }
  __device__ __forceinline__ void issue_v(char* dst, __amdgpu_buffer_rsrc_t rs, int64_t key0) const {
    issue<true>(dst, rs, key0);
  }
};

// Direct global->LDS loads of one KV block gathered through a page table:
// the pool is [page][kv head][slot][128] with page size P >= 4, so the 4
// consecutive keys of one load instruction lie in one page.  That page,
// read from the table by a scalar load, is uniform across the wave; the lanes
// only add their row within the group and their swizzled chunk, and the LDS
// side is the layout of BlockLoader.  Keys at or past kv_len read the
// sequence's last page (clear_tail then zeroes their V rows in LDS); page ids
// outside [0, num_pages) are clamped into the pool, so a bad table cannot
// fault (its result is unspecified).
template <int BK, int NW>
struct PagedLoader {
  using L = TileLayout<BK>;
  static constexpr int NI = L::kLoadsPerRegion / NW;
  static_assert(NW % 4 == 0, "swizzle bits must not depend on the load index");
  int wave;
  int kbyte0;               // lane's byte offset within its 4-row group (K swizzle)
  int vbyte0;               // the same with the V swizzle
  const int32_t* table;     // page ids of this sequence
  int log2_P;
  int last_idx;             // table index of the page that holds key kv_len-1
  int64_t num_pages;
  int64_t page_elems;       // Hkv * P * 128
  int64_t head_elems;       // hk * P * 128

  __device__ __forceinline__ void init(const int32_t* tab, int lp, int64_t kv_len, int64_t pages, int Hkv, int hk) {
    wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int p = lane & 15;
    const int r = 4 * wave + g;
    kbyte0 = g * 256 + ((p ^ L::k_swz(r)) << 4);
    vbyte0 = g * 256 + ((p ^ L::v_swz(r)) << 4);
    table = tab;
    log2_P = lp;
    last_idx = kv_len > 0 ? static_cast<int>((kv_len - 1) >> lp) : 0;
    num_pages = pages;
    page_elems = static_cast<int64_t>(Hkv) * (int64_t{1} << lp) * kHeadDim;
    head_elems = static_cast<int64_t>(hk) * (int64_t{1} << lp) * kHeadDim;
  }

  template <bool V>
  __device__ __forceinline__ void issue(char* dst, const uint16_t* pool, int64_t key0) const {
    typedef const __attribute__((address_space(4))) int32_t ctab;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int idx = min(static_cast<int>((key0 + 4 * (wave + NW * i)) >> log2_P), last_idx);
      load_one<V>(dst, pool, key0, i, ((ctab*)table)[idx]);
    }
  }

  template <bool V>
  __device__ __forceinline__ void load_one(char* dst, const uint16_t* pool, int64_t key0, int i, int64_t page) const {
    const int n = wave + NW * i;
    const int64_t key = key0 + 4 * n;
    page = page < 0 ? 0 : (page >= num_pages ? num_pages - 1 : page);
    const int64_t slot = key & ((int64_t{1} << log2_P) - 1);
    const char* base = reinterpret_cast<const char*>(pool + page * page_elems + head_elems + slot * kHeadDim);
    direct_load16(reinterpret_cast<const uint16_t*>(base + (V ? vbyte0 : kbyte0)), dst + n * 1024);
  }

  // Zero the rows at or past kv_len among those this wave loaded for the
  // block at key0 (call once the loads have landed).
  __device__ __forceinline__ void clear_tail(char* dst, int64_t key0, int64_t kv_len) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = wave + NW * i;
      if (key0 + 4 * n + (lane >> 4) >= kv_len) *reinterpret_cast<u32x4*>(dst + n * 1024 + lane * 16) = u32x4{0, 0, 0, 0};
    }
  }
};

// Direct buffer->LDS loads of one KV block gathered through a page table,
// into the layout of BlockLoader, for a loading team of NW waves: each load
// instruction moves 4 consecutive keys, which lie in one page (page size
// P >= 4), through a buffer resource over that page's rows below kv_len, so
// rows at or past kv_len read as zeros (as the contiguous path's do).  Page
// ids are scalar reads of the table; ids outside [0, num_pages) are clamped
// into the pool, so a bad table cannot fault (its result is unspecified).
// LOG2P > 0 fixes the page size at compile time (it must be at least 4*NW
// keys): then the table entry and the in-page row of every load of a block
// are constants plus the block's first entry and the wave's row, and a block
// that ends at or before kv_len takes a short path (whole pages, no clamp of
// the table index), a few scalar instructions per load.  LOG2P == 0 takes the
// page size at run time.
template <int BK, int NW, int LOG2P = 0>
struct PagedBufLoader {
  using L = TileLayout<BK>;
  static constexpr int NI = L::kLoadsPerRegion / NW;
  static_assert(NW % 4 == 0, "swizzle bits must not depend on the load index");
  static_assert(LOG2P == 0 || (1 << LOG2P) >= 4 * NW, "a fixed page holds a whole row of the team's loads");
  int wave;
  int koff, voff;          // lane's byte offset within its 4-row group (K / V swizzle)
  const int32_t* table;    // page ids of this sequence
  int log2_P;
  int last_idx;            // table index of the page that holds key kv_len-1
  int max_page;            // num_pages - 1
  uint32_t page_bytes;     // Hkv * P * 256
  uint32_t head_bytes;     // hk * P * 256
  int kv_len;

  __device__ __forceinline__ void init(const int32_t* tab, int lp, int64_t kvl, int64_t pages, int Hkv, int hk,
                                       int w) {
    wave = w;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int p = lane & 15;
    const int r = 4 * wave + g;
    koff = g * 256 + ((p ^ L::k_swz(r)) << 4);
    voff = g * 256 + ((p ^ L::v_swz(r)) << 4);
    table = tab;
    log2_P = LOG2P > 0 ? LOG2P : lp;
    last_idx = kvl > 0 ? static_cast<int>((kvl - 1) >> log2_P) : 0;
    max_page = static_cast<int>((pages < 0x7fffffff ? pages : 0x7fffffff) - 1);
    page_bytes = static_cast<uint32_t>(Hkv) << (log2_P + 8);
    head_bytes = static_cast<uint32_t>(hk) << (log2_P + 8);
    kv_len = static_cast<int>(kvl);
  }

  __device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const uint16_t* pool, int page, int rows) const {
    page = page < 0 ? 0 : (page > max_page ? max_page : page);
    const char* base = reinterpret_cast<const char*>(pool) + head_bytes +
                       static_cast<uint64_t>(static_cast<uint32_t>(page)) * page_bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, rows * 256, 0x00020000);
  }

  template <bool V>
  __device__ __forceinline__ void issue(char* dst, const uint16_t* pool, int key0) const {
    typedef const __attribute__((address_space(4))) int32_t ctab;
    if (LOG2P > 0 && key0 + BK <= kv_len) {
      // whole pages, entries [key0/P, (key0+BK)/P) of the table
      constexpr int P = 1 << (LOG2P > 0 ? LOG2P : 2);
      const ctab* t = (ctab*)table + (key0 >> LOG2P);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int n = wave + NW * i;
        constexpr int kTeamRows = 4 * NW;  // rows one load index covers across the team
        const int entry = (kTeamRows * i) >> LOG2P;
        const int row = ((kTeamRows * i) & (P - 1)) + 4 * wave;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(page_rsrc(pool, t[entry], P), (lds_void*)(dst + n * 1024), 16,
                                                 V ? voff : koff, row * 256, 0, 0);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = wave + NW * i;
      const int key = key0 + 4 * n;
      const int idx = min(key >> log2_P, last_idx);
      const int pkey0 = (key >> log2_P) << log2_P;
      const int left = kv_len - pkey0;
      const int rows = left <= 0 ? 0 : (left >= (1 << log2_P) ? (1 << log2_P) : left);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(page_rsrc(pool, ((ctab*)table)[idx], rows),
                                               (lds_void*)(dst + n * 1024), 16, V ? voff : koff,
                                               (key - pkey0) * 256, 0, 0);
    }
  }
};

// Tile order of a grid of n_tiles query tiles x n_bh (b, kv head[, head
// subgroup]) pairs, heaviest tile (the last) first.  Workgroup wg runs on XCD
// wg % 8.  When n_bh is a multiple of 16, the XCD owns the pairs bh = XCD + 8i
// and takes them two at a time, heaviest tiles first within the pair group,
// so the tiles in flight on one XCD read the K/V of two pairs instead of all
// of its pairs and a block's re-reads by later tiles mostly hit that XCD's
// L2; otherwise the grid is tile-major over all pairs.  Either way the map is
// a bijection of the grid and changes nothing a row computes.
constexpr int kXcdPairs = 2;

__device__ __forceinline__ void heavy_first_tile(int64_t wg, int n_bh, int n_tiles, int& bh, int& tile) {
  if (n_bh % (8 * kXcdPairs) == 0) {
    const int64_t k = wg >> 3;
    const int64_t per_group = static_cast<int64_t>(kXcdPairs) * n_tiles;
    const int r = static_cast<int>(k % per_group);
    bh = static_cast<int>(wg & 7) + 8 * (static_cast<int>(k / per_group) * kXcdPairs + r % kXcdPairs);
    tile = n_tiles - 1 - r / kXcdPairs;
  } else {
    bh = static_cast<int>(wg % n_bh);
    tile = n_tiles - 1 - static_cast<int>(wg / n_bh);
  }
}

// Wait until at most n of this wave's vector-memory loads are outstanding
// (they retire in issue order); n is one of 0, NI, 2*NI of a loader, chosen
// by a wave-uniform branch so the count stays an immediate.
template <int NI>
__device__ __forceinline__ void wait_loads_leq(int n) {
  static_assert(2 * NI < 64, "vmcnt field");
  if (n <= 0) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), lgkm/exp untouched
  } else if (n <= NI) {
    __builtin_amdgcn_s_waitcnt(0x0F70 | (NI & 15) | ((NI >> 4) << 14));
  } else {
    __builtin_amdgcn_s_waitcnt(0x0F70 | ((2 * NI) & 15) | (((2 * NI) >> 4) << 14));
  }
}

// Wait until this wave's direct loads have landed in LDS (vmcnt(0)).
__device__ __forceinline__ void wait_direct_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A-fragment of K for sub-tile kt, head-dim step ds (lane: key row kt*32+col,
// dims 16ds + 8*half + 0..7).  kreg points at the K region.
template <int BK>
__device__ __forceinline__ bf16x8 k_frag(const char* kreg, int kt, int ds, int col, int half) {
  return as_bf16x8(lds_load16(kreg, TileLayout<BK>::k_off(kt * 32 + col, 2 * ds + half)));
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

// 32-bit LDS address of a __shared__ object.
__device__ __forceinline__ int lds_address(const void* p) {
  return static_cast<int>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)p));
}

// x + c computed into a register whose value the compiler does not track,
// at this point of the program (volatile: never hoisted out of a loop).
__device__ __forceinline__ int opaque_add(int x, int c) {
  int r;
  asm volatile("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(c), "v"(x));
  return r;
}

// Fragment reads of one K or V region (the layouts above).  The swizzles
// depend only on lane bits, so
//  * the K A-fragment of sub-tile kt, head-dim step ds sits at
//    k_off(col, 2ds + half) + kt*32*256;
//  * the two transposed V reads of dim tile dt at key step (kt, s) sit at
//    v_rel(4h + k, c) + (j&1)*8 + (32kt + 16s)*256 and the same at row
//    4h + k + 8 (rows of the step; c = 4dt + 2(g&1) + j/2).
// The constructor turns the per-lane parts into absolute LDS addresses held
// in registers the compiler treats as opaque (computed where the object is
// built, never hoisted); each read is then written as
// region + (addr - region_address + imm), which the compiler reduces to
// addr + imm: one register per offset and the immediate offset field,
// whatever the region's place in LDS (LDS immediates are 16-bit, so a region
// above 64 KiB would otherwise cost one address add per read).
// The lane index as a value computed at this point of the program: address
// arithmetic derived from it is redone where it is used instead of being
// hoisted out of a loop (where it would hold registers for the whole loop).
__device__ __forceinline__ int opaque_lane() {
  int l;
  asm volatile("v_and_b32 %0, 63, %1" : "=v"(l) : "v"(static_cast<int>(threadIdx.x)));
  return l;
}

template <int BK>
struct KReads {
  const char* reg;
  int ref;
  int a[kDSteps];
  __device__ __forceinline__ explicit KReads(const char* kreg) : KReads(kreg, static_cast<int>(threadIdx.x & 63)) {}
  __device__ __forceinline__ KReads(const char* kreg, int lane) : reg(kreg), ref(lds_address(kreg)) {
    const int col = lane & 31;
    const int half = lane >> 5;
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) a[ds] = opaque_add(TileLayout<BK>::k_off(col, 2 * ds + half), ref);
  }
  // K A-fragment of sub-tile kt, step ds
  __device__ __forceinline__ bf16x8 frag(int kt, int ds) const {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(reg + (a[ds] - ref + kt * 32 * 256)));
  }
};

template <int BK>
struct VReads {
  const char* reg;
  int ref;
  int a[kDTiles][2];
  __device__ __forceinline__ explicit VReads(const char* vreg) { init(vreg, static_cast<int>(threadIdx.x & 63)); }
  __device__ __forceinline__ VReads(const char* vreg, int lane) { init(vreg, lane); }
  __device__ __forceinline__ VReads() {}
  // Bind to a region (at this point of the program, so the address registers
  // live from here on).
  __device__ __forceinline__ void init(const char* vreg) { init(vreg, static_cast<int>(threadIdx.x & 63)); }
  __device__ __forceinline__ void init(const char* vreg, int lane) {
    reg = vreg;
    ref = lds_address(vreg);
    using L = TileLayout<BK>;
    const int i = lane & 15;
    const int g = lane >> 4;
    const int h = g >> 1;
    const int kk = i >> 2;
    const int j = i & 3;
#pragma unroll
    for (int dt = 0; dt < kDTiles; ++dt) {
      const int c = dt * 4 + 2 * (g & 1) + (j >> 1);
      a[dt][0] = opaque_add(L::v_rel(4 * h + kk, c) + (j & 1) * 8, ref);
      a[dt][1] = opaque_add(L::v_rel(4 * h + kk + 8, c) + (j & 1) * 8, ref);
    }
  }
  __device__ __forceinline__ bf16x8 frag(int dt, int kt, int s) const {
    const int step = (32 * kt + 16 * s) * 256;
    const char* p1 = reg + (a[dt][0] - ref + step);
    const char* p2 = reg + (a[dt][1] - ref + step);
    v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p1));
    v4i16 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p2));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    v8i16 xy = __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, xy);
  }
};

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Workgroup barrier that orders LDS only: waits for this wave's LDS operations
// (lgkmcnt) and meets the other waves, but leaves global loads in flight, so
// register prefetches of the next KV block keep streaming across it.  (A full
// __syncthreads() would also wait for every outstanding global load.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

}  // namespace rla
