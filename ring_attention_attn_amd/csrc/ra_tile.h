// Device helpers shared by the MFMA attention kernels (gfx950, wave64).
//
// MFMA v_mfma_f32_32x32x16_bf16 lane layouts (verified on gfx950):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. +8
//   B (16 x 32): lane l holds col l%32, k = 8*(l/32) .. +8
//   C (32 x 32): lane l holds col l%32, register r is row 8*(r/4) + 4*(l/32) + r%4
//
// Row permutation sigma (swap bits 2 and 3 of a 0..31 row index): if the A
// operand of a product C = A B is loaded with lane l32 holding logical row
// sigma(l32), then C register r of lane half hi is logical row
// 16*(r/8) + 8*hi + r%8. Registers 0..7 (and 8..15) of a lane then cover 8
// CONSECUTIVE logical rows, so C can be reused directly as the B operand of a
// product that contracts over those rows, with the other operand read from a
// transposed LDS tile by one 16-byte load.
#pragma once
#include <limits.h>
#include "ra_internal.h"

__device__ __forceinline__ int sigma32(int l32) {
  return (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Registers 8*half .. 8*half+7 of an accumulator, rounded to bf16.
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int half) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16_t)x[8 * half + e];
  return r;
}

// Eight floats rounded to bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack_bf16x8(const float (&x)[8]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16_t)x[e];
  return r;
}

// max of three floats in one instruction (v_max3_f32); inputs are never NaN
__device__ __forceinline__ float fmax3(float a, float b, float c) {
  return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}

// Reductions over the two halves of a wave (lanes l and l ^ 32) with
// v_permlane32_swap instead of an LDS permute: with both operands = x, the
// swap leaves x[l % 32] in the first result and x[l % 32 + 32] in the second,
// so every lane combines the same two values in the same order.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- global -> LDS staging by LDS-DMA buffer loads (no registers, no ds_write).
// A buffer descriptor spans the rows [row0, row0 + rows) of one head (row
// stride ss elements); reads past its end return zeros, so ragged tails need no
// selects. Instruction j of the workgroup fills LDS bytes [1024 j, 1024 j +
// 1024): lane i writes the 16 bytes at 1024 j + 16 i.
typedef __attribute__((address_space(3))) void lds_void;

// Descriptor of the T-row tile starting at row row0 of a tensor with nrows
// rows: only rows that exist are in range. row_bytes = row stride in bytes; the
// host keeps T * row_bytes and the row counts below 2^31, so the range and the
// clamp are 32-bit arithmetic and the tile offset one 32 x 32 -> 64-bit product.
template <int T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const bf16_t* base, uint32_t row_bytes,
                                                            int row0, int nrows) {
  // (all values are wave-uniform; readfirstlane keeps the descriptor in scalar
  // registers, where the compiler would otherwise build a per-lane loop)
  row0 = __builtin_amdgcn_readfirstlane(row0);
  row_bytes = __builtin_amdgcn_readfirstlane(row_bytes);
  const int left = __builtin_amdgcn_readfirstlane(nrows) - row0;
  const int rows = __builtin_amdgcn_readfirstlane(left <= 0 ? 0 : (left >= T ? T : left));
  const char* ptr = (const char*)base + (uint64_t)(uint32_t)row0 * row_bytes;
  return __builtin_amdgcn_make_buffer_rsrc((void*)ptr, (short)0, (int)(rows * row_bytes),
                                           0x00020000);
}

// ---- XOR-swizzled row-major tiles (no padding): rows of D bf16, 16-byte
// chunk c of row r stored at chunk c ^ swz(r). Reads of one chunk from 16
// consecutive rows (16-byte loads) and transposing reads of 4 rows x 64 bytes
// both hit distinct banks (64 banks of 4 bytes: 16 chunk slots per 256 bytes).
template <int D>
__host__ __device__ __forceinline__ int swz(int r) {
  if (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  const int j = r >> 1;  // D == 64: two rows per 256 bytes
  return 4 * (j & 1) + ((j >> 1) & 3);
}
// byte offset of chunk c of row r
template <int D>
__host__ __device__ __forceinline__ int swz_off(int r, int c) {
  return r * 2 * D + 16 * (c ^ swz<D>(r));
}

// LDS-DMA staging of a T x D bf16 tile into the swizzled layout: instruction j
// fills bytes [1024 j, 1024 j + 1024); lane i writes physical chunk slot
// (16 i % (2D)) / 16 of row (1024 j + 16 i) / (2D), loading the logical chunk
// that the swizzle maps there.
// TAG only makes each kernel's instantiation distinct: with one shared
// specialization, hipcc left a kernel's host launch stub undefined.
template <int T, int D, int NW, int TAG>
struct DmaSwz {
  static constexpr int NJ = T * 2 * D / 1024;
  static constexpr int PER = (NJ + NW - 1) / NW;
  static_assert(T * 2 * D % 1024 == 0, "whole 1 KiB blocks");
  uint32_t voff[PER];
  uint32_t row_bytes;
  int wave;
  __device__ __forceinline__ void init(int64_t ss, int wave_, int lane) {
    wave = wave_;
    row_bytes = (uint32_t)(ss * 2);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int pb = 1024 * (wave + k * NW) + 16 * lane;
      int row = pb / (2 * D);
      const int phys = (pb % (2 * D)) / 16;
      row = row < T ? row : 0;
      const int c = phys ^ swz<D>(row);
      voff[k] = (uint32_t)(((int64_t)row * ss + 8 * c) * 2);
    }
  }
  // tile rows [row0, row0 + T) of `base` (of nrows rows) into `lds`
  __device__ __forceinline__ void issue(const bf16_t* base, int row0, int nrows,
                                        bf16_t* lds) const {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc<T>(base, row_bytes, row0, nrows);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int j = wave + k * NW;
      if (NJ % NW == 0 || j < NJ)  // every wave issues PER loads when NW divides NJ
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)((char*)lds + 1024 * j), 16,
                                                 voff[k], 0, 0, 0);
    }
  }
};

// Workgroup barrier ordering LDS only: waits for this wave's LDS operations
// but, unlike __syncthreads(), not for its outstanding vector-memory loads
// (LDS-DMA included); the memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until this wave's outstanding vector-memory operations (LDS-DMA loads
// included) are complete.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x3f70); }
// ... until at most N (< 16) of them are outstanding
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x3f70 | N);
}

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i of
// the four 8-byte rows addressed by lanes 4e + (i/4) (e = 0..3), i.e. a 4x16
// block read transposed. With lane roles (tr_row, tr_col) below, the pair of
// reads at rows R and R+8 gives the 8-value MFMA operand of column C.
__device__ __forceinline__ bf16x4 ds_read_tr(const bf16_t* lds_ptr) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
  return __builtin_bit_cast(bf16x4, r);
}

// Branch-free key/query positions of one tile of rows [t0, t0 + n): when the
// tile lies inside one segment, row t0 + off is at base + off. Positions fit in
// int32 (checked on the host).
struct TilePos {
  int base, nvalid;
  bool one_seg;
  const SegMap* m;
  int64_t t0;
  __device__ __forceinline__ TilePos(const SegMap& map, int64_t start, int n) : m(&map), t0(start) {
    one_seg = (start + n <= map.seg_len) || (start >= map.seg_len);
    base = (int)seg_pos(map, start);
    const int64_t left = map.len - start;
    nvalid = left < n ? (int)left : n;
  }
  __device__ __forceinline__ int pos(int off) const {
    return one_seg ? base + off : (int)seg_pos(*m, t0 + off);
  }
};

// x ? a : b on values. (A conditional over two struct members is an lvalue
// select, which can leave the struct in scratch memory.)
__device__ __forceinline__ int sel_int(bool x, int a, int b) { return x ? a : b; }
// int64 -> int32, saturating
__device__ __forceinline__ int sat_int(int64_t x) {
  return x > INT_MAX ? INT_MAX : (x < INT_MIN ? INT_MIN : (int)x);
}

// int32 positions of the rows [t0, t0 + n) of a SegMap, for branch-free
// masking: row t0 + off is at pos(off) while off < split (first run), and
// rows at or past nvalid do not exist. All fields are wave-uniform.
struct TileRows {
  int base0, base1, split, nvalid;
  __device__ __forceinline__ TileRows(const SegMap& m, int64_t t0, int n) {
    base0 = (int)(m.pos0 + t0);
    base1 = (int)(m.pos1 + t0 - m.seg_len);
    const int64_t s = m.seg_len - t0;
    split = s < 0 ? 0 : (s > n ? n : (int)s);
    const int64_t v = m.len - t0;
    nvalid = v < 0 ? 0 : (v > n ? n : (int)v);
  }
  __device__ __forceinline__ int pos(int off) const { return sel_int(off < split, base0, base1) + off; }
};

// Rows of a SegMap whose position is <= x: [0, c0) of the first run and
// [seg_len, seg_len + c1) of the second (positions increase along each run).
// int32 results: lengths and positions fit in int32 (checked on the host).
__device__ __forceinline__ void rows_upto(const SegMap& m, int64_t x, int& c0, int& c1) {
  const int64_t a = x - m.pos0 + 1, b = x - m.pos1 + 1, n1 = m.len - m.seg_len;
  c0 = (int)(a < 0 ? 0 : (a > m.seg_len ? m.seg_len : a));
  c1 = (int)(b < 0 ? 0 : (b > n1 ? n1 : b));
}

// Key tiles of TK rows of a KV chunk as seen by a block of queries, in int32:
// tiles holding a key at or before the block's last query position
// (visible: [0, a1) and [b0, b1)), and whether a tile is free of keys after
// the block's first query position and of rows past the end (mask-free).
template <int TK>
struct KeyTiles {
  int n, len, seg, a1, b0, b1, e0, e1;
  __device__ __forceinline__ KeyTiles(const SegMap& km, int causal, int64_t q_first,
                                      int64_t q_last) {
    len = (int)km.len;
    seg = (int)km.seg_len;
    n = (len + TK - 1) / TK;
    if (causal) {
      int c0, c1;
      rows_upto(km, q_last, c0, c1);
      a1 = (c0 + TK - 1) / TK;
      b0 = seg / TK;
      b1 = c1 > 0 ? (seg + c1 + TK - 1) / TK : b0;
      rows_upto(km, q_first, e0, e1);
    } else {
      a1 = n;
      b0 = b1 = 0;
      e0 = seg;
      e1 = len - seg;
    }
  }
  // first visible tile at or after t (n if none)
  __device__ __forceinline__ int next(int t) const {
    if (t < a1) return t;
    const int u = t > b0 ? t : b0;
    return u < b1 ? u : n;
  }
  __device__ __forceinline__ bool mask_free(int t) const {
    const int r0 = t * TK, r1 = r0 + TK;
    if (r1 > len) return false;
    if (r1 <= e0) return true;
    const bool second_ok = r1 <= seg + e1;
    if (r0 >= seg) return second_ok;
    return e0 == seg && second_ok;  // straddles the runs: both parts unmasked
  }
};

// Visibility of the keys of a tile to one query of position qlim (the lane's
// query), for key offsets c + u where u is the lane's part of the offset and
// c a compile-time constant: c + u must exist (< nvalid) and, when causal, sit
// at a position <= qlim.
struct MaskBounds {
  int nv, sp, a0, a1;
  __device__ __forceinline__ MaskBounds(const TileRows& t, int qlim, int u, int causal) {
    nv = t.nvalid - u;
    sp = t.split - u;
    // qlim - base - u, saturated to the int32 range
    a0 = causal ? sat_int((int64_t)qlim - t.base0 - u) : INT_MAX;
    a1 = causal ? sat_int((int64_t)qlim - t.base1 - u) : INT_MAX;
  }
  __device__ __forceinline__ bool key_visible(int c) const {
    return (c < nv) & (c <= sel_int(c < sp, a0, a1));
  }
};

// Query tiles of TQ rows as seen by a block of keys (positions [k_first,
// k_last]), in int32: tiles holding a query at or after k_first (visible: the
// suffixes [a0, a1) of the first run and [b0, n) of the second), and whether a
// tile has only existing rows at positions >= k_last (mask-free).
template <int TQ>
struct QueryTiles {
  int n, len, seg, a0, a1, b0, f0, f1;
  __device__ __forceinline__ QueryTiles(const SegMap& qm, int causal, int64_t k_first,
                                        int64_t k_last) {
    len = (int)qm.len;
    seg = (int)qm.seg_len;
    n = (len + TQ - 1) / TQ;
    const int64_t n1 = qm.len - qm.seg_len;
    if (causal) {
      // first row of each run at a position >= x
      auto from = [&](int64_t x, int& r0, int& r1) {
        const int64_t a = x - qm.pos0, b = x - qm.pos1;
        r0 = (int)(a < 0 ? 0 : (a > qm.seg_len ? qm.seg_len : a));
        r1 = (int)(b < 0 ? 0 : (b > n1 ? n1 : b));
      };
      int r0, r1;
      from(k_first, r0, r1);
      a0 = r0 / TQ;
      a1 = r0 < seg ? (seg + TQ - 1) / TQ : a0;
      b0 = (seg + r1) / TQ;
      if (seg + r1 >= len) b0 = n;
      from(k_last, f0, f1);
    } else {
      a0 = 0;
      a1 = n;
      b0 = n;
      f0 = 0;
      f1 = 0;
    }
  }
  __device__ __forceinline__ int next(int t) const {
    if (t < a0) t = a0;
    if (t < a1) return t;
    return t > b0 ? (t < n ? t : n) : (b0 < n ? b0 : n);
  }
  // last visible tile at or before t (-1 if none)
  __host__ __device__ __forceinline__ int prev(int t) const {
    if (t >= n) t = n - 1;
    if (t >= b0) return t;  // in the second run's suffix [b0, n)
    if (t >= a1) t = a1 - 1;  // between the runs: the first run's last tile
    return t >= a0 ? t : -1;
  }
  __device__ __forceinline__ bool mask_free(int t) const {
    const int r0 = t * TQ, r1 = r0 + TQ;
    if (r1 > len) return false;
    if (r1 <= seg) return r0 >= f0;
    if (r0 >= seg) return r0 >= seg + f1;
    return r0 >= f0 && f1 == 0;  // straddles the runs
  }
};

// Visibility of a tile's query rows to the lane's key (position kpos), for
// query offsets c + u (u = the lane's part, c a compile-time constant): the row
// must exist (< nvalid) and, when causal, sit at a position >= kpos. A key
// that does not exist sees nothing.
struct QMaskBounds {
  int nv, sp, a0, a1;
  __device__ __forceinline__ QMaskBounds(const TileRows& t, int kpos, bool key_ok, int u,
                                         int causal) {
    nv = t.nvalid - u;
    sp = t.split - u;
    // kpos - base - u, saturated to the int32 range (selects, no branches:
    // key_ok differs between lanes)
    const int c0 = causal ? sat_int((int64_t)kpos - t.base0 - u) : INT_MIN;
    const int c1 = causal ? sat_int((int64_t)kpos - t.base1 - u) : INT_MIN;
    a0 = sel_int(key_ok, c0, INT_MAX);
    a1 = sel_int(key_ok, c1, INT_MAX);
  }
  __device__ __forceinline__ bool row_visible(int c) const {
    return (c < nv) & (c >= sel_int(c < sp, a0, a1));
  }
};

// Workgroup id -> logical id = group * (total / groups) + tile, where the
// dispatcher places workgroup w on XCD w % 8 and runs an XCD's workgroups in
// order of w / 8. With 8 or more groups each XCD gets consecutive logical ids
// (whole groups, sharing its L2). With fewer (8 % groups == 0), a group spans
// 8 / groups XCDs and its tiles are dealt to them in turn, so every XCD gets
// an even share of each tile range: with paired blocks one half of the rows
// (or keys) of a ring step often has no work, and contiguous ranges would
// leave whole XCDs idle. A bijection either way.
__device__ __forceinline__ int xcd_remap(int w, int total, int groups) {
  if (total % 8 != 0) return w;
  const int x = w % 8, i = w / 8;
  if (groups >= 8 || 8 % groups != 0) return x * (total / 8) + i;
  const int per_group = 8 / groups;  // XCDs per group
  return (x / per_group) * (total / groups) + i * per_group + x % per_group;
}
