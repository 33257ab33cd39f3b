// Tiles of latent (MLA-shaped) attention shared by its kernels: one cached
// row of d_qk = 576 bf16 per position (a 512-wide latent that is also the
// value, and a 64-wide positional part), staged through LDS in 64-row tiles.
#pragma once

#include "mala_common.hpp"

namespace mala {
namespace latent {

constexpr int LQK = 576;  // d_qk
constexpr int LV = 512;   // d_v
constexpr int LBQ = 64;
constexpr int LBK = 64;
constexpr int LKC = LQK / 32;            // 16x16x32 contraction chunks of S
constexpr int LVC = LV / 32;             // 16x16x32 contraction chunks of dP
constexpr int LUNITS = LQK / 8;          // 16-byte units per K row (72)
constexpr int LTILE = LBK * LQK;         // bf16 elements per K tile
constexpr int LCOPY = LBK * LUNITS / 64; // 1 KB copy instructions per K tile (72)

// K tile layout: row-major 1152-byte rows; within each aligned group of
// eight 16-byte units the unit index is XORed with a 3-bit function of
// m = (row / 2) % 8. Rows alternate between the two halves of the LDS banks
// (1152 = 4.5 x 256). Two variants, chosen per kernel with an LDS probe on
// gfx950 (bank-conflict counters per access pattern) and kernel timings:
//  - REV = true (the forward and decode kernels): f(m) = (m0, m1 ^ m2, m2)
//    as bits (2, 1, 0). Sixteen consecutive rows read at one column (score
//    operands, 16-byte reads), four rows x 32 columns (the forward's value
//    operands) and rows r .. r + 3 with r + 8 .. r + 11 (the 16x16x32
//    transposing reads) are all free of bank conflicts.
//  - REV = false (the backward kernels): f(m) = m, which also keeps the
//    sixteen-row score-operand reads free of conflicts; it measured faster
//    there than the variant above.
template <bool REV = true>
__device__ __forceinline__ int lk_swz(int row) {
  const int m = (row >> 1) & 7;
  return REV ? (((m & 1) << 2) | ((((m >> 1) ^ (m >> 2)) & 1) << 1) | ((m >> 2) & 1)) : m;
}
template <bool REV = true>
__device__ __forceinline__ int lk_idx(int row, int col) {
  const int u = col >> 3;
  return row * LQK + ((((u & ~7) | ((u & 7) ^ lk_swz<REV>(row)))) << 3) + (col & 7);
}
// P tile: 64 rows x 64 keys bf16, 16-byte units XORed with (row / 2) % 8.
__device__ __forceinline__ int lp_idx(int row, int col) {
  return row * LBK + ((((col >> 3) ^ ((row >> 1) & 7))) << 3) + (col & 7);
}

typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ u32x4_t lds_ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// Copy K rows k0 .. k0 + 63 (clamped to n - 1) into a K tile with NW waves:
// instruction n moves physical units 64 n .. 64 n + 63 of the tile; lane i
// fetches the logical unit that the swizzle places at physical unit 64 n + i.
// ORDERED selects the builtin form of the copy (see lds_dma16_ordered).
template <int NW, bool REV = true, bool ORDERED = false>
__device__ __forceinline__ void lk_copy_w(uint16_t* tile, const uint16_t* base, size_t rs, int k0, int n,
                                          int wave, int lane) {
  static_assert(LCOPY % NW == 0, "copy instructions split evenly over the waves");
#pragma unroll
  for (int c = 0; c < LCOPY / NW; ++c) {
    const int ins = wave + c * NW;
    const int p = ins * 64 + lane;
    const int row = p / LUNITS, pu = p % LUNITS;
    const int lu = (pu & ~7) | ((pu & 7) ^ lk_swz<REV>(row));
    const int grow = min(k0 + row, n - 1);
    if (ORDERED)
      lds_dma16_ordered(base + (size_t)grow * rs + lu * 8, tile + ins * 512);
    else
      lds_dma16(base + (size_t)grow * rs + lu * 8, lds_address(tile + ins * 512));
  }
}

// Transposing read of a row-major bf16 tile: lane l of 16-lane group g
// receives column c0 + l % 16 of rows r0 + 8 g .. + 7 (the k-major operand
// layout of the 16x16x32 MFMA), idx(row, col) being the tile's layout.
template <typename Idx>
__device__ __forceinline__ u32x4_t lds_tr8(const uint16_t* tile, int r0, int c0, int lane, Idx idx) {
  const int g = lane >> 4, y = lane & 15;
  const int row = r0 + 8 * g + (y >> 2), col = c0 + 4 * (y & 3);
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)&tile[idx(row, col)]);
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)&tile[idx(row + 4, col)]);
  const u32x2_t lw = __builtin_bit_cast(u32x2_t, lo), hw = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{lw[0], lw[1], hw[0], hw[1]};
}

template <bool REV = true>
struct LkIdxT {
  __device__ int operator()(int r, int c) const { return lk_idx<REV>(r, c); }
};
using LkIdx = LkIdxT<true>;
struct LpIdx {
  __device__ int operator()(int r, int c) const { return lp_idx(r, c); }
};

}  // namespace latent
}  // namespace mala
