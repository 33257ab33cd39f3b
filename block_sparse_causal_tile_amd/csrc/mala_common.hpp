// Shared device helpers for the MALA HIP kernels (gfx950 / CDNA4).
//
// Everything here is plumbing: vector types, 16-byte loads and stores, bf16
// packing, and the lane layout of the 32x32x16 bf16 MFMA. The attention
// arithmetic lives in the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mala_internal.hpp"

namespace mala {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Natural log through the hardware log2 (v_log_f32, about one ulp for a
// normal argument) for the per-tile tests: their argument is a running
// softmax sum, a normal float of at least 1 once any key is retained, and a
// decision that depends on the last ulp of the log lies inside the rounding
// of the scores anyway. The stored normalizers keep the full-precision log.
__device__ __forceinline__ float test_log(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}
__device__ __forceinline__ u32x4_t zero16() { return u32x4_t{0u, 0u, 0u, 0u}; }

// Two floats -> two bf16 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// What rounding (a, b) to the bf16 pair `hi` (= pack_bf16x2(a, b)) left
// over, itself rounded to bf16. hi + residual carries a and b to about 16
// significant bits, so a contraction that runs the matrix core on both
// pairs and sums the results sees its operand to within 2^-16 relative
// instead of bf16's 2^-9. The residual keeps fp32's exponent range (no
// overflow or extra underflow, unlike a narrower-range 16-bit format).
__device__ __forceinline__ uint32_t pack_bf16x2_residual(float a, float b, uint32_t hi) {
  return pack_bf16x2(a - bf16_lo(hi), b - bf16_hi(hi));
}

// D = A * B + C on a 32x32x16 bf16 matrix core op. Lane l supplies
//   A[l % 32][8 * (l / 32) + 0..7]  and  B[8 * (l / 32) + 0..7][l % 32],
// and holds C/D[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32] in register r.
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D = A * B + C on a 16x16x32 bf16 matrix core op. Lane l supplies
//   A[l % 16][8 * (l / 16) + 0..7]  and  B[8 * (l / 16) + 0..7][l % 16],
// and holds C/D[4 * (l / 16) + r][l % 16] in register r.
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Row (within a 32-row MFMA block) of accumulator register r in lane half hh.
__device__ __forceinline__ constexpr int acc_row(int r, int hh) {
  return 8 * (r >> 2) + 4 * hh + (r & 3);
}

// Reductions over the partner lanes l and l ^ 32 (l ^ 16) of a wave. The
// gfx950 lane swaps exchange the upper half (the odd 16-lane rows) of their
// first operand with the lower half (the even rows) of their second; given x
// twice, every lane then holds x of both partners, so the reduction needs no
// LDS round trip and, the ops being commutative, gives the same bits as
// x op (x of the partner lane).
__device__ __forceinline__ float wave_max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float row_pair_max(float x) {  // lanes l, l ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row_pair_sum(float x) {  // lanes l, l ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mala

namespace mala {

// ---------------------------------------------------------------------------
// ROWS x D bf16 tiles in LDS (64 or 128 rows), row-major, 16-byte units XOR-swizzled
// per row. The swizzle keeps three access patterns free of bank conflicts:
// 16-byte row reads by 32 lanes on 32 different rows (MFMA operands along a
// row), 16-byte stores of whole rows, and the transposing 8-byte reads below
// (four consecutive rows x 64 bytes per half-wavefront).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int tile_swz(int row) {
  return (((row & 3) << 2) | ((row >> 2) & 3)) & (D / 8 - 1);
}
template <int D>
__device__ __forceinline__ int tile_idx(int row, int col) {
  return row * D + ((((col >> 3) ^ tile_swz<D>(row)) << 3) | (col & 7));
}

// Eight consecutive columns col0..col0+7 (col0 % 8 == 0) of one row.
template <int D>
__device__ __forceinline__ u32x4_t tile_row8(const uint16_t* s, int row, int col0) {
  return *reinterpret_cast<const u32x4_t*>(&s[tile_idx<D>(row, col0)]);
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// MFMA operand that runs down a column: lane l receives
// T[rowbase + 8 (l / 32) + t][colbase + l % 32] for t = 0..7, read with two
// LDS transpose loads. Within each 16-lane group the transpose load hands
// lane x element x % 4 of the 8-byte chunks addressed by lanes x / 4 + 4 t,
// so lane y of the group addresses row rowbase + 8 (l / 32) + y / 4 at
// column colbase + 16 ((l / 16) % 2) + 4 (y % 4).
template <int D>
__device__ __forceinline__ u32x4_t tile_col8(const uint16_t* s, int rowbase, int colbase, int lane) {
  const int grp = lane >> 4, y = lane & 15;
  const int row = rowbase + 8 * (grp >> 1) + (y >> 2);
  const int col = colbase + 16 * (grp & 1) + 4 * (y & 3);
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&s[tile_idx<D>(row, col)]));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(&s[tile_idx<D>(row + 4, col)]));
  const u32x2_t a = __builtin_bit_cast(u32x2_t, lo), b = __builtin_bit_cast(u32x2_t, hi);
  return u32x4_t{a[0], a[1], b[0], b[1]};
}

// Buffer resource over `bytes` bytes from `base` (raw addressing, the gfx9
// descriptor word). A load whose byte offset lies at or past `bytes` returns
// zero: the hardware range check zero-fills tile rows past the end of a
// sequence with no per-lane compare or address clamp.
// `base` and `bytes` must be wave-uniform; they are read from the first
// lane so the descriptor lives in scalar registers (a descriptor the compiler
// cannot prove uniform costs a per-load loop over the distinct values).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_ld16(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0));
}

// A ROWS x D bf16 tile staged through registers: thread t holds the 16-byte
// chunks c = t + NT * k (row c / (D / 8), column 8 (c % (D / 8))). load()
// reads rows r0..r0+ROWS-1 of a BSHD tensor (row stride rs elements; rows at
// or past n read as zero) with buffer loads whose base and size are
// wave-uniform, so the per-tile cost is scalar; store() writes the chunks
// into a swizzled LDS tile.
template <int D, int NT, int ROWS = 64>
struct TileRegs {
  static constexpr int CHUNKS = ROWS * D / 8;
  static constexpr int PER_T = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "tile must split evenly over the threads");
  u32x4_t r[PER_T];
  __device__ __forceinline__ void load(const uint16_t* base, int rs, int r0, int n, int tid) {
    const int rows = min(max(n - r0, 0), ROWS);
    const rsrc_t rsrc = make_rsrc(base + (size_t)r0 * rs, (uint32_t)rows * (uint32_t)rs * 2u);
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const int c = tid + k * NT;
      r[k] = buf_ld16(rsrc, (uint32_t)((c / (D / 8)) * rs + (c % (D / 8)) * 8) * 2u);
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, int tid) const {
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const int c = tid + k * NT;
      st16(&s[tile_idx<D>(c / (D / 8), (c % (D / 8)) * 8)], r[k]);
    }
  }
};

}  // namespace mala

namespace mala {

// Wait until at most n vector-memory operations of this wave are
// outstanding (s_waitcnt vmcnt(n); the other counters are left free).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Direct global -> LDS copies (global_load_lds): lane l's bytes land at
// the wave-uniform LDS address lds + size l. They are issued through inline
// assembly: the compiler, seeing a builtin copy in flight, would take every
// later LDS read as possibly reading its destination and wait for the copy
// before it, which turns a copy meant to overlap the current tile's work
// into a stall. Callers wait for their own copies (wait_vmcnt) before the
// barrier that publishes them; the compiler's waits for ordinary loads count
// only those loads, which at worst makes them wait longer. The "memory"
// clobber keeps ordinary loads and stores on their side of a copy, so a
// count of the loads issued after it (wait_vmcnt) stays valid.
__device__ __forceinline__ uint32_t lds_address(const void* lds) {
  typedef __attribute__((address_space(3))) const void lvoid;
  return (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lvoid*)lds);
}
// The compiler inserts no wait states around inline assembly, so each block
// carries its own: s_nop 4 after the M0 write gives the five a vector-memory
// read of an SGPR needs after a vector instruction wrote it (v_readfirstlane
// of the base or of the LDS address), which also covers the M0 write.
// 16 bytes per lane from a per-lane global address
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
               : "memory", "m0");
}
// 16 bytes per lane from a wave-uniform base plus a per-lane byte offset
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, uint32_t lds) {
  const uint64_t p = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);  // readfirstlane yields int: widen unsigned
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint64_t b = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(b), "s"(lds)
               : "memory", "m0");
}

// The same copies through the compiler's builtin, which then orders every
// later LDS read after them by itself. The latent backward and the 128-key
// forward walk keep this form, which measured as fast or faster there (the
// latent key-major kernel spills, and the waits of its scratch reloads,
// counting only the loads the compiler knows, would also drain copies it
// does not).
__device__ __forceinline__ void lds_dma16_ordered(const void* src, void* lds) {
  typedef __attribute__((address_space(1))) void gvoid;
  typedef __attribute__((address_space(3))) void lvoid;
  __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4_ordered(const void* src, void* lds) {
  typedef __attribute__((address_space(1))) void gvoid;
  typedef __attribute__((address_space(3))) void lvoid;
  __builtin_amdgcn_global_load_lds((gvoid*)src, (lvoid*)lds, 4, 0, 0);
}

// Direct global -> LDS copy of a ROWS x D bf16 tile into the swizzled
// row-major layout of tile_idx: one wave instruction moves 1 KB (64 lanes x
// 16 bytes) into consecutive LDS slots, so lane p fills physical slot p of
// its block and fetches the logical 16-byte unit that the swizzle places
// there. Rows at or beyond n are clamped to row n - 1 (finite data the
// callers never use). Instructions are spread over the NW waves. ORDERED
// selects the builtin form of the copy (lds_dma16_ordered).
template <int D, int ROWS, int NW, bool ORDERED = false>
__device__ __forceinline__ void tile_to_lds(uint16_t* s, const uint16_t* base, size_t rs, int r0, int n,
                                            int wave, int lane) {
  constexpr int UNITS = D / 8;              // 16-byte units per row
  constexpr int ROWS_PER = 64 / UNITS;      // rows per 1 KB instruction
  constexpr int INSTR = ROWS * UNITS / 64;  // instructions per tile
  const int pr = lane / UNITS, pu = lane % UNITS;
#pragma unroll
  for (int k = 0; k < (INSTR + NW - 1) / NW; ++k) {
    const int ins = wave + k * NW;
    if (INSTR % NW == 0 || ins < INSTR) {
      const int row = ins * ROWS_PER + pr;
      const int lu = pu ^ tile_swz<D>(row);
      const int grow = min(r0 + row, n - 1);
      if (ORDERED)
        lds_dma16_ordered(base + (size_t)grow * rs + lu * 8, s + ins * 512);
      else
        lds_dma16(base + (size_t)grow * rs + lu * 8, lds_address(s + ins * 512));
    }
  }
}

}  // namespace mala

namespace mala {

// The same copy with the per-lane part of the addresses computed once: each
// of this wave's copy instructions fetches a fixed byte offset from the first
// row of the tile, which is wave-uniform, so a full tile costs one address
// add per copy instruction. The offsets are 32-bit: a tile spans at most 128
// rows of at most 2^24 elements (the entry points reject longer rows). A
// tile that runs past row n - 1 takes the clamped path of tile_to_lds.
// `wave` must be wave-uniform (readfirstlane).
template <int D, int ROWS, int NW, bool ORDERED = false>
struct TileCopy {
  static constexpr int UNITS = D / 8;
  static constexpr int ROWS_PER = 64 / UNITS;
  static constexpr int INSTR = ROWS * UNITS / 64;
  static constexpr int CI = (INSTR + NW - 1) / NW;  // copy instructions per wave
  uint32_t off[CI];
  __device__ __forceinline__ void init(size_t rs, int wave, int lane) {
    const int pr = lane / UNITS, pu = lane % UNITS;
#pragma unroll
    for (int k = 0; k < CI; ++k) {
      const int row = (wave + k * NW) * ROWS_PER + pr;
      off[k] = (uint32_t)(((size_t)row * rs + (pu ^ tile_swz<D>(row)) * 8) * 2);
    }
  }
  __device__ __forceinline__ void copy(uint16_t* s, const uint16_t* base, size_t rs, int r0, int n, int wave,
                                       int lane) const {
    if (r0 + ROWS > n) {
      tile_to_lds<D, ROWS, NW, ORDERED>(s, base, rs, r0, n, wave, lane);
      return;
    }
    const char* tb = reinterpret_cast<const char*>(base + (size_t)r0 * rs);
#pragma unroll
    for (int k = 0; k < CI; ++k) {
      const int ins = wave + k * NW;
      if (INSTR % NW == 0 || ins < INSTR) {
        if (ORDERED)
          lds_dma16_ordered(tb + off[k], s + ins * 512);
        else
          lds_dma16(tb, off[k], lds_address(s + ins * 512));
      }
    }
  }
};

// Workgroup barrier that orders LDS work only: waits for this wave's LDS
// operations, then s_barrier. Unlike __syncthreads() it does not drain
// vector-memory operations, so a direct HBM -> LDS copy may stay in flight
// across it; callers wait for such copies (wait_vmcnt) before reading them.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wave issue priority around a run of MFMAs: while a wave feeds the matrix
// core it wins instruction arbitration over the other wave on its SIMD, whose
// vector-ALU work (softmax, masks, packing) then fills the gaps between the
// MFMAs instead of delaying them.
__device__ __forceinline__ void mfma_run_begin() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void mfma_run_end() { __builtin_amdgcn_s_setprio(0); }

// Scheduling hint for an unrolled run of NMFMA MFMAs that each take READS
// LDS reads: issue the reads of the next MFMA before the current one, so
// an MFMA waits for its own operands only.
template <int NMFMA, int READS>
__device__ __forceinline__ void interleave_ds_mfma() {
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * READS, 0);
#pragma unroll
  for (int i = 0; i < NMFMA - 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

}  // namespace mala
